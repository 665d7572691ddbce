"""fp64 CPU oracle (test infrastructure only; see la_oracle.py)."""
from .la_oracle import (  # noqa: F401
    FMAP_ELU1,
    FMAP_IDENTITY,
    delta_decode_step,
    delta_prefill,
    delta_step,
    feature_map,
    linear_decode_step,
    linear_backward,
    linear_decode_step_conv,
    linear_denominators,
    linear_prefill,
    linear_prefill_conv,
    linear_quadratic,
    linear_step,
    phi_elu1,
    short_conv,
)
