"""Comparison helpers for the GPU-vs-oracle parity tests.

Error metric (one reading, stated once): for outputs, the largest over
output rows (one token of one head, length dv) of
    max_c |o_gpu - o_ref| / max_c |o_ref|;
for states, the same over (b, h) blocks of S (d x dv) and z (d).  Rows whose
reference is exactly zero are compared absolutely.  Elementwise relative
error is not used: outputs are weighted averages of zero-mean values and
single elements can sit arbitrarily close to zero.  For the same reason a
row's scale is floored at a quarter of the median row norm of the tensor:
with a very small dv (2 or 3 values per row) a whole row of a weighted
average can cancel to near zero while the bf16 rounding of the weights
stays proportional to the values being averaged.  With dv >= 16 the floor
does not bind in practice.
"""
import numpy as np
import torch

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def f64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def row_rel_err(got, ref, axes=(-1,)):
    """max over rows of ||got - ref||_inf / ||ref||_inf (rows = all axes but
    `axes`)."""
    g, r = f64(got), f64(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    if g.size == 0:
        return 0.0
    if not np.all(np.isfinite(g)):
        return float("inf")
    diff = np.abs(g - r).max(axis=axes)
    scale = np.abs(r).max(axis=axes)
    scale = np.maximum(scale, 0.25 * np.median(scale))
    scale = np.where(scale > 0, scale, 1.0)
    return float((diff / scale).max())


def assert_close(got, ref, tol, what="", axes=(-1,)):
    e = row_rel_err(got, ref, axes)
    print(f"[parity] {what}: {e:.3e} (tol {tol:.0e})", flush=True)
    assert e <= tol, f"{what}: max row-relative error {e:.3e} > {tol:.1e}"
    return e


def cpu(t):
    return None if t is None else t.detach().to("cpu")
