"""GPU parity for the short causal convolution in front of the gated DELTA
rule (What Is Linear Attention? 5.4 with 5.2-5.3): chunked prefill (the
convolution pass, then the rule on the convolved copies) and decode step
against the fp64 oracle, through the C ABI, on seeded inputs of the delta
workload's recipe (q, k unit rows, v normal, g = sigmoid(normal)).  Filters
are the unit tap on the current token plus seeded noise, so the convolved
keys stay near unit length and the rule contracts.  The conv cache holds
raw input values and is compared exactly."""
import numpy as np
import pytest
import torch

import causal_linear_attention_attn_amd as la
from causal_linear_attention_attn_amd import inputs
import oracle
from parity import TOL, assert_close, assert_terms_close, cpu, delta_output_scale

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _draw(B, H, N, d, dv, dtype, seed):
    wid = 800 + seed  # private generator streams, the delta workload's recipe
    q = inputs.unit_rows((B, H, N, d), wid, 1, "cpu", dtype).to(DEV)
    k = inputs.unit_rows((B, H, N, d), wid, 2, "cpu", dtype).to(DEV)
    v = inputs.normal((B, H, N, dv), wid, 3, "cpu", 1.0, dtype).to(DEV)
    g = inputs.sigmoid_gate((B, H, N), wid, 4, "cpu").to(DEV)
    return q, k, v, g


def _filters(H, w, d, dv, seed, noise=0.25):
    W = inputs.normal((H, w, 2 * d + dv), 800 + seed, 5, "cpu", noise / np.sqrt(w))
    W[:, w - 1] += 1.0
    return W.to(DEV)


def _cache(B, H, w, d, dv, dtype, seed):
    x = inputs.normal((B, H, w - 1, 2 * d + dv), 800 + seed, 6, "cpu", 1.0, dtype)
    x[..., :2 * d] *= d ** -0.5  # q and k channels at the scale of unit rows
    return x.to(DEV)


def _same(got, want, what):
    np.testing.assert_array_equal(cpu(got).double().numpy(), want, err_msg=what)


SHAPES = [  # (B, H, N, d, dv, w)
    (1, 1, 1, 128, 128, 4), (1, 2, 2, 64, 64, 4), (2, 1, 63, 64, 64, 4),
    (1, 2, 65, 64, 64, 3), (1, 1, 64, 128, 128, 2), (2, 2, 200, 128, 128, 4),
    (1, 3, 130, 64, 128, 4), (1, 2, 97, 128, 64, 1), (1, 1, 17, 4, 3, 4),
    (2, 1, 50, 100, 72, 3),
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("with_cache", [False, True], ids=["zeros", "cache"])
def test_delta_conv_prefill_small(shape, dtype, with_cache):
    B, H, N, d, dv, w = shape
    seed = (B * 7 + H * 11 + N * 13 + d * 17 + dv * 19 + w * 23) % 97 \
        + 3 * (dtype == torch.bfloat16) + 5 * with_cache
    q, k, v, g = _draw(B, H, N, d, dv, dtype, seed)
    W = _filters(H, w, d, dv, seed)
    C = _cache(B, H, w, d, dv, dtype, seed) if with_cache and w > 1 else None
    C0 = None if C is None else C.clone()
    o, S, _ = la.prefill(q, k, v, rule="delta", g=g, conv_weight=W, conv_cache=C)
    torch.cuda.synchronize()
    ro, rS, rC = oracle.delta_prefill_conv(cpu(q), cpu(k), cpu(v), cpu(g), cpu(W),
                                           conv_cache=None if C0 is None else cpu(C0))
    tol = TOL[dtype]
    # a row of o_t = S_t^T q_t can cancel (more so on convolved keys): judged
    # against the sum of its terms' magnitudes, on the convolved inputs
    cw, cc = cpu(W).double().numpy(), None if C0 is None else cpu(C0).double().numpy()
    ys = [oracle.short_conv(cpu(x), cw[..., sl], None if cc is None else cc[..., sl])[0]
          for x, sl in ((q, slice(0, d)), (k, slice(d, 2 * d)), (v, slice(2 * d, None)))]
    assert_terms_close(o, ro, delta_output_scale(*ys, cpu(g)), tol, "o")
    assert_close(S, rS, tol, "S", axes=(-2, -1))
    if C is not None:
        _same(C, rC, "conv cache")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_delta_conv_prefill_decay_state_and_separate_cache(dtype):
    """With the scalar decay alpha, an initial state updated in place, and
    the conv cache written to a separate buffer (the input cache kept)."""
    B, H, N, d, dv, w = 2, 3, 150, 64, 64, 4
    q, k, v, g = _draw(B, H, N, d, dv, dtype, 60)
    al = inputs.decay_gate((B, H, N), 860, 6, "cpu", 0.5).to(DEV)
    W = _filters(H, w, d, dv, 61)
    C = _cache(B, H, w, d, dv, dtype, 62)
    C0 = C.clone()
    Cout = torch.empty_like(C)
    S = inputs.normal((B, H, d, dv), 863, 5, "cpu", 0.3).to(DEV)
    S0 = S.clone()
    o, _, _ = la.prefill(q, k, v, rule="delta", g=g, alpha=al, conv_weight=W, conv_cache=C,
                         conv_cache_out=Cout, S_in=S, S_out=S)
    torch.cuda.synchronize()
    ro, rS, rC = oracle.delta_prefill_conv(cpu(q), cpu(k), cpu(v), cpu(g), cpu(W),
                                           conv_cache=cpu(C0), S0=cpu(S0), alpha=cpu(al))
    assert_close(o, ro, TOL[dtype], "o")
    assert_close(S, rS, TOL[dtype], "S", axes=(-2, -1))
    _same(Cout, rC, "conv cache out")
    _same(C, cpu(C0).double().numpy(), "conv cache in (unchanged)")


DECODE_CASES = [  # (d, dv, w, dtype)
    *[(d, dv, w, dt) for d, dv, w in ((64, 64, 4), (128, 128, 3), (24, 40, 2), (16, 16, 4))
      for dt in (torch.float32, torch.bfloat16)],
    (4, 3, 4, torch.float32),
]


@pytest.mark.parametrize("case", DECODE_CASES,
                         ids=lambda c: "x".join(map(str, c[:3])) + ("-bf16" if
                                                                    c[3] == torch.bfloat16
                                                                    else "-f32"))
def test_delta_conv_prefill_then_decode(case):
    """A prefill shorter than the conv window, a second one carrying S and
    the conv cache (in place), then decode steps with the cache: every
    output against the oracle's single pass over the whole sequence.  The
    three-entry output rows of d = 4, dv = 3 run in fp32 only: with keys
    rounded to bf16 after the convolution their bf16 row error reached 3.2%
    over 80 tokens, above the 2% bound (the fp32 run checks the same code at
    1e-4)."""
    d, dv, w, dtype = case
    B, H, N = 2, 2, 90
    q, k, v, g = _draw(B, H, N, d, dv, dtype, 70 + d % 7 + w)
    al = inputs.decay_gate((B, H, N), 870, 6, "cpu", 0.7).to(DEV)
    W = _filters(H, w, d, dv, 71)
    ro, rS, rC = oracle.delta_prefill_conv(cpu(q), cpu(k), cpu(v), cpu(g), cpu(W),
                                           alpha=cpu(al))
    C = torch.zeros((B, H, w - 1, 2 * d + dv), dtype=dtype, device=DEV)
    S = torch.zeros((B, H, d, dv), dtype=torch.float32, device=DEV)
    cuts = (0, 1, 80)
    tol = TOL[dtype]
    for a, b in zip(cuts, cuts[1:]):
        o, _, _ = la.prefill(q[:, :, a:b].contiguous(), k[:, :, a:b].contiguous(),
                             v[:, :, a:b].contiguous(), rule="delta",
                             g=g[:, :, a:b].contiguous(), alpha=al[:, :, a:b].contiguous(),
                             conv_weight=W, conv_cache=C, S_in=S, S_out=S)
        torch.cuda.synchronize()
        assert_close(o, ro[:, :, a:b], tol, f"o tokens {a}..{b}")
    for t in range(80, N):
        o = la.decode_step(q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                           v[:, :, t].contiguous(), S, rule="delta",
                           g=g[:, :, t].contiguous(), alpha=al[:, :, t].contiguous(),
                           conv_weight=W, conv_cache=C)
        torch.cuda.synchronize()
        assert_close(o, ro[:, :, t], tol, f"o decode step {t}")
    assert_close(S, rS, tol, "S", axes=(-2, -1))
    _same(C, rC, "conv cache")
