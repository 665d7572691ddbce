"""GPU parity for the backward of the gated delta rule (training): dq, dk,
dv, dg, dalpha and the initial-state gradient of la_delta_backward against
the fp64 oracle's token-by-token reverse pass, through the C ABI, on seeded
inputs (unit-norm q and k rows, as the gated delta workload draws them).
Token rows of dq, dk, dv are compared row by row; dg and dalpha (one value
per token) per head over the sequence; dS_in per head; each against the sum
of its terms' magnitudes (parity.delta_grad_scales)."""
import numpy as np
import pytest
import torch

import causal_linear_attention_attn_amd as la
from causal_linear_attention_attn_amd import inputs
import oracle
from parity import TOL, assert_grad_close, cpu, delta_grad_scales

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF16 = TOL[torch.bfloat16]


def _rand(shape, seed, scale=1.0, dtype=torch.float32):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype).to(DEV)


def _unit(shape, seed):
    x = _rand(shape, seed)
    return (x / x.norm(dim=-1, keepdim=True)).to(torch.bfloat16)


def _case(B, H, N, d, dv, seed, decay, lo=0.9, state=False):
    x = {"q": _unit((B, H, N, d), seed), "k": _unit((B, H, N, d), seed + 1),
         "v": _rand((B, H, N, dv), seed + 2, dtype=torch.bfloat16),
         "g": torch.sigmoid(_rand((B, H, N), seed + 3)),
         "do": _rand((B, H, N, dv), seed + 4, dtype=torch.bfloat16)}
    x["alpha"] = lo + (1 - lo) * torch.sigmoid(_rand((B, H, N), seed + 5)) if decay else None
    x["S_in"] = _rand((B, H, d, dv), seed + 6, 0.3) if state else None
    x["dS_out"] = _rand((B, H, d, dv), seed + 7, 0.3) if state else None
    return x


def _check(x, tol=BF16):
    dq, dk, dv, dg, da, dS0 = la.delta_backward(x["q"], x["k"], x["v"], x["g"], x["do"],
                                                alpha=x["alpha"], S_in=x["S_in"],
                                                dS_out=x["dS_out"])
    torch.cuda.synchronize()
    ref = oracle.delta_backward(*(cpu(x[n]) for n in ("q", "k", "v", "g", "do")),
                                alpha=cpu(x["alpha"]), S0=cpu(x["S_in"]), dS_N=cpu(x["dS_out"]))
    rq, rk, rv, rg, ra, rS = ref
    # every gradient is a sum of terms of both signs (a row of dq_t = S_t do_t
    # can cancel): judged against the sum of its terms' magnitudes
    sq, sk, sv, sg, sa, sS = delta_grad_scales(*(cpu(x[n]) for n in ("q", "k", "v", "g", "do")),
                                               alpha=cpu(x["alpha"]), S0=cpu(x["S_in"]),
                                               dS_N=cpu(x["dS_out"]))
    assert_grad_close(dq, rq, sq, tol, "dq")
    assert_grad_close(dk, rk, sk, tol, "dk")
    assert_grad_close(dv, rv, sv, tol, "dv")
    assert_grad_close(dg, rg, sg, tol, "dg (per head over tokens)")
    if x["alpha"] is not None:
        assert_grad_close(da, ra, sa, tol, "dalpha (per head over tokens)")
    else:
        assert da is None
    assert_grad_close(dS0.flatten(-2), rS.reshape(*rS.shape[:-2], -1),
                      sS.reshape(*sS.shape[:-2], -1), tol, "dS_in")


SHAPES = [  # (B, H, N, d, dv)
    (1, 1, 1, 16, 16), (1, 2, 3, 64, 64), (2, 1, 63, 64, 64), (1, 1, 64, 128, 128),
    (1, 2, 65, 64, 64), (2, 2, 200, 128, 128), (1, 3, 130, 64, 128), (1, 2, 97, 128, 64),
    (1, 1, 17, 24, 40), (2, 1, 50, 100, 72), (1, 1, 70, 8, 8),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("decay", [False, True], ids=["nodecay", "decay"])
def test_delta_backward_small(shape, decay):
    B, H, N, d, dv = shape
    seed = 2400 + B * 7 + H * 11 + N * 13 + d * 17 + dv * 19 + 5 * decay
    _check(_case(B, H, N, d, dv, seed, decay))


@pytest.mark.parametrize("decay", [False, True], ids=["nodecay", "decay"])
def test_delta_backward_state_gradients_and_long_sequence(decay):
    """An initial state, a final-state gradient, 1000 tokens (16 chunks, a
    ragged last one), decays down to 0.3."""
    _check(_case(1, 2, 1000, 128, 128, 2500 + decay, decay, lo=0.3, state=True))


def test_delta_backward_gate_zero_and_no_tokens():
    """g = 0: the state never changes, so dk = dv = 0 and dS_in is the sum of
    q_t do_t^T (plus dS_out); N = 0 passes dS_out through."""
    x = _case(1, 2, 77, 64, 64, 2600, False, state=True)
    x["g"] = torch.zeros_like(x["g"])
    _check(x)
    q = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device=DEV)
    g = torch.empty((1, 2, 0), dtype=torch.float32, device=DEV)
    dS = _rand((1, 2, 64, 64), 2601)
    *_, dS0 = la.delta_backward(q, q, q, g, q, dS_out=dS)
    torch.cuda.synchronize()
    assert torch.equal(dS0, dS)


def test_delta_backward_deterministic():
    x = _case(2, 2, 300, 128, 128, 2700, True)
    a = la.delta_backward(x["q"], x["k"], x["v"], x["g"], x["do"], alpha=x["alpha"])
    b = la.delta_backward(x["q"], x["k"], x["v"], x["g"], x["do"], alpha=x["alpha"])
    torch.cuda.synchronize()
    for name, u, w in zip(("dq", "dk", "dv", "dg", "dalpha", "dS_in"), a, b):
        assert torch.equal(u, w), name


@pytest.mark.parametrize("wid", [5, 6])
def test_delta_backward_workload_full_size_sampled(wid):
    """B2 H16 N8192 d128: the gated delta workload (and with its decay) as a
    training step runs it: the prefill, then the backward for a seeded
    dL/do; two whole heads against the oracle."""
    w = inputs.WORKLOADS[wid]
    x = inputs.make_prefill(w, DEV)
    do = inputs.make_grad_out(w, DEV)
    la.prefill(x["q"], x["k"], x["v"], rule="delta", g=x["g"], alpha=x.get("alpha"),
               return_state=False)
    dq, dk, dv, dg, da, _ = la.delta_backward(x["q"], x["k"], x["v"], x["g"], do,
                                              alpha=x.get("alpha"), state_grad=False)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (1, 15)):
        hd = lambda t: None if t is None else cpu(t[b:b + 1, h:h + 1])  # noqa: E731
        args = [hd(x["q"]), hd(x["k"]), hd(x["v"]), hd(x["g"]), hd(do)]
        rq, rk, rv, rg, ra, _ = oracle.delta_backward(*args, alpha=hd(x.get("alpha")))
        sq, sk, sv, sg, sa, _ = delta_grad_scales(*args, alpha=hd(x.get("alpha")))
        assert_grad_close(hd(dq), rq, sq, BF16, f"dq head ({b},{h})")
        assert_grad_close(hd(dk), rk, sk, BF16, f"dk head ({b},{h})")
        assert_grad_close(hd(dv), rv, sv, BF16, f"dv head ({b},{h})")
        assert_grad_close(hd(dg), rg, sg, BF16, f"dg head ({b},{h})")
        if ra is not None:
            assert_grad_close(hd(da), ra, sa, BF16, f"dalpha head ({b},{h})")
