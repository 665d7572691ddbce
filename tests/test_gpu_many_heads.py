"""GPU parity with more than 65 535 sequences (B*H) in one call: grids that
put one row of workgroups per head on y continue on z past the y limit.
Heads on both sides of that fold, and the last one, are checked against the
oracle."""
import numpy as np
import pytest
import torch

import causal_linear_attention_attn_amd as la
import oracle
from parity import TOL, assert_close, assert_grad_close, cpu, linear_grad_scales

pytestmark = pytest.mark.gpu
DEV = "cuda"
B, H = 2, 33000                       # 66 000 heads
SAMPLE = (0, 65534, 65535, B * H - 1)  # flattened (b, h): last of y, first of z, last


def _rand(shape, dtype, seed, scale=1.0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype).to(DEV)


def _heads(t):
    """The sampled heads of a [B, H, ...] tensor as [1, len(SAMPLE), ...] on the CPU."""
    if t is None:
        return None
    flat = t.reshape(B * H, *t.shape[2:])
    return cpu(flat[list(SAMPLE)]).unsqueeze(0)


def _gamma_of(gamma):
    return None if gamma is None else cpu(gamma)[[i % H for i in SAMPLE]]


def test_linear_prefill_many_heads():
    N, d, dv = 70, 16, 8
    q = _rand((B, H, N, d), torch.bfloat16, 2200, 0.25)
    k = _rand((B, H, N, d), torch.bfloat16, 2201, 0.25)
    v = _rand((B, H, N, dv), torch.bfloat16, 2202)
    gamma = (0.5 + 0.5 * torch.rand(H, generator=torch.Generator().manual_seed(2203))).to(DEV)
    o, S, z = la.prefill(q, k, v, gamma=gamma, eps=1e-6)
    torch.cuda.synchronize()
    ro, rS, rz = oracle.linear_prefill(_heads(q), _heads(k), _heads(v), gamma=_gamma_of(gamma),
                                       eps=1e-6)
    assert_close(_heads(o), ro, TOL[torch.bfloat16], "o")
    assert_close(_heads(S), rS, TOL[torch.bfloat16], "S", axes=(-2, -1))
    assert_close(_heads(z), rz, TOL[torch.bfloat16], "z")


def test_delta_prefill_many_heads():
    N, d, dv = 70, 16, 16
    qn = _rand((B, H, N, d), torch.float32, 2210)
    kn = _rand((B, H, N, d), torch.float32, 2211)
    q = (qn / qn.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    k = (kn / kn.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    v = _rand((B, H, N, dv), torch.bfloat16, 2212)
    g = torch.sigmoid(_rand((B, H, N), torch.float32, 2213))
    o, S, _ = la.prefill(q, k, v, rule="delta", g=g)
    torch.cuda.synchronize()
    ro, rS = oracle.delta_prefill(_heads(q), _heads(k), _heads(v), _heads(g))
    assert_close(_heads(o), ro, TOL[torch.bfloat16], "o")
    assert_close(_heads(S), rS, TOL[torch.bfloat16], "S", axes=(-2, -1))


def test_linear_backward_many_heads():
    N, d, dv = 40, 16, 8
    q = _rand((B, H, N, d), torch.bfloat16, 2220, 0.25)
    k = _rand((B, H, N, d), torch.bfloat16, 2221, 0.25)
    v = _rand((B, H, N, dv), torch.bfloat16, 2222)
    do = _rand((B, H, N, dv), torch.bfloat16, 2223)
    den = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    o, _, _ = la.prefill(q, k, v, eps=1e-6, den_out=den, return_state=False)
    dq, dk, dv_, _, _ = la.backward(q, k, v, o, den, do, state_grad=False)
    torch.cuda.synchronize()
    hq, hk, hv, hdo = (_heads(t) for t in (q, k, v, do))
    rq, rk, rv, _, _ = oracle.linear_backward(hq, hk, hv, hdo, eps=1e-6)
    ro, _, _ = oracle.linear_prefill(hq, hk, hv, eps=1e-6)
    rden = oracle.linear_denominators(hq, hk, eps=1e-6)
    assert_close(_heads(den)[..., None], rden[..., None], 1e-2, "den")
    sq, sk, sv, _, _ = linear_grad_scales(hq, hk, hv, hdo, ro, rden)
    tol = TOL[torch.bfloat16]
    assert_grad_close(_heads(dq), rq, sq, tol, "dq")
    assert_grad_close(_heads(dk), rk, sk, tol, "dk")
    assert_grad_close(_heads(dv_), rv, sv, tol, "dv")
