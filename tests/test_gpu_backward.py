"""GPU parity for the backward of the LINEAR rule (training): the forward's
per-token denominators and dq, dk, dv and the initial-state gradients
against the fp64 oracle, through the C ABI, on seeded inputs.  As in
training, the GPU backward consumes the GPU forward's own output and
denominators; the oracle differentiates its own fp64 forward.

Gradients are compared against the magnitude of the terms they sum
(parity.assert_grad_close): with the normaliser, dq and dk are differences
of large terms (the output is a weighted average, so a shift of every score
by the same factor changes nothing), and an element's rounding error scales
with the terms, not with what is left after they cancel.  fp32 results also
meet the plain row-relative metric."""
import numpy as np
import pytest
import torch

import causal_linear_attention_attn_amd as la
from causal_linear_attention_attn_amd import inputs
import oracle
from parity import TOL, assert_close, assert_grad_close, cpu, linear_grad_scales

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _rand(shape, dtype, seed, scale=1.0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype).to(DEV)


def _case(B, H, N, d, dv, dtype, seed, decay, fmap="elu1"):
    sc = 1 / np.sqrt(d)
    if fmap == "elu1":
        q = _rand((B, H, N, d), dtype, seed, sc)
        k = _rand((B, H, N, d), dtype, seed + 1, sc)
    else:  # non-negative features given directly
        q = _rand((B, H, N, d), dtype, seed, sc).abs()
        k = _rand((B, H, N, d), dtype, seed + 1, sc).abs()
    v = _rand((B, H, N, dv), dtype, seed + 2)
    do = _rand((B, H, N, dv), dtype, seed + 3)
    gamma = inputs.per_head_gamma(H, DEV) if decay else None
    return q, k, v, do, gamma


def _check(q, k, v, do, gamma, fmap, tol, S0=None, z0=None, dS=None, dz=None, eps=1e-6):
    B, H, N, _ = q.shape
    den = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    o, _, _ = la.prefill(q, k, v, fmap=fmap, gamma=gamma, eps=eps, S_in=S0, z_in=z0,
                         den_out=den, return_state=False)
    dq, dk, dv, dS0, dz0 = la.backward(q, k, v, o, den, do, fmap=fmap, gamma=gamma,
                                       S_in=S0, z_in=z0, dS_out=dS, dz_out=dz)
    torch.cuda.synchronize()
    rden = oracle.linear_denominators(cpu(q), cpu(k), gamma=cpu(gamma), eps=eps, fmap=fmap,
                                      z0=cpu(z0))
    assert_close(den[..., None], rden[..., None], 1e-5 if q.dtype == torch.float32 else 1e-2,
                 "den")
    rq, rk, rv, rS0, rz0 = oracle.linear_backward(cpu(q), cpu(k), cpu(v), cpu(do),
                                                  gamma=cpu(gamma), eps=eps, fmap=fmap,
                                                  S0=cpu(S0), z0=cpu(z0), dS_N=cpu(dS),
                                                  dz_N=cpu(dz))
    ro, _, _ = oracle.linear_prefill(cpu(q), cpu(k), cpu(v), gamma=cpu(gamma), eps=eps,
                                     fmap=fmap, S0=cpu(S0), z0=cpu(z0))
    sq, sk, sv, sS, sz = linear_grad_scales(cpu(q), cpu(k), cpu(v), cpu(do), ro, rden,
                                            gamma=cpu(gamma), fmap=fmap, S0=cpu(S0),
                                            z0=cpu(z0), dS_N=cpu(dS), dz_N=cpu(dz))
    assert_grad_close(dq, rq, sq, tol, "dq")
    assert_grad_close(dk, rk, sk, tol, "dk")
    assert_grad_close(dv, rv, sv, tol, "dv")
    assert_grad_close(dS0, rS0, sS, tol, "dS_in")
    assert_grad_close(dz0[..., None], rz0[..., None], sz[..., None], tol, "dz_in")
    if q.dtype == torch.float32 and N > 1:
        # fp32 dv and dS_in also meet the plain row-relative metric (dq and dk
        # rows cancel exactly in places: the first token's o_0 = v_0 makes
        # dphi(q_0) a difference of equal terms)
        assert_close(dv, rv, tol, "dv rows")
        assert_close(dS0, rS0, tol, "dS_in", axes=(-2, -1))


SHAPES = [  # (B, H, N, d, dv)
    (1, 1, 1, 64, 64), (1, 2, 3, 16, 16), (2, 1, 63, 64, 64), (1, 1, 64, 64, 64),
    (1, 2, 65, 64, 64), (2, 2, 200, 128, 128), (1, 3, 130, 64, 128), (1, 2, 97, 128, 64),
    (1, 1, 17, 4, 3), (2, 1, 50, 100, 72), (1, 1, 70, 24, 40),
    (1, 1, 130, 6, 5),  # several segments, d not a multiple of 4 (scalar slot moves)
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("decay", [False, True], ids=["nodecay", "decay"])
def test_backward_small(shape, dtype, decay):
    B, H, N, d, dv = shape
    seed = 1600 + B * 7 + H * 11 + N * 13 + d * 17 + dv * 19 + 3 * (dtype == torch.bfloat16) \
        + 5 * decay
    q, k, v, do, gamma = _case(B, H, N, d, dv, dtype, seed, decay)
    _check(q, k, v, do, gamma, "elu1", TOL[dtype])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_backward_segments_and_state_gradients(dtype):
    """Several segments (forward prefix scan, reverse summary and scan), an
    initial state, and a final-state gradient; the initial-state gradient is
    checked too."""
    B, H, N, d, dv = 1, 4, 4099, 64, 64
    seed = 1700 + (dtype == torch.bfloat16)
    q, k, v, do, gamma = _case(B, H, N, d, dv, dtype, seed, True)
    S0 = _rand((B, H, d, dv), torch.float32, seed + 4, 0.3)
    z0 = _rand((B, H, d), torch.float32, seed + 5, 0.3).abs() + 1.0
    dS = _rand((B, H, d, dv), torch.float32, seed + 6, 0.01)
    dz = _rand((B, H, d), torch.float32, seed + 7, 0.01)
    _check(q, k, v, do, gamma, "elu1", TOL[dtype], S0=S0, z0=z0, dS=dS, dz=dz)


def test_backward_identity_map_bf16_128():
    q, k, v, do, _ = _case(1, 2, 300, 128, 128, torch.bfloat16, 1750, False, fmap="identity")
    _check(q, k, v, do, None, "identity", TOL[torch.bfloat16])


@pytest.mark.parametrize("decay", [False, True], ids=["nodecay", "decay"])
def test_backward_reuses_forward_workspace(decay):
    """With the forward's workspace passed in, the backward reads the
    segment-entering states the forward computed instead of recomputing
    them: the same kernels on the same inputs, so the gradients agree bit
    for bit; a workspace below the forward's size is refused."""
    B, H, N, d, dv = 1, 4, 4099, 64, 64
    q, k, v, do, gamma = _case(B, H, N, d, dv, torch.bfloat16, 1770 + decay, decay)
    S0 = _rand((B, H, d, dv), torch.float32, 1772, 0.3)
    z0 = _rand((B, H, d), torch.float32, 1773, 0.3).abs() + 1.0
    need = la.workspace_size(q, k, v, gamma=gamma)
    assert need > 0  # several segments
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    den = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    o, _, _ = la.prefill(q, k, v, gamma=gamma, S_in=S0, z_in=z0, den_out=den, workspace=ws,
                         return_state=False)
    ref = la.backward(q, k, v, o, den, do, gamma=gamma, S_in=S0, z_in=z0)
    got = la.backward(q, k, v, o, den, do, gamma=gamma, S_in=S0, z_in=z0, fwd_workspace=ws)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv", "dS_in", "dz_in"), got, ref):
        assert torch.equal(a, b), name
    with pytest.raises(RuntimeError):  # below the forward's workspace size
        la.backward(q, k, v, o, den, do, gamma=gamma, S_in=S0, z_in=z0, fwd_workspace=ws[:-4])
    big = torch.empty(need + 8, dtype=torch.uint8, device=DEV)
    with pytest.raises(RuntimeError):  # not 4-byte aligned
        la.backward(q, k, v, o, den, do, gamma=gamma, S_in=S0, z_in=z0,
                    fwd_workspace=big[1:1 + need])


def test_backward_no_tokens_passes_state_gradient():
    B, H, d, dv = 2, 3, 64, 64
    q = torch.empty((B, H, 0, d), dtype=torch.bfloat16, device=DEV)
    v = torch.empty((B, H, 0, dv), dtype=torch.bfloat16, device=DEV)
    den = torch.empty((B, H, 0), dtype=torch.float32, device=DEV)
    dS = _rand((B, H, d, dv), torch.float32, 1760)
    dz = _rand((B, H, d), torch.float32, 1761)
    _, _, _, dS0, dz0 = la.backward(q, q, v, v, den, v, dS_out=dS, dz_out=dz)
    torch.cuda.synchronize()
    assert torch.equal(dS0, dS) and torch.equal(dz0, dz)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_backward_fast_decay(dtype):
    """Per-head decays 0.05, 0.25, 0.45 over several segments, with an
    initial state and a final-state gradient."""
    B, H, N, d, dv = 1, 3, 2000 + 5, 64, 64
    seed = 1790 + (dtype == torch.bfloat16)
    q, k, v, do, _ = _case(B, H, N, d, dv, dtype, seed, False)
    gamma = torch.tensor([0.05, 0.25, 0.45], device=DEV)
    S0 = _rand((B, H, d, dv), torch.float32, seed + 4, 0.3)
    z0 = _rand((B, H, d), torch.float32, seed + 5, 0.3).abs() + 1.0
    dS = _rand((B, H, d, dv), torch.float32, seed + 6, 0.01)
    dz = _rand((B, H, d), torch.float32, seed + 7, 0.01)
    _check(q, k, v, do, gamma, "elu1", TOL[dtype], S0=S0, z0=z0, dS=dS, dz=dz)


@pytest.mark.parametrize("shape", [(1, 2, 3000, 128, 128), (1, 1, 2500, 96, 72)],
                         ids=lambda s: "x".join(map(str, s)))
def test_backward_fp32_wide_value_halves(shape):
    """fp32 with d and dv both above 64 runs over the value columns [0, 64)
    and [64, dv): several segments per half, a per-head decay, an initial
    state and both final-state gradients (the normaliser's only in the
    first half), against the oracle; with the forward's workspace given the
    gradients are the same bit for bit (the halves recompute their own
    segment states)."""
    B, H, N, d, dv = shape
    seed = 1800 + d + dv
    q, k, v, do, gamma = _case(B, H, N, d, dv, torch.float32, seed, True)
    S0 = _rand((B, H, d, dv), torch.float32, seed + 4, 0.3)
    z0 = _rand((B, H, d), torch.float32, seed + 5, 0.3).abs() + 1.0
    dS = _rand((B, H, d, dv), torch.float32, seed + 6, 0.01)
    dz = _rand((B, H, d), torch.float32, seed + 7, 0.01)
    _check(q, k, v, do, gamma, "elu1", TOL[torch.float32], S0=S0, z0=z0, dS=dS, dz=dz)
    ws = torch.empty(max(1, la.workspace_size(q, k, v, gamma=gamma)), dtype=torch.uint8,
                     device=DEV)
    den = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    o, _, _ = la.prefill(q, k, v, gamma=gamma, S_in=S0, z_in=z0, den_out=den, workspace=ws,
                         return_state=False)
    ref = la.backward(q, k, v, o, den, do, gamma=gamma, S_in=S0, z_in=z0, dS_out=dS, dz_out=dz)
    got = la.backward(q, k, v, o, den, do, gamma=gamma, S_in=S0, z_in=z0, dS_out=dS, dz_out=dz,
                      fwd_workspace=ws)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv", "dS_in", "dz_in"), got, ref):
        assert torch.equal(a, b), name
