"""GPU parity for training with GLA's per-key-channel decay ("Efficient
attention variants" 7.2; the gradients are the chain rule, the pages give
none): the forward keeping its denominators under the decay, then
la_backward with alpha; dq, dk, dv, the initial-state gradients and dalpha
against the fp64 oracle, every gradient judged against the sum of its
terms' magnitudes (parity.gla_grad_scales: dq, dk and dalpha are sums of
terms of both signs)."""
import numpy as np
import pytest
import torch

import causal_linear_attention_attn_amd as la
from causal_linear_attention_attn_amd import inputs
import oracle
from parity import TOL, assert_close, assert_grad_close, cpu, gla_grad_scales

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(B, H, N, d, dv, dtype, wid, lo):
    sc = d ** -0.5
    q = inputs.normal((B, H, N, d), wid, 1, "cpu", sc, dtype).to(DEV)
    k = inputs.normal((B, H, N, d), wid, 2, "cpu", sc, dtype).to(DEV)
    v = inputs.normal((B, H, N, dv), wid, 3, "cpu", 1.0, dtype).to(DEV)
    do = inputs.normal((B, H, N, dv), wid, 4, "cpu", 1.0, dtype).to(DEV)
    al = inputs.decay_gate((B, H, N, d), wid, 5, "cpu", lo).to(DEV)
    return q, k, v, do, al


def _check(q, k, v, do, al, tol, S0=None, z0=None, dS=None, dz=None, eps=1e-6):
    B, H, N, _ = q.shape
    den = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    o, _, _ = la.prefill(q, k, v, alpha=al, eps=eps, S_in=S0, z_in=z0, den_out=den,
                         return_state=False)
    dq, dk, dv, dS0, dz0, dal = la.backward(q, k, v, o, den, do, alpha=al, S_in=S0, z_in=z0,
                                            dS_out=dS, dz_out=dz)
    torch.cuda.synchronize()
    c = lambda t: None if t is None else cpu(t)  # noqa: E731
    rden = oracle.linear_denominators(cpu(q), cpu(k), alpha=cpu(al), eps=eps, z0=c(z0))
    assert_close(den[..., None], rden[..., None], 1e-5 if q.dtype == torch.float32 else 1e-2,
                 "den")
    r = oracle.linear_backward(cpu(q), cpu(k), cpu(v), cpu(do), alpha=cpu(al), eps=eps,
                               S0=c(S0), z0=c(z0), dS_N=c(dS), dz_N=c(dz))
    ro, _, _ = oracle.linear_prefill(cpu(q), cpu(k), cpu(v), alpha=cpu(al), eps=eps, S0=c(S0),
                                     z0=c(z0))
    sq, sk, sv, sS, sz, sa = gla_grad_scales(cpu(q), cpu(k), cpu(v), cpu(do), ro, rden, cpu(al),
                                             S0=c(S0), z0=c(z0), dS_N=c(dS), dz_N=c(dz))
    assert_grad_close(dq, r[0], sq, tol, "dq")
    assert_grad_close(dk, r[1], sk, tol, "dk")
    assert_grad_close(dv, r[2], sv, tol, "dv")
    assert_grad_close(dS0, r[3], sS, tol, "dS_in")
    assert_grad_close(dz0[..., None], r[4][..., None], sz[..., None], tol, "dz_in")
    assert_grad_close(dal, r[5], sa, tol, "dalpha")


SHAPES = [  # (B, H, N, d, dv)
    (1, 1, 1, 64, 64), (1, 2, 3, 16, 16), (2, 1, 63, 64, 64), (1, 1, 64, 64, 64),
    (1, 2, 65, 64, 64), (2, 2, 200, 128, 128), (1, 3, 130, 64, 128), (1, 2, 97, 128, 64),
    (1, 1, 17, 4, 3), (2, 1, 50, 100, 72), (1, 1, 70, 24, 40), (1, 1, 130, 6, 5),
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gla_backward_small(shape, dtype):
    B, H, N, d, dv = shape
    if dtype == torch.float32 and d > 64:
        pytest.skip("fp32 with a per-channel decay takes d <= 64 (EUNSUPPORTED: LDS)")
    wid = 1900 + (B * 7 + H * 11 + N * 13 + d * 17 + dv * 19) % 89 + 3 * (dtype == torch.bfloat16)
    q, k, v, do, al = _case(B, H, N, d, dv, dtype, wid, 0.9)
    _check(q, k, v, do, al, TOL[dtype])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("lo", [0.9, 0.3, 1e-3], ids=["slow", "fast", "fastest"])
def test_gla_backward_segments_and_state_gradients(dtype, lo):
    """Several segments (per-channel segment decays in the reverse scan), an
    initial state, both final-state gradients, decays down to lo."""
    B, H, N, d, dv = 1, 4, 4099, 64, 64
    wid = 1990 + (dtype == torch.bfloat16) + int(10 * lo)
    q, k, v, do, al = _case(B, H, N, d, dv, dtype, wid, lo)
    S0 = inputs.normal((B, H, d, dv), wid, 6, "cpu", 0.3).to(DEV)
    z0 = inputs.normal((B, H, d), wid, 7, "cpu", 0.3).abs().to(DEV) + 1.0
    dS = inputs.normal((B, H, d, dv), wid, 8, "cpu", 0.01).to(DEV)
    dz = inputs.normal((B, H, d), wid, 9, "cpu", 0.01).to(DEV)
    _check(q, k, v, do, al, TOL[dtype], S0=S0, z0=z0, dS=dS, dz=dz)


def test_gla_backward_reuses_forward_workspace():
    """The forward's segment states read from its workspace give the same
    gradients bit for bit as recomputing them."""
    B, H, N, d, dv = 1, 4, 4099, 64, 64
    q, k, v, do, al = _case(B, H, N, d, dv, torch.bfloat16, 1995, 0.9)
    ws = torch.empty(max(1, la.workspace_size(q, k, v, alpha=al)), dtype=torch.uint8, device=DEV)
    den = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    o, _, _ = la.prefill(q, k, v, alpha=al, den_out=den, workspace=ws, return_state=False)
    ref = la.backward(q, k, v, o, den, do, alpha=al)
    got = la.backward(q, k, v, o, den, do, alpha=al, fwd_workspace=ws)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv", "dS_in", "dz_in", "dalpha"), got, ref):
        assert torch.equal(a, b), name


def test_gla_backward_refusals():
    """fp32 with d > 64 and alpha together with gamma are refused before
    anything runs (the workspace query already fails)."""
    q = torch.zeros((1, 1, 8, 128), dtype=torch.float32, device=DEV)
    al = torch.full((1, 1, 8, 128), 0.9, device=DEV)
    den = torch.ones((1, 1, 8), device=DEV)
    with pytest.raises(ValueError):  # fp32, d > 64
        la.backward(q, q, q, q, den, q, alpha=al)
    g = torch.ones(1, device=DEV)
    q = q[..., :64].contiguous()
    with pytest.raises(ValueError):  # alpha with gamma
        la.backward(q, q, q, q, den, q, alpha=al[..., :64].contiguous(), gamma=g)


def test_gla_workload_training_sampled():
    """B4 H16 N4096 d64 with GLA's decay as a training step runs it (the
    forward keeping denominators, the backward with the forward's
    workspace); two whole heads against the oracle."""
    w = inputs.WORKLOADS[7]
    x = inputs.make_prefill(w, DEV)
    do = inputs.make_grad_out(w, DEV)
    q, k, v, al = x["q"], x["k"], x["v"], x["alpha"]
    B, H, N = w.B, w.H, w.N
    ws = torch.empty(max(1, la.workspace_size(q, k, v, alpha=al)), dtype=torch.uint8, device=DEV)
    den = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    o, _, _ = la.prefill(q, k, v, alpha=al, eps=w.eps, den_out=den, workspace=ws,
                         return_state=False)
    dq, dk, dv, _, _, dal = la.backward(q, k, v, o, den, do, alpha=al, fwd_workspace=ws)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (B - 1, H - 1)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        qs, ks, vs, dos, als = (cpu(t[sl]) for t in (q, k, v, do, al))
        r = oracle.linear_backward(qs, ks, vs, dos, alpha=als, eps=w.eps)
        ro, _, _ = oracle.linear_prefill(qs, ks, vs, alpha=als, eps=w.eps)
        rden = oracle.linear_denominators(qs, ks, alpha=als, eps=w.eps)
        sq, sk, sv, _, _, sa = gla_grad_scales(qs, ks, vs, dos, ro, rden, als)
        tol = TOL[torch.bfloat16]
        assert_grad_close(dq[sl], r[0], sq, tol, f"dq head {b},{h}")
        assert_grad_close(dk[sl], r[1], sk, tol, f"dk head {b},{h}")
        assert_grad_close(dv[sl], r[2], sv, tol, f"dv head {b},{h}")
        assert_grad_close(dal[sl], r[5], sa, tol, f"dalpha head {b},{h}")


@pytest.mark.parametrize("reuse", [True, False], ids=["fwd_ws", "recompute"])
def test_gla_training_through_conv(reuse):
    """GLA's decay behind the short convolution: the training forward (the
    convolution as a pass, then the rule keeping denominators under alpha)
    and la_backward with both, against the oracle's backward through the
    convolution; input, filter, cache, state and decay gradients."""
    B, H, N, d, dv, w = 2, 2, 300, 64, 64, 4
    wid = 1996
    q, k, v, do, al = _case(B, H, N, d, dv, torch.bfloat16, wid, 0.5)
    W = inputs.normal((H, w, 2 * d + dv), wid, 6, "cpu", 0.25 / np.sqrt(w))
    W[:, w - 1] += 1.0
    W = W.to(DEV)
    C0 = inputs.normal((B, H, w - 1, 2 * d + dv), wid, 7, "cpu", 0.1, torch.bfloat16).to(DEV)
    dCo = inputs.normal((B, H, w - 1, 2 * d + dv), wid, 8, "cpu", 1.0, torch.bfloat16).to(DEV)
    C = C0.clone()
    den = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(1, la.workspace_size(q, k, v, alpha=al, conv_weight=W, den_out=den)),
                     dtype=torch.uint8, device=DEV)
    o, _, _ = la.prefill(q, k, v, alpha=al, conv_weight=W, conv_cache=C, den_out=den,
                         workspace=ws, return_state=False)
    dq, dk, dv_, dS, dz, dW, dC, dal = la.backward(
        q, k, v, o, den, do, alpha=al, conv_weight=W, conv_cache=C0, dconv_cache_out=dCo,
        fwd_workspace=ws if reuse else None)
    torch.cuda.synchronize()
    r = oracle.linear_backward_conv(cpu(q), cpu(k), cpu(v), cpu(do), cpu(W), conv_cache=cpu(C0),
                                    dconv_cache_out=cpu(dCo), alpha=cpu(al), eps=1e-6)
    tol = TOL[torch.bfloat16]
    # the convolved inputs' gradients' scales, then the chain rule on magnitudes
    cw, cc = cpu(W).double().numpy(), cpu(C0).double().numpy()
    ys = [oracle.short_conv(cpu(x), cw[..., sl], cc[..., sl])[0]
          for x, sl in ((q, slice(0, d)), (k, slice(d, 2 * d)), (v, slice(2 * d, None)))]
    yo, _, _ = oracle.linear_prefill(*ys, alpha=cpu(al), eps=1e-6)
    yden = oracle.linear_denominators(ys[0], ys[1], alpha=cpu(al), eps=1e-6)
    sq, sk, sv, sS, sz, sa = gla_grad_scales(*ys, cpu(do), yo, yden, cpu(al))
    from test_gpu_conv_backward import _conv_scales
    sx, sW, sC = _conv_scales(q, k, v, W, C0, dCo, (sq, sk, sv))
    for name, got, want, sc in zip(("dq", "dk", "dv"), (dq, dk, dv_), r[:3], sx):
        assert_grad_close(got, want, sc, tol, name)
    assert_grad_close(dW, r[3], sW, tol, "dconv_weight")
    assert_grad_close(dC, r[4], sC, tol, "dconv_cache")
    assert_grad_close(dS, r[5], sS, tol, "dS_in")
    assert_grad_close(dal, r[7], sa, tol, "dalpha")
