"""GPU parity for training through the short causal convolution (What Is
Linear Attention? 5.4; the gradients are the chain rule, the pages give
none): the LINEAR training forward (the convolution as a pass of its own,
then the prefill keeping denominators) and la_backward with the forward's
convolution, with and without the forward's workspace, and la_delta_backward
with one; dq, dk, dv with respect to the raw inputs, the filter gradient,
the conv-cache gradient (including dL/d(the returned cache)) and the state
gradients against the oracle's backward: the LINEAR rule's input, filter and
cache gradients against the sum of their terms' magnitudes (dq and dk are
small differences of large terms), everything else on the plain row
metric."""
import numpy as np
import pytest
import torch

import causal_linear_attention_attn_amd as la
from causal_linear_attention_attn_amd import inputs
import oracle
from parity import TOL, assert_close, assert_grad_close, cpu, f64, linear_grad_scales

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _filters(H, w, d, dv, wid):
    W = inputs.normal((H, w, 2 * d + dv), wid, 5, "cpu", 0.25 / np.sqrt(w))
    W[:, w - 1] += 1.0
    return W.to(DEV)


def _cache(B, H, w, d, dv, dtype, wid):
    x = inputs.normal((B, H, w - 1, 2 * d + dv), wid, 6, "cpu", 1.0, dtype)
    x[..., :2 * d] *= d ** -0.5
    return x.to(DEV)


LINEAR = [  # (B, H, N, d, dv, w)
    (1, 2, 100, 64, 64, 4), (2, 2, 300, 64, 64, 3), (1, 1, 17, 4, 3, 2),
    (2, 1, 2, 64, 64, 4), (1, 2, 5000, 64, 64, 4), (1, 3, 70, 128, 128, 4),
    (2, 1, 90, 24, 40, 1),
]


def _close(got, ref, tol, what, axes=(-1,)):
    assert_close(got, ref, tol, what, axes=axes)


def _conv_scales(q, k, v, W, C0, dCo, s_y):
    """Per-element sums of |terms| of the raw-input, filter and cache
    gradients: the convolution's chain rule taken on absolute values, from
    the |terms| scales s_y of dL/d(convolved q, k, v)."""
    d = q.shape[-1]
    a = lambda t: None if t is None else np.abs(f64(t))  # noqa: E731
    Wa, Ca, Ga = a(W), a(C0), a(dCo)
    out = []
    for x, lo, hi, sy in ((q, 0, d, s_y[0]), (k, d, 2 * d, s_y[1]), (v, 2 * d, None, s_y[2])):
        sl = slice(lo, hi)
        out.append(oracle.short_conv_backward(a(x), Wa[..., sl], sy,
                                              None if Ca is None else Ca[..., sl],
                                              None if Ga is None else Ga[..., sl]))
    return ([o[0] for o in out], np.concatenate([o[1] for o in out], -1),
            np.concatenate([o[2] for o in out], -1))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("shape", LINEAR, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("reuse", [True, False], ids=["fwd_ws", "recompute"])
def test_linear_training_through_conv(shape, dtype, reuse):
    B, H, N, d, dv, w = shape
    wid = 1300 + (B * 7 + H * 11 + N * 13 + d * 17 + dv * 19 + w * 23) % 89 \
        + 3 * (dtype == torch.bfloat16)
    sc = d ** -0.5
    q = inputs.normal((B, H, N, d), wid, 1, "cpu", sc, dtype).to(DEV)
    k = inputs.normal((B, H, N, d), wid, 2, "cpu", sc, dtype).to(DEV)
    v = inputs.normal((B, H, N, dv), wid, 3, "cpu", 1.0, dtype).to(DEV)
    do = inputs.normal((B, H, N, dv), wid, 4, "cpu", 1.0, dtype).to(DEV)
    gamma = inputs.per_head_gamma(H, DEV)
    W = _filters(H, w, d, dv, wid)
    C0 = _cache(B, H, w, d, dv, dtype, wid) if w > 1 else None
    dCo = inputs.normal((B, H, w - 1, 2 * d + dv), wid, 7, "cpu", 1.0, dtype).to(DEV) \
        if w > 1 else None
    C = None if C0 is None else C0.clone()
    den = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(1, la.workspace_size(q, k, v, gamma=gamma, conv_weight=W, den_out=den)),
                     dtype=torch.uint8, device=DEV)
    o, _, _ = la.prefill(q, k, v, gamma=gamma, eps=1e-6, conv_weight=W, conv_cache=C,
                         den_out=den, workspace=ws, return_state=False)
    dq, dk, dv_, dS, dz, dW, dC = la.backward(
        q, k, v, o, den, do, gamma=gamma, conv_weight=W, conv_cache=C0, dconv_cache_out=dCo,
        fwd_workspace=ws if reuse else None)
    torch.cuda.synchronize()
    r = oracle.linear_backward_conv(cpu(q), cpu(k), cpu(v), cpu(do), cpu(W),
                                    conv_cache=None if C0 is None else cpu(C0),
                                    dconv_cache_out=None if dCo is None else cpu(dCo),
                                    gamma=cpu(gamma), eps=1e-6)
    ro, _, _, rC = oracle.linear_prefill_conv(cpu(q), cpu(k), cpu(v), cpu(W),
                                              conv_cache=None if C0 is None else cpu(C0),
                                              gamma=cpu(gamma), eps=1e-6)
    tol = TOL[dtype]
    assert_close(o, ro, tol, "o")
    if C is not None:
        np.testing.assert_array_equal(cpu(C).double().numpy(), rC, err_msg="conv cache out")
    # dq, dk (and through the convolution every gradient) are sums of terms
    # that can cancel: judged against the sum of the terms' magnitudes
    cw = cpu(W).double().numpy()
    cc = None if C0 is None else cpu(C0).double().numpy()
    ys = [oracle.short_conv(cpu(x), cw[..., sl],
                            None if cc is None else cc[..., sl])[0]
          for x, sl in ((q, slice(0, d)), (k, slice(d, 2 * d)), (v, slice(2 * d, None)))]
    yo, _, _ = oracle.linear_prefill(*ys, gamma=cpu(gamma), eps=1e-6)
    yden = oracle.linear_denominators(ys[0], ys[1], gamma=cpu(gamma), eps=1e-6)
    s_y = linear_grad_scales(*ys, cpu(do), yo, yden, gamma=cpu(gamma))
    sx, sW, sC = _conv_scales(q, k, v, W, C0, dCo, s_y[:3])
    for name, got, want, sc in zip(("dq", "dk", "dv"), (dq, dk, dv_), r[:3], sx):
        assert_grad_close(got, want, sc, tol, name)
    assert_grad_close(dW, r[3], sW, tol, "dconv_weight")
    if w > 1:
        assert_grad_close(dC, r[4], sC, tol, "dconv_cache")
    assert_grad_close(dS, r[5], s_y[3], tol, "dS_in")
    assert_grad_close(dz, r[6], s_y[4], tol, "dz_in")


DELTA = [  # (B, H, N, d, dv, w)
    (1, 2, 100, 64, 64, 4), (2, 2, 200, 128, 128, 3), (1, 1, 17, 16, 16, 2),
    (2, 1, 3, 64, 64, 4), (1, 2, 1000, 128, 128, 4),
]


@pytest.mark.parametrize("shape", DELTA, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("decay", [False, True], ids=["plain", "decay"])
def test_delta_training_through_conv(shape, decay):
    B, H, N, d, dv, w = shape
    wid = 1400 + (B * 7 + H * 11 + N * 13 + d * 17 + dv * 19 + w * 23) % 89 + 5 * decay
    q = inputs.unit_rows((B, H, N, d), wid, 1, "cpu", torch.bfloat16).to(DEV)
    k = inputs.unit_rows((B, H, N, d), wid, 2, "cpu", torch.bfloat16).to(DEV)
    v = inputs.normal((B, H, N, dv), wid, 3, "cpu", 1.0, torch.bfloat16).to(DEV)
    g = inputs.sigmoid_gate((B, H, N), wid, 4, "cpu").to(DEV)
    al = inputs.decay_gate((B, H, N), wid, 8, "cpu", 0.6).to(DEV) if decay else None
    do = inputs.normal((B, H, N, dv), wid, 9, "cpu", 1.0, torch.bfloat16).to(DEV)
    W = _filters(H, w, d, dv, wid)
    C0 = _cache(B, H, w, d, dv, torch.bfloat16, wid)
    dCo = inputs.normal((B, H, w - 1, 2 * d + dv), wid, 7, "cpu", 1.0, torch.bfloat16).to(DEV)
    S0 = inputs.normal((B, H, d, dv), wid, 10, "cpu", 0.3).to(DEV)
    out = la.delta_backward(q, k, v, g, do, alpha=al, S_in=S0, conv_weight=W, conv_cache=C0,
                            dconv_cache_out=dCo)
    torch.cuda.synchronize()
    dq, dk, dv_, dg, da, dS, dW, dC = out
    r = oracle.delta_backward_conv(cpu(q), cpu(k), cpu(v), cpu(g), cpu(do), cpu(W),
                                   conv_cache=cpu(C0), dconv_cache_out=cpu(dCo),
                                   alpha=None if al is None else cpu(al), S0=cpu(S0))
    tol = TOL[torch.bfloat16]
    for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv_), r[:3]):
        _close(got, want, tol, name)
    _close(dg, r[3], tol, "dg", axes=(-2, -1))
    if decay:
        _close(da, r[4], tol, "dalpha", axes=(-2, -1))
    _close(dW, r[5], tol, "dconv_weight")
    _close(dC, r[6], tol, "dconv_cache")
    _close(dS, r[7], tol, "dS_in", axes=(-2, -1))
