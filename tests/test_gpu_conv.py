"""GPU parity for the short causal convolution in front of the LINEAR rule
(What Is Linear Attention? 5.4): chunked prefill and decode step against the
fp64 oracle through the C ABI, on seeded inputs.  The conv cache holds raw
input values, so it is compared exactly."""
import numpy as np
import pytest
import torch

import causal_linear_attention_attn_amd as la
from causal_linear_attention_attn_amd import inputs
import oracle
from parity import TOL, assert_close, assert_terms_close, cpu, linear_output_scale

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _rand(shape, dtype, seed, scale=1.0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype).to(DEV)


def _filters(H, w, d, dv, seed):
    return _rand((H, w, 2 * d + dv), torch.float32, seed, w ** -0.5)


def _oracle(q, k, v, W, cache=None, **kw):
    return oracle.linear_prefill_conv(cpu(q), cpu(k), cpu(v), cpu(W),
                                      conv_cache=None if cache is None else cpu(cache), **kw)


def _same(got, want, what):
    np.testing.assert_array_equal(cpu(got).double().numpy(), want, err_msg=what)


SHAPES = [  # (B, H, N, d, dv, w)
    (1, 1, 1, 64, 64, 4), (1, 2, 2, 64, 64, 4), (2, 1, 63, 64, 64, 4),
    (1, 2, 65, 64, 64, 3), (1, 1, 64, 64, 64, 2), (2, 2, 200, 128, 128, 4),
    (1, 3, 130, 64, 128, 4), (1, 2, 97, 128, 64, 1), (1, 1, 17, 4, 3, 4),
    (2, 1, 50, 100, 72, 3),
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("with_cache", [False, True], ids=["zeros", "cache"])
def test_conv_prefill_small(shape, dtype, with_cache):
    B, H, N, d, dv, w = shape
    seed = 1100 + B * 7 + H * 11 + N * 13 + d * 17 + dv * 19 + w * 23 \
        + 3 * (dtype == torch.bfloat16) + 5 * with_cache
    sc = 1 / np.sqrt(d)
    q = _rand((B, H, N, d), dtype, seed, sc)
    k = _rand((B, H, N, d), dtype, seed + 1, sc)
    v = _rand((B, H, N, dv), dtype, seed + 2)
    W = _filters(H, w, d, dv, seed + 3)
    C = _rand((B, H, w - 1, 2 * d + dv), dtype, seed + 4, sc) if with_cache else None
    C0 = None if C is None else C.clone()
    o, S, z = la.prefill(q, k, v, eps=1e-6, conv_weight=W, conv_cache=C)
    torch.cuda.synchronize()
    ro, rS, rz, rC = _oracle(q, k, v, W, C0, eps=1e-6)
    tol = TOL[dtype]
    if dv < 16:  # rows of 2 or 3 values: judged against their terms' magnitudes
        cw, cc = cpu(W).double().numpy(), None if C0 is None else cpu(C0).double().numpy()
        ys = [oracle.short_conv(cpu(x), cw[..., sl], None if cc is None else cc[..., sl])[0]
              for x, sl in ((q, slice(0, d)), (k, slice(d, 2 * d)), (v, slice(2 * d, None)))]
        assert_terms_close(o, ro, linear_output_scale(*ys), tol, "o")
    else:
        assert_close(o, ro, tol, "o")
    assert_close(S, rS, tol, "S", axes=(-2, -1))
    assert_close(z, rz, tol, "z")
    if C is not None:
        _same(C, rC, "conv cache")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("decay", ["gamma", "channel"])
def test_conv_prefill_segments_in_place(dtype, decay):
    """Several segments (summary, scan and chunk kernels; the chunk kernel
    reads the summary kernel's copy of the cache), S, z and the conv cache
    updated in place, with a per-head or a per-key-channel decay."""
    B, H, N, d, dv, w = 1, 4, 4099, 64, 64, 4
    seed = 1200 + (dtype == torch.bfloat16) + 2 * (decay == "channel")
    q = _rand((B, H, N, d), dtype, seed, 0.125)
    k = _rand((B, H, N, d), dtype, seed + 1, 0.125)
    v = _rand((B, H, N, dv), dtype, seed + 2)
    W = _filters(H, w, d, dv, seed + 3)
    C = _rand((B, H, w - 1, 2 * d + dv), dtype, seed + 4, 0.125)
    S = _rand((B, H, d, dv), torch.float32, seed + 5, 0.3)
    z = _rand((B, H, d), torch.float32, seed + 6, 0.3).abs() + 1.0
    kw = {}
    if decay == "gamma":
        kw["gamma"] = inputs.per_head_gamma(H, DEV)
    else:
        kw["alpha"] = inputs.decay_gate((B, H, N, d), 7, 0, DEV, 0.5)
    C0, S0, z0 = C.clone(), S.clone(), z.clone()
    o, _, _ = la.prefill(q, k, v, eps=1e-6, S_in=S, z_in=z, S_out=S, z_out=z,
                         conv_weight=W, conv_cache=C, **kw)
    torch.cuda.synchronize()
    ro, rS, rz, rC = _oracle(q, k, v, W, C0, eps=1e-6, S0=cpu(S0), z0=cpu(z0),
                             **{k_: cpu(x) for k_, x in kw.items()})
    tol = TOL[dtype]
    assert_close(o, ro, tol, "o")
    assert_close(S, rS, tol, "S", axes=(-2, -1))
    assert_close(z, rz, tol, "z")
    _same(C, rC, "conv cache")


def test_conv_prefill_no_tokens_keeps_cache():
    B, H, d, dv, w = 2, 3, 64, 64, 4
    q = torch.empty((B, H, 0, d), dtype=torch.bfloat16, device=DEV)
    v = torch.empty((B, H, 0, dv), dtype=torch.bfloat16, device=DEV)
    W = _filters(H, w, d, dv, 1300)
    C = _rand((B, H, w - 1, 2 * d + dv), torch.bfloat16, 1301)
    C0 = C.clone()
    la.prefill(q, q, v, conv_weight=W, conv_cache=C)
    torch.cuda.synchronize()
    assert torch.equal(C, C0)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("dims", [(128, 128, 4), (64, 64, 2), (4, 3, 3), (100, 72, 1)],
                         ids=lambda s: "x".join(map(str, s)))
def test_conv_decode_steps(dims, dtype):
    d, dv, w = dims
    B, H, steps = 3, 5, 6
    W = _filters(H, w, d, dv, 1400 + d)
    S = _rand((B, H, d, dv), torch.float32, 1401, 0.3)
    z = _rand((B, H, d), torch.float32, 1402, 0.3).abs() + 1.0
    C = _rand((B, H, w - 1, 2 * d + dv), dtype, 1403, d ** -0.5)
    rS, rz, rC = cpu(S).double().numpy(), cpu(z).double().numpy(), cpu(C).double().numpy()
    gamma = inputs.per_head_gamma(H, DEV)
    for t in range(steps):
        q = _rand((B, H, d), dtype, 1410 + 5 * t, d ** -0.5)
        k = _rand((B, H, d), dtype, 1411 + 5 * t, d ** -0.5)
        v = _rand((B, H, dv), dtype, 1412 + 5 * t)
        o = la.decode_step(q, k, v, S, z, gamma=gamma, eps=1e-6, conv_weight=W,
                           conv_cache=C if w > 1 else None)
        torch.cuda.synchronize()
        ro, rS, rz, rC = oracle.linear_decode_step_conv(cpu(q), cpu(k), cpu(v), rS, rz,
                                                        cpu(W), rC, gamma=cpu(gamma),
                                                        eps=1e-6)
        assert_close(o, ro, TOL[dtype], f"o step {t}")
        if w > 1:
            _same(C, rC, f"conv cache step {t}")
    assert_close(S, rS, 1e-5, "S", axes=(-2, -1))
    assert_close(z, rz, 1e-5, "z")


def test_conv_prefill_then_decode_handoff():
    """A prefill leaves S, z and the conv cache; decode steps continue the
    sequence as one longer prefill would."""
    B, H, N, d, dv, w, extra = 2, 2, 257, 64, 64, 4, 3
    q = _rand((B, H, N + extra, d), torch.bfloat16, 1500, 0.125)
    k = _rand((B, H, N + extra, d), torch.bfloat16, 1501, 0.125)
    v = _rand((B, H, N + extra, dv), torch.bfloat16, 1502)
    W = _filters(H, w, d, dv, 1503)
    C = torch.zeros((B, H, w - 1, 2 * d + dv), dtype=torch.bfloat16, device=DEV)
    sl = lambda x: x[:, :, :N].contiguous()  # noqa: E731
    _, S, z = la.prefill(sl(q), sl(k), sl(v), eps=1e-6, conv_weight=W, conv_cache=C)
    outs = []
    for t in range(N, N + extra):
        at = lambda x: x[:, :, t].contiguous()  # noqa: E731
        outs.append(la.decode_step(at(q), at(k), at(v), S, z, eps=1e-6, conv_weight=W,
                                   conv_cache=C))
    torch.cuda.synchronize()
    ro, _, _, rC = _oracle(q, k, v, W, None, eps=1e-6)
    for i, o in enumerate(outs):
        assert_close(o, ro[:, :, N + i], TOL[torch.bfloat16], f"o decode {i}")
    _same(C, rC, "conv cache")
