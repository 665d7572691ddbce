"""GPU parity for the gated DELTA rule: chunked prefill and decode step
against the fp64 oracle, through the C ABI, on seeded inputs of the
workload's recipe (q, k unit rows, v normal, g = sigmoid(normal))."""
import numpy as np
import pytest
import torch

import causal_linear_attention_attn_amd as la
from causal_linear_attention_attn_amd import inputs
import oracle
from parity import TOL, assert_close, cpu

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _draw(B, H, N, d, dv, dtype, seed):
    wid = 500 + seed  # private generator streams, same recipe as the workload
    q = inputs.unit_rows((B, H, N, d), wid, 1, "cpu", dtype).to(DEV)
    k = inputs.unit_rows((B, H, N, d), wid, 2, "cpu", dtype).to(DEV)
    v = inputs.normal((B, H, N, dv), wid, 3, "cpu", 1.0, dtype).to(DEV)
    g = inputs.sigmoid_gate((B, H, N), wid, 4, "cpu").to(DEV)
    return q, k, v, g


def _oracle(q, k, v, g, S0=None):
    return oracle.delta_prefill(cpu(q), cpu(k), cpu(v), cpu(g), S0=cpu(S0))


SHAPES = [  # (B, H, N, d, dv)
    (1, 1, 1, 128, 128), (1, 2, 3, 16, 16), (2, 1, 63, 64, 64), (1, 1, 64, 128, 128),
    (1, 2, 65, 64, 64), (2, 2, 200, 128, 128), (1, 3, 130, 64, 128),
    (1, 2, 97, 128, 64), (1, 1, 17, 4, 3), (2, 1, 50, 100, 72), (1, 1, 70, 2, 2),
    (1, 8, 150, 128, 40),
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_delta_prefill_small(shape, dtype):
    B, H, N, d, dv = shape
    seed = B * 7 + H * 11 + N * 13 + d * 17 + dv * 19 + 3 * (dtype == torch.bfloat16)
    q, k, v, g = _draw(B, H, N, d, dv, dtype, seed)
    o, S, z = la.prefill(q, k, v, rule="delta", g=g)
    torch.cuda.synchronize()
    assert z is None
    ro, rS = _oracle(q, k, v, g)
    assert_close(o, ro, TOL[dtype], "o")
    assert_close(S, rS, TOL[dtype], "S", axes=(-2, -1))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_delta_prefill_initial_state_in_place(dtype):
    """S_in given and S_out aliasing it; heads not a multiple of 8."""
    B, H, N, d, dv = 1, 3, 333, 128, 128
    q, k, v, g = _draw(B, H, N, d, dv, dtype, 40)
    S = inputs.normal((B, H, d, dv), 540, 5, "cpu", 0.3).to(DEV)
    S0 = S.clone()
    o, _, _ = la.prefill(q, k, v, rule="delta", g=g, S_in=S, S_out=S)
    torch.cuda.synchronize()
    ro, rS = _oracle(q, k, v, g, S0)
    assert_close(o, ro, TOL[dtype], "o")
    assert_close(S, rS, TOL[dtype], "S", axes=(-2, -1))


def test_delta_gate_zero_keeps_state():
    """g = 0 writes nothing: S_out = S_in and o_t = S_in^T q_t."""
    B, H, N, d, dv = 1, 8, 100, 128, 128
    q, k, v, _ = _draw(B, H, N, d, dv, torch.float32, 41)
    g = torch.zeros((B, H, N), device=DEV)
    S0 = inputs.normal((B, H, d, dv), 541, 5, "cpu", 0.3).to(DEV)
    o, S, _ = la.prefill(q, k, v, rule="delta", g=g, S_in=S0)
    torch.cuda.synchronize()
    assert torch.equal(S, S0)
    ref = torch.einsum("bhnd,bhde->bhne", cpu(q).double(), cpu(S0).double())
    assert_close(o, ref.numpy(), 1e-5, "o = S_in^T q")


def test_delta_deterministic_and_guarded():
    B, H, N, d, dv = 2, 4, 333, 128, 128
    q, k, v, g = _draw(B, H, N, d, dv, torch.bfloat16, 42)
    n = B * H * N * dv
    guard = 4096
    buf = torch.full((n + 2 * guard,), float("nan"), dtype=torch.bfloat16, device=DEV)
    o = buf[guard:guard + n].view(B, H, N, dv)
    la.prefill(q, k, v, rule="delta", g=g, o=o, return_state=False)
    o1 = o.clone()
    la.prefill(q, k, v, rule="delta", g=g, o=o, return_state=False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o)
    assert torch.isnan(buf[:guard]).all() and torch.isnan(buf[guard + n:]).all()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("dims", [(128, 128), (64, 64), (4, 3), (100, 72)],
                         ids=lambda s: "x".join(map(str, s)))
def test_delta_decode_steps(dims, dtype):
    d, dv = dims
    B, H, steps = 3, 5, 6
    S = inputs.normal((B, H, d, dv), 542, 5, "cpu", 0.3).to(DEV)
    rS = cpu(S).double().numpy()
    for t in range(steps):
        q, k, v, g = _draw(B, H, 1, d, dv, dtype, 60 + t)
        q, k, v, g = q[:, :, 0].contiguous(), k[:, :, 0].contiguous(), \
            v[:, :, 0].contiguous(), g[:, :, 0].contiguous()
        o = la.decode_step(q, k, v, S, rule="delta", g=g)
        torch.cuda.synchronize()
        ro, rS = oracle.delta_decode_step(cpu(q), cpu(k), cpu(v), cpu(g), rS)
        assert_close(o, ro, TOL[dtype], f"o step {t}")
    assert_close(S, rS, 1e-5, "S", axes=(-2, -1))


def test_delta_prefill_then_decode_handoff():
    """prefill(N) then one decode step equals row N of prefill(N+1)."""
    B, H, N, d, dv = 2, 2, 257, 128, 128
    q, k, v, g = _draw(B, H, N + 1, d, dv, torch.bfloat16, 43)
    _, S, _ = la.prefill(q[:, :, :N].contiguous(), k[:, :, :N].contiguous(),
                         v[:, :, :N].contiguous(), rule="delta", g=g[:, :, :N].contiguous())
    o = la.decode_step(q[:, :, N].contiguous(), k[:, :, N].contiguous(),
                       v[:, :, N].contiguous(), S, rule="delta", g=g[:, :, N].contiguous())
    torch.cuda.synchronize()
    ro, rS = _oracle(q, k, v, g)
    assert_close(o, ro[:, :, N], 2e-2, "decode after prefill")
    assert_close(S, rS, 2e-2, "S", axes=(-2, -1))


@pytest.mark.parametrize("wid", [5, 6], ids=["plain", "alpha"])
def test_delta_workload_full_size_sampled(wid):
    """The gated-delta workloads at full size (B=2 H=16 N=8192 d=dv=128,
    bf16; without and with the state decay alpha), launched as the benchmark
    launches them; two whole heads are checked against the oracle token by
    token."""
    w = inputs.WORKLOADS[wid]
    x = inputs.make_prefill(w, DEV)
    al = x.get("alpha")
    o, S, _ = la.prefill(x["q"], x["k"], x["v"], rule="delta", g=x["g"], alpha=al)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (1, 13)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ro, rS = oracle.delta_prefill(cpu(x["q"][sl]), cpu(x["k"][sl]), cpu(x["v"][sl]),
                                      cpu(x["g"][sl]),
                                      alpha=None if al is None else cpu(al[sl]))
        assert_close(o[sl], ro, 2e-2, f"o head ({b},{h})")
        assert_close(S[sl], rS, 2e-2, f"S head ({b},{h})", axes=(-2, -1))


# --- scalar state decay (Gated DeltaNet) ------------------------------------

def _alpha(B, H, N, seed, lo):
    return inputs.decay_gate((B, H, N), 500 + seed, 6, "cpu", lo).to(DEV)


GDN_SHAPES = [  # (B, H, N, d, dv)
    (1, 1, 1, 128, 128), (1, 2, 3, 16, 16), (2, 1, 63, 64, 64), (1, 2, 65, 64, 64),
    (2, 2, 200, 128, 128), (1, 3, 130, 64, 128), (1, 1, 17, 4, 3), (2, 1, 50, 100, 72),
    (1, 8, 150, 128, 40),
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("shape", GDN_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gdn_prefill_small(shape, dtype):
    """Decay in (0.9, 1), the range gated models use."""
    B, H, N, d, dv = shape
    seed = B * 5 + H * 7 + N * 3 + d + dv * 2 + 9 * (dtype == torch.bfloat16)
    q, k, v, g = _draw(B, H, N, d, dv, dtype, seed)
    al = _alpha(B, H, N, seed, 0.9)
    o, S, _ = la.prefill(q, k, v, rule="delta", g=g, alpha=al)
    torch.cuda.synchronize()
    ro, rS = oracle.delta_prefill(cpu(q), cpu(k), cpu(v), cpu(g), alpha=cpu(al))
    assert_close(o, ro, TOL[dtype], "o")
    assert_close(S, rS, TOL[dtype], "S", axes=(-2, -1))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_gdn_prefill_strong_decay_initial_state(dtype):
    """Decay down to 0.3 (chunk products reach ~1e-20), initial state given,
    several chunks and a ragged tail."""
    B, H, N, d, dv = 1, 4, 333, 128, 128
    q, k, v, g = _draw(B, H, N, d, dv, dtype, 70)
    al = _alpha(B, H, N, 70, 0.3)
    S0 = inputs.normal((B, H, d, dv), 570, 5, "cpu", 0.3).to(DEV)
    o, S, _ = la.prefill(q, k, v, rule="delta", g=g, alpha=al, S_in=S0)
    torch.cuda.synchronize()
    ro, rS = oracle.delta_prefill(cpu(q), cpu(k), cpu(v), cpu(g), S0=cpu(S0), alpha=cpu(al))
    assert_close(o, ro, TOL[dtype], "o")
    assert_close(S, rS, TOL[dtype], "S", axes=(-2, -1))


def test_gdn_alpha_one_is_plain_rule():
    """alpha = 1 everywhere reproduces the plain rule.  The decay path only
    multiplies by exact ones, but it is a separate kernel instantiation whose
    fp32 operations may be ordered differently; a last-bit difference can flip
    the bf16 rounding of the state copy that feeds the next chunk, so the two
    agree to a couple of bf16 ulps (each is within ~3e-3 of the oracle),
    not bit for bit."""
    B, H, N, d, dv = 2, 2, 200, 128, 128
    q, k, v, g = _draw(B, H, N, d, dv, torch.bfloat16, 71)
    o1, S1, _ = la.prefill(q, k, v, rule="delta", g=g)
    o2, S2, _ = la.prefill(q, k, v, rule="delta", g=g, alpha=torch.ones_like(g))
    torch.cuda.synchronize()
    assert_close(o2, cpu(o1).double().numpy(), 1e-2, "o vs plain rule")
    assert_close(S2, cpu(S1).double().numpy(), 1e-2, "S vs plain rule", axes=(-2, -1))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("dims", [(128, 128), (4, 3), (100, 72)],
                         ids=lambda s: "x".join(map(str, s)))
def test_gdn_decode_steps(dims, dtype):
    d, dv = dims
    B, H, steps = 3, 5, 6
    S = inputs.normal((B, H, d, dv), 572, 5, "cpu", 0.3).to(DEV)
    rS = cpu(S).double().numpy()
    for t in range(steps):
        q, k, v, g = _draw(B, H, 1, d, dv, dtype, 80 + t)
        q, k, v, g = q[:, :, 0].contiguous(), k[:, :, 0].contiguous(), \
            v[:, :, 0].contiguous(), g[:, :, 0].contiguous()
        al = _alpha(B, H, 1, 80 + t, 0.5)[:, :, 0].contiguous()
        o = la.decode_step(q, k, v, S, rule="delta", g=g, alpha=al)
        torch.cuda.synchronize()
        ro, rS = oracle.delta_decode_step(cpu(q), cpu(k), cpu(v), cpu(g), rS, alpha=cpu(al))
        assert_close(o, ro, TOL[dtype], f"o step {t}")
    assert_close(S, rS, 1e-5, "S", axes=(-2, -1))


def test_gdn_prefill_then_decode_handoff():
    """prefill(N) then one decode step equals row N of prefill(N+1), with decay."""
    B, H, N, d, dv = 2, 2, 257, 128, 128
    q, k, v, g = _draw(B, H, N + 1, d, dv, torch.bfloat16, 73)
    al = _alpha(B, H, N + 1, 73, 0.8)
    sl = lambda x: x[:, :, :N].contiguous()  # noqa: E731
    at = lambda x: x[:, :, N].contiguous()  # noqa: E731
    _, S, _ = la.prefill(sl(q), sl(k), sl(v), rule="delta", g=sl(g), alpha=sl(al))
    o = la.decode_step(at(q), at(k), at(v), S, rule="delta", g=at(g), alpha=at(al))
    torch.cuda.synchronize()
    ro, _ = oracle.delta_prefill(cpu(q), cpu(k), cpu(v), cpu(g), alpha=cpu(al))
    assert_close(o, ro[:, :, N], TOL[torch.bfloat16], "o")
