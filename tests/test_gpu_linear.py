"""GPU parity for the LINEAR rule: chunked prefill and decode step against the
fp64 oracle, through the C ABI, on seeded inputs."""
import numpy as np
import pytest
import torch

import causal_linear_attention_attn_amd as la
from causal_linear_attention_attn_amd import inputs
import oracle
from parity import TOL, assert_close, assert_terms_close, linear_output_scale, cpu

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _rand(shape, dtype, seed, scale=1.0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype).to(DEV)


def _oracle_prefill(q, k, v, gamma, eps, fmap, S0=None, z0=None):
    return oracle.linear_prefill(cpu(q), cpu(k), cpu(v),
                                 gamma=None if gamma is None else cpu(gamma),
                                 eps=eps, fmap=fmap, S0=cpu(S0), z0=cpu(z0))


def test_handworked_example_on_gpu():
    x = inputs.handworked_example(DEV)
    o, S, z = la.prefill(x["q"], x["k"], x["v"], fmap="identity", eps=0.0)
    torch.cuda.synchronize()
    np.testing.assert_allclose(o[0, 0, 2].cpu().numpy(), [10 / 6, 7 / 6], rtol=1e-6)
    np.testing.assert_allclose(o[0, 0, :2].cpu().numpy(), [[1, 0], [1 / 3, 4 / 3]],
                               rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(S[0, 0].cpu().numpy(), [[4, 1], [3, 3]], rtol=1e-6)
    np.testing.assert_allclose(z[0, 0].cpu().numpy(), [2, 2], rtol=1e-6)
    # and with eps = 1e-6, as the workload runs it, against the oracle
    o2, _, _ = la.prefill(x["q"], x["k"], x["v"], fmap="identity", eps=1e-6)
    ref, _, _ = _oracle_prefill(x["q"], x["k"], x["v"], None, 1e-6, "identity")
    assert_close(o2, ref, 1e-6, "hand-worked example")


SHAPES = [  # (B, H, N, d, dv)
    (1, 1, 1, 64, 64), (1, 2, 3, 16, 16), (2, 1, 63, 64, 64), (1, 1, 64, 64, 64),
    (1, 2, 65, 64, 64), (2, 2, 200, 128, 128), (1, 3, 130, 64, 128),
    (1, 2, 97, 128, 64), (1, 1, 17, 4, 3), (2, 1, 50, 100, 72), (1, 1, 70, 2, 2),
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("decay", [False, True], ids=["nodecay", "decay"])
def test_prefill_small(shape, dtype, decay):
    B, H, N, d, dv = shape
    seed = (B * 7919 + H * 104729 + N * 31 + d * 17 + dv * 3
            + 1000 * (dtype == torch.bfloat16) + 5000 * decay)
    sc = 1 / np.sqrt(d)
    q = _rand((B, H, N, d), dtype, seed, sc)
    k = _rand((B, H, N, d), dtype, seed + 1, sc)
    v = _rand((B, H, N, dv), dtype, seed + 2)
    gamma = inputs.per_head_gamma(H, DEV) if decay else None
    o, S, z = la.prefill(q, k, v, gamma=gamma, eps=1e-6)
    torch.cuda.synchronize()
    ro, rS, rz = _oracle_prefill(q, k, v, gamma, 1e-6, "elu1")
    tol = TOL[dtype]
    if dv < 16:
        # 2 or 3 values per row: a weighted average of zero-mean values can
        # cancel to a few percent of what it averages, so the row is judged
        # against the sum of its terms' magnitudes
        assert_terms_close(o, ro, linear_output_scale(cpu(q), cpu(k), cpu(v), gamma=cpu(gamma)),
                           tol, "o")
    else:
        assert_close(o, ro, tol, "o")
    assert_close(S, rS, tol, "S", axes=(-2, -1))
    assert_close(z, rz, tol, "z")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_prefill_with_initial_state_and_identity_map(dtype):
    B, H, N, d, dv = 2, 3, 150, 64, 64
    q = _rand((B, H, N, d), dtype, 1).abs()
    k = _rand((B, H, N, d), dtype, 2).abs()
    v = _rand((B, H, N, dv), dtype, 3)
    S0 = _rand((B, H, d, dv), torch.float32, 4).abs()
    z0 = _rand((B, H, d), torch.float32, 5).abs()
    gamma = torch.tensor([0.9, 1.0, 0.99], device=DEV)
    o, S, z = la.prefill(q, k, v, fmap="identity", gamma=gamma, eps=1e-3,
                         S_in=S0, z_in=z0)
    torch.cuda.synchronize()
    ro, rS, rz = _oracle_prefill(q, k, v, gamma, 1e-3, "identity", S0, z0)
    assert_close(o, ro, TOL[dtype], "o")
    assert_close(S, rS, TOL[dtype], "S", axes=(-2, -1))
    assert_close(z, rz, TOL[dtype], "z")


@pytest.mark.parametrize("N", [3000, 4096 + 17])
def test_prefill_many_segments(N):
    """Few heads and a long sequence: the two-level scan runs with many
    segments and a ragged last chunk; S_in is given and S_out aliases it."""
    B, H, d, dv = 1, 2, 64, 64
    dtype = torch.bfloat16
    q = _rand((B, H, N, d), dtype, 10, 0.125)
    k = _rand((B, H, N, d), dtype, 11, 0.125)
    v = _rand((B, H, N, dv), dtype, 12, 0.125)
    gamma = torch.tensor([0.999, 1.0], device=DEV)
    S = _rand((B, H, d, dv), torch.float32, 13).abs()
    z = _rand((B, H, d), torch.float32, 14).abs() + 1
    S0, z0 = S.clone(), z.clone()
    assert la.workspace_size(q, k, v, gamma=gamma) > 0
    o, _, _ = la.prefill(q, k, v, gamma=gamma, S_in=S, z_in=z, S_out=S, z_out=z)
    torch.cuda.synchronize()
    ro, rS, rz = _oracle_prefill(q, k, v, gamma, 1e-6, "elu1", S0, z0)
    assert_close(o, ro, 2e-2, "o")
    assert_close(S, rS, 2e-2, "S", axes=(-2, -1))
    assert_close(z, rz, 2e-2, "z")


@pytest.mark.parametrize("case", ["d6", "misaligned_ws"])
def test_prefill_segments_scalar_slots(case):
    """Several segments where the workspace slots cannot take 16-byte
    accesses: d not a multiple of 4, or a workspace that starts 4 bytes past
    a 16-byte boundary (the summary, scan and chunk kernels then move the
    transposed slots element by element)."""
    B, H, N = 1, 2, 1000
    d, dv = (6, 5) if case == "d6" else (64, 64)
    dtype = torch.bfloat16
    q = _rand((B, H, N, d), dtype, 20, 0.5)
    k = _rand((B, H, N, d), dtype, 21, 0.5)
    v = _rand((B, H, N, dv), dtype, 22)
    gamma = torch.tensor([0.995, 1.0], device=DEV)
    S = _rand((B, H, d, dv), torch.float32, 23, 0.3)
    z = _rand((B, H, d), torch.float32, 24, 0.3).abs() + 1.0
    need = la.workspace_size(q, k, v, gamma=gamma)
    assert need > 0
    ws = None
    if case == "misaligned_ws":
        ws = torch.empty(need + 16, dtype=torch.uint8, device=DEV)[4:4 + need]
        assert ws.data_ptr() % 16 == 4
    o, S1, z1 = la.prefill(q, k, v, gamma=gamma, S_in=S, z_in=z, workspace=ws)
    torch.cuda.synchronize()
    ro, rS, rz = _oracle_prefill(q, k, v, gamma, 1e-6, "elu1", S, z)
    assert_close(o, ro, 2e-2, "o")
    assert_close(S1, rS, 2e-2, "S", axes=(-2, -1))
    assert_close(z1, rz, 2e-2, "z")


def test_gla_segments_scalar_slots():
    """Per-channel decay over several segments with d not a multiple of 4:
    the scan reads each element's row log decay from the transposed slot."""
    B, H, N, d, dv = 1, 2, 1000, 6, 5
    dtype = torch.bfloat16
    q = _rand((B, H, N, d), dtype, 30, 0.5)
    k = _rand((B, H, N, d), dtype, 31, 0.5)
    v = _rand((B, H, N, dv), dtype, 32)
    al = _alpha((B, H, N, d), 33, 0.9)
    S = _rand((B, H, d, dv), torch.float32, 34, 0.3)
    z = _rand((B, H, d), torch.float32, 35, 0.3).abs() + 1.0
    assert la.workspace_size(q, k, v, alpha=al) > 0
    o, S1, z1 = la.prefill(q, k, v, alpha=al, eps=1e-6, S_in=S, z_in=z)
    torch.cuda.synchronize()
    ro, rS, rz = _oracle_gla(q, k, v, al, S0=S, z0=z)
    assert_close(o, ro, 2e-2, "o")
    assert_close(S1, rS, 2e-2, "S", axes=(-2, -1))
    assert_close(z1, rz, 2e-2, "z")


def test_prefill_empty_sequence_passes_state_through():
    q = torch.empty((2, 2, 0, 8), dtype=torch.bfloat16, device=DEV)
    v = torch.empty((2, 2, 0, 4), dtype=torch.bfloat16, device=DEV)
    S0 = _rand((2, 2, 8, 4), torch.float32, 20)
    z0 = _rand((2, 2, 8), torch.float32, 21)
    o, S, z = la.prefill(q, q, v, S_in=S0, z_in=z0)
    torch.cuda.synchronize()
    assert o.shape == (2, 2, 0, 4)
    assert torch.equal(S, S0) and torch.equal(z, z0)
    _, S, z = la.prefill(q, q, v)
    torch.cuda.synchronize()
    assert not S.any() and not z.any()


def test_prefill_deterministic_and_guarded():
    """Two runs agree bit for bit, and nothing is written outside o."""
    B, H, N, d, dv = 2, 4, 333, 128, 128
    q = _rand((B, H, N, d), torch.bfloat16, 30, 0.09)
    k = _rand((B, H, N, d), torch.bfloat16, 31, 0.09)
    v = _rand((B, H, N, dv), torch.bfloat16, 32)
    n = B * H * N * dv
    guard = 4096
    buf = torch.full((n + 2 * guard,), float("nan"), dtype=torch.bfloat16, device=DEV)
    o = buf[guard:guard + n].view(B, H, N, dv)
    la.prefill(q, k, v, o=o, return_state=False)
    o1 = o.clone()
    la.prefill(q, k, v, o=o, return_state=False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o)
    assert torch.isnan(buf[:guard]).all() and torch.isnan(buf[guard + n:]).all()


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("dims", [(128, 128), (64, 64), (4, 3), (100, 72), (2, 2),
                                  (128, 66)], ids=lambda s: "x".join(map(str, s)))
def test_decode_steps(dims, dtype):
    d, dv = dims
    B, H, steps = 3, 5, 6
    S = _rand((B, H, d, dv), torch.float32, 40).abs() * 0.1
    z = _rand((B, H, d), torch.float32, 41).abs() + 0.5
    gamma = inputs.per_head_gamma(H, DEV)
    rS, rz = cpu(S).double().numpy(), cpu(z).double().numpy()
    for t in range(steps):
        q = _rand((B, H, d), dtype, 50 + t, 1 / np.sqrt(d))
        k = _rand((B, H, d), dtype, 60 + t, 1 / np.sqrt(d))
        v = _rand((B, H, dv), dtype, 70 + t)
        o = la.decode_step(q, k, v, S, z, gamma=gamma, eps=1e-6)
        torch.cuda.synchronize()
        ro, rS, rz = oracle.linear_decode_step(cpu(q), cpu(k), cpu(v), rS, rz,
                                               gamma=cpu(gamma), eps=1e-6)
        assert_close(o, ro, TOL[dtype], f"o step {t}")
    assert_close(S, rS, 1e-5, "S", axes=(-2, -1))
    assert_close(z, rz, 1e-5, "z")


def test_prefill_then_decode_handoff():
    """prefill(N) then one decode step equals row N of prefill(N+1)."""
    B, H, N, d, dv = 2, 2, 257, 128, 128
    sc = 1 / np.sqrt(d)
    q = _rand((B, H, N + 1, d), torch.bfloat16, 80, sc)
    k = _rand((B, H, N + 1, d), torch.bfloat16, 81, sc)
    v = _rand((B, H, N + 1, dv), torch.bfloat16, 82, sc)
    gamma = torch.tensor([0.995, 1.0], device=DEV)
    _, S, z = la.prefill(q[:, :, :N].contiguous(), k[:, :, :N].contiguous(),
                         v[:, :, :N].contiguous(), gamma=gamma)
    o = la.decode_step(q[:, :, N].contiguous(), k[:, :, N].contiguous(),
                       v[:, :, N].contiguous(), S, z, gamma=gamma)
    torch.cuda.synchronize()
    ro, rS, rz = _oracle_prefill(q, k, v, gamma, 1e-6, "elu1")
    assert_close(o, ro[:, :, N], 2e-2, "decode after prefill")
    assert_close(S, rS, 2e-2, "S", axes=(-2, -1))


def test_state_init_zeroes():
    S = torch.randn((3, 2, 16, 8), device=DEV)
    z = torch.randn((3, 2, 16), device=DEV)
    la.state_init(S, z)
    torch.cuda.synchronize()
    assert not S.any() and not z.any()


# --- per-key-channel decay (GLA) --------------------------------------------

def _alpha(shape, seed, lo):
    """Decay per key channel in (lo, 1): lo + (1 - lo) sigmoid(N(0,1))."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (lo + (1.0 - lo) * torch.sigmoid(torch.randn(shape, generator=g))).to(DEV)


def _oracle_gla(q, k, v, al, eps=1e-6, fmap="elu1", S0=None, z0=None):
    return oracle.linear_prefill(cpu(q), cpu(k), cpu(v), eps=eps, fmap=fmap,
                                 S0=cpu(S0), z0=cpu(z0), alpha=cpu(al))


GLA_SHAPES = [  # (B, H, N, d, dv)
    (1, 1, 1, 64, 64), (1, 2, 3, 16, 16), (2, 1, 63, 64, 64), (1, 2, 65, 64, 64),
    (2, 2, 200, 128, 128), (1, 3, 130, 64, 128), (1, 2, 97, 128, 64), (1, 1, 17, 4, 3),
    (2, 1, 50, 100, 72), (1, 1, 333, 64, 64),
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("shape", GLA_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gla_prefill_small(shape, dtype):
    B, H, N, d, dv = shape
    seed = 900 + B * 7 + H * 11 + N * 13 + d * 17 + dv * 19 + 3 * (dtype == torch.bfloat16)
    sc = 1 / np.sqrt(d)
    q = _rand((B, H, N, d), dtype, seed, sc)
    k = _rand((B, H, N, d), dtype, seed + 1, sc)
    v = _rand((B, H, N, dv), dtype, seed + 2)
    al = _alpha((B, H, N, d), seed + 3, 0.9)
    o, S, z = la.prefill(q, k, v, alpha=al, eps=1e-6)
    torch.cuda.synchronize()
    ro, rS, rz = _oracle_gla(q, k, v, al)
    assert_close(o, ro, TOL[dtype], "o")
    assert_close(S, rS, TOL[dtype], "S", axes=(-2, -1))
    assert_close(z, rz, TOL[dtype], "z")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("lo", [0.9, 0.3], ids=["mild", "strong"])
def test_gla_prefill_segments_and_initial_state(dtype, lo):
    """Long enough for several segments (summary + scan + chunk kernels), an
    initial state updated in place, decays down to 0.3."""
    B, H, N, d, dv = 1, 4, 4099, 64, 64
    seed = 950 + int(lo * 10) + (dtype == torch.bfloat16)
    q = _rand((B, H, N, d), dtype, seed, 0.125)
    k = _rand((B, H, N, d), dtype, seed + 1, 0.125)
    v = _rand((B, H, N, dv), dtype, seed + 2)
    al = _alpha((B, H, N, d), seed + 3, lo)
    S = _rand((B, H, d, dv), torch.float32, seed + 4, 0.3)
    z = _rand((B, H, d), torch.float32, seed + 5, 0.3).abs() + 1.0
    S0, z0 = S.clone(), z.clone()
    o, _, _ = la.prefill(q, k, v, alpha=al, eps=1e-6, S_in=S, z_in=z, S_out=S, z_out=z)
    torch.cuda.synchronize()
    ro, rS, rz = _oracle_gla(q, k, v, al, S0=S0, z0=z0)
    assert_close(o, ro, TOL[dtype], "o")
    assert_close(S, rS, TOL[dtype], "S", axes=(-2, -1))
    assert_close(z, rz, TOL[dtype], "z")


def _alpha_log(shape, seed, lo):
    """Decay per key channel log-uniform in (lo, 1): lo^u, u ~ U(0, 1)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.exp(torch.rand(shape, generator=g, dtype=torch.float64) * np.log(lo)) \
        .to(torch.float32).to(DEV)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("lo", [1e-2, 1e-3, 2.0 ** -15, 1e-6],
                         ids=["1e-2", "1e-3", "2^-15", "1e-6"])
@pytest.mark.parametrize("N", [150, 4099])
def test_gla_fast_decay(dtype, lo, N):
    """Decays log-uniform down to lo per channel and token ("Efficient
    attention variants" 7.2 lets the gate forget quickly): the block
    references keep every factor inside the fp32/bf16 range.  Below 2^-15 a
    token's decay is clamped there, where an earlier token weighs under
    3.1e-5 of the current one, inside the fp32 bound.  One segment (N = 150)
    and several (summary, scan, chunk kernels; N = 4099), with an initial
    state."""
    B, H, d, dv = 1, 4, 64, 64
    seed = 990 + int(-np.log2(lo)) + 7 * (dtype == torch.bfloat16) + N % 7
    q = _rand((B, H, N, d), dtype, seed, 0.125)
    k = _rand((B, H, N, d), dtype, seed + 1, 0.125)
    v = _rand((B, H, N, dv), dtype, seed + 2)
    al = _alpha_log((B, H, N, d), seed + 3, lo)
    S = _rand((B, H, d, dv), torch.float32, seed + 4, 0.3)
    z = _rand((B, H, d), torch.float32, seed + 5, 0.3).abs() + 1.0
    o, S1, z1 = la.prefill(q, k, v, alpha=al, eps=1e-6, S_in=S, z_in=z)
    torch.cuda.synchronize()
    ro, rS, rz = _oracle_gla(q, k, v, al, S0=S, z0=z)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S1).all()
    assert_close(o, ro, TOL[dtype], "o")
    assert_close(S1, rS, TOL[dtype], "S", axes=(-2, -1))
    assert_close(z1, rz, TOL[dtype], "z")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("dims", [(128, 128), (64, 128), (24, 40)],
                         ids=lambda s: "x".join(map(str, s)))
def test_gla_mixed_channel_decays(dtype, dims):
    """Half the key channels barely decay (alpha ~ 0.999), half forget almost
    at once (alpha ~ 1e-4): factors of both extremes in one tile."""
    d, dv = dims
    B, H, N = 2, 2, 300
    seed = 1010 + d + dv + (dtype == torch.bfloat16)
    q = _rand((B, H, N, d), dtype, seed, d ** -0.5)
    k = _rand((B, H, N, d), dtype, seed + 1, d ** -0.5)
    v = _rand((B, H, N, dv), dtype, seed + 2)
    slow = _alpha((B, H, N, d), seed + 3, 0.998)
    fast = _alpha_log((B, H, N, d), seed + 4, 1e-4) * 1e-2
    al = torch.where(torch.arange(d, device=DEV) % 2 == 0, slow, fast.clamp_min(1e-6))
    o, S, z = la.prefill(q, k, v, alpha=al, eps=1e-6)
    torch.cuda.synchronize()
    ro, rS, rz = _oracle_gla(q, k, v, al)
    assert_close(o, ro, TOL[dtype], "o")
    assert_close(S, rS, TOL[dtype], "S", axes=(-2, -1))
    assert_close(z, rz, TOL[dtype], "z")


def test_gla_uniform_alpha_matches_gamma():
    """alpha = gamma_h on every channel and token reproduces the per-head decay
    path (to bf16 resolution: different kernel instantiations)."""
    B, H, N, d, dv = 1, 4, 700, 128, 128
    q = _rand((B, H, N, d), torch.bfloat16, 960, d ** -0.5)
    k = _rand((B, H, N, d), torch.bfloat16, 961, d ** -0.5)
    v = _rand((B, H, N, dv), torch.bfloat16, 962)
    gamma = torch.tensor([0.9, 0.97, 0.99, 1.0], device=DEV)
    al = gamma[None, :, None, None].expand(B, H, N, d).contiguous()
    o1, S1, z1 = la.prefill(q, k, v, gamma=gamma, eps=1e-6)
    o2, S2, z2 = la.prefill(q, k, v, alpha=al, eps=1e-6)
    torch.cuda.synchronize()
    assert_close(o2, cpu(o1).double().numpy(), 1e-2, "o vs gamma path")
    assert_close(S2, cpu(S1).double().numpy(), 1e-2, "S vs gamma path", axes=(-2, -1))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("dims", [(128, 128), (4, 3), (100, 72)],
                         ids=lambda s: "x".join(map(str, s)))
def test_gla_decode_steps(dims, dtype):
    d, dv = dims
    B, H, steps = 3, 5, 6
    S = _rand((B, H, d, dv), torch.float32, 970, 0.3)
    z = _rand((B, H, d), torch.float32, 971, 0.3).abs() + 1.0
    rS, rz = cpu(S).double().numpy(), cpu(z).double().numpy()
    for t in range(steps):
        q = _rand((B, H, d), dtype, 972 + 5 * t, d ** -0.5)
        k = _rand((B, H, d), dtype, 973 + 5 * t, d ** -0.5)
        v = _rand((B, H, dv), dtype, 974 + 5 * t)
        al = _alpha((B, H, d), 975 + 5 * t, 0.5)
        o = la.decode_step(q, k, v, S, z, alpha=al, eps=1e-6)
        torch.cuda.synchronize()
        ro, rS, rz = oracle.linear_decode_step(cpu(q), cpu(k), cpu(v), rS, rz, eps=1e-6,
                                               alpha=cpu(al))
        assert_close(o, ro, TOL[dtype], f"o step {t}")
    assert_close(S, rS, 1e-5, "S", axes=(-2, -1))
    assert_close(z, rz, 1e-5, "z")


def test_gla_prefill_then_decode_handoff():
    B, H, N, d, dv = 2, 2, 257, 64, 64
    q = _rand((B, H, N + 1, d), torch.bfloat16, 980, 0.125)
    k = _rand((B, H, N + 1, d), torch.bfloat16, 981, 0.125)
    v = _rand((B, H, N + 1, dv), torch.bfloat16, 982)
    al = _alpha((B, H, N + 1, d), 983, 0.8)
    sl = lambda x: x[:, :, :N].contiguous()  # noqa: E731
    at = lambda x: x[:, :, N].contiguous()  # noqa: E731
    _, S, z = la.prefill(sl(q), sl(k), sl(v), alpha=sl(al), eps=1e-6)
    o = la.decode_step(at(q), at(k), at(v), S, z, alpha=at(al), eps=1e-6)
    torch.cuda.synchronize()
    ro, _, _ = _oracle_gla(q, k, v, al)
    assert_close(o, ro[:, :, N], TOL[torch.bfloat16], "o")


# --- fast decays ---------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_prefill_fast_decay_segments_then_decode(dtype):
    """Per-head decays across (0, 1]: 0.05, 0.25, 0.45 and 1e-3 forget within a
    few tokens ("What Is Linear Attention?" 5.1: smaller gamma forgets
    faster), 0.9 and 1 for contrast.  Long enough for several segments, an
    initial state, a ragged last chunk; then decode steps continue from the
    final state."""
    B, H, N, d, dv = 1, 6, 3000 + 17, 64, 64
    seed = 2100 + (dtype == torch.bfloat16)
    q = _rand((B, H, N, d), dtype, seed, 0.5)
    k = _rand((B, H, N, d), dtype, seed + 1, 0.5)
    v = _rand((B, H, N, dv), dtype, seed + 2)
    gamma = torch.tensor([0.05, 0.25, 0.45, 1e-3, 0.9, 1.0], device=DEV)
    S0 = _rand((B, H, d, dv), torch.float32, seed + 3, 0.3)
    z0 = _rand((B, H, d), torch.float32, seed + 4, 0.3).abs() + 1.0
    assert la.workspace_size(q, k, v, gamma=gamma) > 0  # several segments
    o, S, z = la.prefill(q, k, v, gamma=gamma, eps=1e-6, S_in=S0, z_in=z0)
    torch.cuda.synchronize()
    ro, rS, rz = _oracle_prefill(q, k, v, gamma, 1e-6, "elu1", S0, z0)
    tol = TOL[dtype]
    assert_close(o, ro, tol, "o")
    assert_close(S, rS, tol, "S", axes=(-2, -1))
    assert_close(z, rz, tol, "z")
    for t in range(3):
        q1 = _rand((B, H, d), dtype, seed + 10 + 3 * t, 0.5)
        k1 = _rand((B, H, d), dtype, seed + 11 + 3 * t, 0.5)
        v1 = _rand((B, H, dv), dtype, seed + 12 + 3 * t)
        o1 = la.decode_step(q1, k1, v1, S, z, gamma=gamma, eps=1e-6)
        torch.cuda.synchronize()
        r1, rS, rz = oracle.linear_decode_step(cpu(q1), cpu(k1), cpu(v1), rS, rz,
                                               gamma=cpu(gamma), eps=1e-6)
        assert_close(o1, r1, tol, f"decode step {t}")
    assert_close(S, rS, tol, "S after decode", axes=(-2, -1))


@pytest.mark.parametrize("shape", [(1, 3, 200, 128, 128), (2, 2, 97, 24, 40)],
                         ids=lambda s: "x".join(map(str, s)))
def test_prefill_fast_decay_identity_map(shape):
    """Fast decays with the identity map (features given directly, many of
    them zero) and one segment: scores, state read and state update all take
    their own decay factors."""
    B, H, N, d, dv = shape
    q = _rand((B, H, N, d), torch.bfloat16, 2150, 0.5).abs()
    k = _rand((B, H, N, d), torch.bfloat16, 2151, 0.5).abs()
    v = _rand((B, H, N, dv), torch.bfloat16, 2152)
    gamma = torch.tensor([0.05, 0.3, 0.45][:H], device=DEV)
    S0 = _rand((B, H, d, dv), torch.float32, 2153, 0.3).abs()
    z0 = _rand((B, H, d), torch.float32, 2154, 0.3).abs() + 1.0
    o, S, z = la.prefill(q, k, v, fmap="identity", gamma=gamma, eps=1e-3, S_in=S0, z_in=z0)
    torch.cuda.synchronize()
    ro, rS, rz = _oracle_prefill(q, k, v, gamma, 1e-3, "identity", S0, z0)
    assert_close(o, ro, 2e-2, "o")
    assert_close(S, rS, 2e-2, "S", axes=(-2, -1))
    assert_close(z, rz, 2e-2, "z")
