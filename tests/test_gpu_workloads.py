"""The benchmark's workloads at full size, launched as bench.py launches them
(same seeded inputs, same entry points), with whole heads sampled and
checked against the fp64 oracle token by token.  The gated-delta workloads
have their own full-size test in test_gpu_delta.py."""
import numpy as np
import pytest
import torch

import causal_linear_attention_attn_amd as la
from causal_linear_attention_attn_amd import inputs
import oracle
from parity import TOL, assert_close, assert_grad_close, cpu, linear_grad_scales

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF16 = TOL[torch.bfloat16]


def _head(t, b, h):
    return None if t is None else t[b:b + 1, h:h + 1]


def _gamma_head(gamma, h):
    return None if gamma is None else cpu(gamma)[h:h + 1]


@pytest.mark.parametrize("wid", [2, 7, 8])
def test_prefill_workload_full_size_sampled(wid):
    """B4 H16 N4096 d64 bf16: plain, with per-key-channel decay, behind a
    width-4 short convolution (conv cache in and out)."""
    w = inputs.WORKLOADS[wid]
    x = inputs.make_prefill(w, DEV)
    cin, cout = x.get("conv_cache"), None
    if cin is not None:
        cout = torch.empty_like(cin)
    o, S, z = la.prefill(x["q"], x["k"], x["v"], gamma=x["gamma"], alpha=x.get("alpha"),
                         eps=w.eps, conv_weight=x.get("conv_weight"), conv_cache=cin,
                         conv_cache_out=cout)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (3, 13)):
        q, k, v = (cpu(_head(x[n], b, h)) for n in ("q", "k", "v"))
        al = None if x.get("alpha") is None else cpu(_head(x["alpha"], b, h))
        if cin is not None:
            W = cpu(x["conv_weight"])[h:h + 1]
            ro, rS, rz, rC = oracle.linear_prefill_conv(q, k, v, W, conv_cache=cpu(_head(cin, b, h)),
                                                        eps=w.eps, alpha=al)
            np.testing.assert_array_equal(cpu(_head(cout, b, h)).double().numpy(), rC)
        else:
            ro, rS, rz = oracle.linear_prefill(q, k, v, gamma=_gamma_head(x["gamma"], h),
                                               eps=w.eps, alpha=al)
        assert_close(_head(o, b, h), ro, BF16, f"o head ({b},{h})")
        assert_close(_head(S, b, h), rS, BF16, f"S head ({b},{h})", axes=(-2, -1))
        assert_close(_head(z, b, h), rz, BF16, f"z head ({b},{h})")


def test_long_context_workload_full_size_sampled():
    """B1 H32 N131072 d128 bf16 with per-head decay: one whole head (the
    slowest-decaying, gamma = 1 - 2^-12.75) token by token."""
    w = inputs.WORKLOADS[4]
    x = inputs.make_prefill(w, DEV)
    o, S, z = la.prefill(x["q"], x["k"], x["v"], gamma=x["gamma"], eps=w.eps)
    torch.cuda.synchronize()
    h = w.H - 1
    q, k, v = (cpu(_head(x[n], 0, h)) for n in ("q", "k", "v"))
    ro, rS, rz = oracle.linear_prefill(q, k, v, gamma=_gamma_head(x["gamma"], h), eps=w.eps)
    assert_close(_head(o, 0, h), ro, BF16, f"o head (0,{h})")
    assert_close(_head(S, 0, h), rS, BF16, f"S head (0,{h})", axes=(-2, -1))


def test_config1_fp32_prefill_as_stated():
    """B1 H1 N256 d=dv=64, fp32 q, k, v ~ N(0,1) unscaled from the seed,
    elu+1, gamma = 1, eps = 1e-6, full-sequence prefill: o, S and z against
    the oracle at 1e-4 on the plain row metric.
    (The workload's three-token hand-worked example runs in
    test_gpu_linear.test_handworked_example_on_gpu.)"""
    w = inputs.WORKLOADS[1]
    x = inputs.make_prefill(w, DEV)
    assert x["q"].dtype == torch.float32 and tuple(x["q"].shape) == (1, 1, 256, 64)
    assert x["gamma"] is None and w.scale == 1.0 and w.eps == 1e-6
    o, S, z = la.prefill(x["q"], x["k"], x["v"], eps=w.eps)
    torch.cuda.synchronize()
    ro, rS, rz = oracle.linear_prefill(cpu(x["q"]), cpu(x["k"]), cpu(x["v"]), eps=w.eps)
    tol = TOL[torch.float32]
    assert_close(o, ro, tol, "o")
    assert_close(S, rS, tol, "S", axes=(-2, -1))
    assert_close(z, rz, tol, "z")


def test_decode_workload_full_loop_sampled():
    """B256 H32 d128: the 1024-token prefill that builds the state, then all
    1024 decode steps over every sequence, launched as the benchmark launches
    them; two heads against the oracle at every step (o), and their final
    state."""
    w = inputs.WORKLOADS[3]
    x = inputs.make_prefill(w, DEV)
    _, S, z = la.prefill(x["q"], x["k"], x["v"], eps=w.eps)
    heads = ((0, 0), (255, 31))
    ref = {}
    for b, h in heads:
        ref[b, h] = oracle.linear_prefill(*(cpu(_head(x[n], b, h)) for n in ("q", "k", "v")),
                                          eps=w.eps)[1:]
    del x
    dec = inputs.make_decode(w, DEV, steps=w.decode_steps)
    o = torch.empty((w.B, w.H, w.dv), dtype=w.dtype, device=DEV)
    outs = {bh: [] for bh in heads}
    for t in range(w.decode_steps):
        la.decode_step(dec["q"][t], dec["k"][t], dec["v"][t], S, z, eps=w.eps, o=o)
        for b, h in heads:
            outs[b, h].append(o[b, h].clone())
    torch.cuda.synchronize()
    for b, h in heads:
        rS, rz = ref[b, h]
        got = torch.stack(outs[b, h]).cpu()
        want = []
        for t in range(w.decode_steps):
            ro, rS, rz = oracle.linear_decode_step(
                *(cpu(dec[n][t][b:b + 1, h:h + 1]) for n in ("q", "k", "v")), rS, rz, eps=w.eps)
            want.append(ro[0, 0])
        assert_close(got, np.stack(want), BF16, f"o, 1024 steps, head ({b},{h})")
        assert_close(_head(S, b, h), rS, BF16, f"S head ({b},{h})", axes=(-2, -1))
        assert_close(_head(z, b, h), rz, BF16, f"z head ({b},{h})")


def test_training_step_full_size_sampled():
    """The benchmark's training step (B4 H16 N4096 d64 bf16): prefill with
    denominators into a kept workspace, backward for the seeded dL/do
    reading the forward's segment states from it; dq, dk, dv of two heads
    against the oracle's backward."""
    w = inputs.WORKLOADS[2]
    x = inputs.make_prefill(w, DEV)
    do = inputs.make_grad_out(w, DEV)
    den = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(la.workspace_size(x["q"], x["k"], x["v"], gamma=x["gamma"], eps=w.eps),
                         1), dtype=torch.uint8, device=DEV)
    o, _, _ = la.prefill(x["q"], x["k"], x["v"], gamma=x["gamma"], eps=w.eps, den_out=den,
                         workspace=ws, return_state=False)
    dq, dk, dv, _, _ = la.backward(x["q"], x["k"], x["v"], o, den, do, gamma=x["gamma"],
                                   state_grad=False, fwd_workspace=ws)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (3, 13)):
        q, k, v, g = (cpu(_head(t, b, h)) for t in (x["q"], x["k"], x["v"], do))
        rq, rk, rv, _, _ = oracle.linear_backward(q, k, v, g, eps=w.eps)
        ro, _, _ = oracle.linear_prefill(q, k, v, eps=w.eps)
        rden = oracle.linear_denominators(q, k, eps=w.eps)
        sq, sk, sv, _, _ = linear_grad_scales(q, k, v, g, ro, rden)
        assert_grad_close(_head(dq, b, h), rq, sq, BF16, f"dq head ({b},{h})")
        assert_grad_close(_head(dk, b, h), rk, sk, BF16, f"dk head ({b},{h})")
        assert_grad_close(_head(dv, b, h), rv, sv, BF16, f"dv head ({b},{h})")
