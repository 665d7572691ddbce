"""Seeded synthetic inputs for the benchmark and test workloads.

This module only draws random tensors and rounds them to the storage dtype;
it holds none of the method's arithmetic.  Both the HIP path and the fp64
oracle are fed the very tensors made here (the oracle gets an exact fp64
upcast), so no value is ever generated twice.

Every tensor comes from its own torch.Generator seeded with
1000 * workload + tensor id, on the device the caller asks for.  Draws are
fp32 normal (or the stated transform of it) and are rounded to bf16 by
torch's round-to-nearest-even conversion.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

# tensor ids inside one workload
_Q, _K, _V, _G, _A, _W = 1, 2, 3, 4, 5, 6
_DEC_Q, _DEC_K, _DEC_V = 11, 12, 13
_DO = 21  # gradient of the loss with respect to o (training step)


@dataclass(frozen=True)
class Workload:
    """One workload: shapes, rule, feature map, decay and input recipe."""
    wid: int
    name: str
    B: int
    H: int
    N: int
    d: int
    dv: int
    dtype: torch.dtype
    rule: str              # "linear" or "delta"
    fmap: str              # "elu1" or "identity"
    scale: float           # std of the q, k, v draws
    eps: float = 1e-6
    decay: str = "none"    # "none", "per_head" (gamma_h = 1 - 2^(-5 - h/4)),
                           # "alpha" (delta rule: per-token state decay in (0.9, 1))
                           # or "channel" (linear rule: per-key-channel decay in (0.9, 1))
    decode_steps: int = 0  # > 0: a decode loop follows the prefill
    conv: int = 0          # > 0: short causal convolution of this width in
                           # front of q, k, v (filters N(0, 1/w), zero cache)
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    1: Workload(1, "linear_fp32_B1H1N256d64", 1, 1, 256, 64, 64, torch.float32,
                "linear", "elu1", 1.0),
    2: Workload(2, "linear_bf16_prefill_B4H16N4096d64", 4, 16, 4096, 64, 64,
                torch.bfloat16, "linear", "elu1", 1.0 / math.sqrt(64)),
    3: Workload(3, "linear_bf16_decode_B256H32d128_1024prefill_1024steps", 256,
                32, 1024, 128, 128, torch.bfloat16, "linear", "elu1",
                1.0 / math.sqrt(128), decode_steps=1024),
    4: Workload(4, "linear_bf16_decay_prefill_B1H32N131072d128", 1, 32, 131072,
                128, 128, torch.bfloat16, "linear", "elu1",
                1.0 / math.sqrt(128), decay="per_head"),
    5: Workload(5, "delta_bf16_prefill_B2H16N8192d128", 2, 16, 8192, 128, 128,
                torch.bfloat16, "delta", "identity", 1.0),
    # the gated delta workload with Gated DeltaNet's scalar decay added
    6: Workload(6, "delta_decay_bf16_prefill_B2H16N8192d128", 2, 16, 8192, 128, 128,
                torch.bfloat16, "delta", "identity", 1.0, decay="alpha"),
    # the B4 H16 N4096 d64 prefill with GLA's per-key-channel decay
    7: Workload(7, "linear_gla_bf16_prefill_B4H16N4096d64", 4, 16, 4096, 64, 64,
                torch.bfloat16, "linear", "elu1", 1.0 / math.sqrt(64), decay="channel"),
    # the same prefill behind a width-4 short convolution of q, k, v
    8: Workload(8, "linear_conv_bf16_prefill_B4H16N4096d64", 4, 16, 4096, 64, 64,
                torch.bfloat16, "linear", "elu1", 1.0 / math.sqrt(64), conv=4),
}


def _gen(wid, tid, device):
    g = torch.Generator(device=device)
    g.manual_seed(1000 * wid + tid)
    return g


def normal(shape, wid, tid, device, scale=1.0, dtype=torch.float32):
    """fp32 N(0, scale^2) draws, rounded to `dtype`."""
    x = torch.randn(shape, generator=_gen(wid, tid, device), device=device,
                    dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(dtype)


def unit_rows(shape, wid, tid, device, dtype=torch.float32):
    """N(0,1) draws normalised to unit L2 norm along the last axis in fp32,
    then rounded to `dtype` (so the stored rows are unit to ~2^-8)."""
    x = torch.randn(shape, generator=_gen(wid, tid, device), device=device,
                    dtype=torch.float32)
    x.div_(torch.linalg.vector_norm(x, dim=-1, keepdim=True))
    return x.to(dtype)


def sigmoid_gate(shape, wid, tid, device):
    """g = sigmoid(N(0,1)) in fp32."""
    x = torch.randn(shape, generator=_gen(wid, tid, device), device=device,
                    dtype=torch.float32)
    return torch.sigmoid(x)


def decay_gate(shape, wid, tid, device, lo):
    """alpha = lo + (1 - lo) sigmoid(N(0,1)) in fp32: a per-token state decay
    in (lo, 1)."""
    x = torch.randn(shape, generator=_gen(wid, tid, device), device=device,
                    dtype=torch.float32)
    return lo + (1.0 - lo) * torch.sigmoid(x)


def per_head_gamma(H, device="cpu"):
    """gamma_h = 1 - 2^(-5 - h/4), h = 0..H-1, as fp32."""
    h = torch.arange(H, dtype=torch.float64)
    return (1.0 - torch.pow(2.0, -5.0 - h / 4.0)).to(torch.float32).to(device)


def make_prefill(w: Workload, device, *, B=None, H=None, N=None):
    """q, k, v (and g for the delta rule, gamma for per-head decay) of a
    workload, optionally with a smaller B, H or N (same recipe, same seeds:
    a smaller shape is not a prefix of the full one)."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    N = w.N if N is None else N
    out = {}
    if w.rule == "delta":
        out["q"] = unit_rows((B, H, N, w.d), w.wid, _Q, device, w.dtype)
        out["k"] = unit_rows((B, H, N, w.d), w.wid, _K, device, w.dtype)
        out["v"] = normal((B, H, N, w.dv), w.wid, _V, device, w.scale, w.dtype)
        out["g"] = sigmoid_gate((B, H, N), w.wid, _G, device)
        if w.decay == "alpha":
            out["alpha"] = decay_gate((B, H, N), w.wid, _A, device, 0.9)
    else:
        out["q"] = normal((B, H, N, w.d), w.wid, _Q, device, w.scale, w.dtype)
        out["k"] = normal((B, H, N, w.d), w.wid, _K, device, w.scale, w.dtype)
        out["v"] = normal((B, H, N, w.dv), w.wid, _V, device, w.scale, w.dtype)
        if w.decay == "channel":
            out["alpha"] = decay_gate((B, H, N, w.d), w.wid, _A, device, 0.9)
        if w.conv:
            out["conv_weight"] = normal((H, w.conv, 2 * w.d + w.dv), w.wid, _W, device,
                                        w.conv ** -0.5)
            out["conv_cache"] = torch.zeros((B, H, w.conv - 1, 2 * w.d + w.dv),
                                            dtype=w.dtype, device=device)
    out["gamma"] = per_head_gamma(H, device) if w.decay == "per_head" else None
    return out


def make_grad_out(w: Workload, device):
    """dL/do for a training step: N(0,1) draws of o's shape, in w.dtype."""
    return normal((w.B, w.H, w.N, w.dv), w.wid, _DO, device, 1.0, w.dtype)


def make_decode(w: Workload, device, *, B=None, H=None, steps=None):
    """Fresh q, k, v for every decode step, stacked as [steps, B, H, d]."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    steps = w.decode_steps if steps is None else steps
    return {
        "q": normal((steps, B, H, w.d), w.wid, _DEC_Q, device, w.scale, w.dtype),
        "k": normal((steps, B, H, w.d), w.wid, _DEC_K, device, w.scale, w.dtype),
        "v": normal((steps, B, H, w.dv), w.wid, _DEC_V, device, w.scale, w.dtype),
    }


def handworked_example(device, dtype=torch.float32):
    """The three-token example with features given directly (identity map):
    phi(k) = [1,0],[0,1],[1,1]; v = [1,0],[0,2],[3,1]; phi(q_t) = [1,2] at
    every position.  Shapes [1, 1, 3, 2]."""
    k = torch.tensor([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    v = torch.tensor([[1.0, 0.0], [0.0, 2.0], [3.0, 1.0]])
    q = torch.tensor([[1.0, 2.0]] * 3)
    return {n: t.reshape(1, 1, 3, 2).to(device=device, dtype=dtype)
            for n, t in (("q", q), ("k", k), ("v", v))}
