#!/usr/bin/env python3
"""Benchmark of the causal linear attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2|4|5]
                    [--no-decode] [--no-cpu-baseline]

Prints ONE JSON line.  A "step" is one la_prefill call over the whole batch
of the workload (default: B=4 H=16 N=4096 d=dv=64 bf16, elu+1, gamma=1,
eps=1e-6) with inputs already resident in HBM; `value` is prefill tokens/s
(B*N tokens per step).  Alongside:
  roofline      the dominant kernel (phase-3 chunk kernel) against HBM peak:
                algorithmic bytes per launch (q, k, v read once, o written
                once) over its average duration, timed with HIP events that
                the library records around each kernel on its launch stream;
  mfma          the same kernel's chunk-form matrix flops against the bf16
                dense peak;
  decode        the decode-step loop (B=256 H=32 d=dv=128: state built by a
                1024-token prefill, then 1024 single-token steps): steps/s and
                state GB/s against HBM peak;
  cpu_baseline  the fp64 oracle on the host cores over the same inputs
                (a reported baseline, not a target), plus its parity error.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 (matrix / vector)
METRIC = "prefill tokens/sec + % bf16 MFMA peak; decode state GB/s vs HBM peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2, choices=[2, 4, 5])
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=1024)
    return ap.parse_args()


class KernelTimer:
    """HIP-event kernel durations recorded by the library itself."""

    def __init__(self, lib):
        from causal_linear_attention_attn_amd import _lib

        self.lib, self.KT = lib, _lib.KernelTime

    def __enter__(self):
        self.lib.la_profile_enable(1)
        return self

    def collect(self):
        buf = (self.KT * 65536)()
        n = self.lib.la_profile_collect(buf, 65536)
        if n < 0:
            raise RuntimeError("la_profile_collect failed")
        out = {}
        for i in range(n):
            out.setdefault(buf[i].name.decode(), []).append(buf[i].ms)
        return out

    def __exit__(self, *exc):
        self.lib.la_profile_enable(0)


def chunk_flops_per_head_token(d, dv, C):
    """Matrix flops of the chunk form per head-token: state read 2*d*dv,
    state update 2*d*dv, intra-chunk scores and weighted sum 2*C*(d+dv)
    (the full C x C tiles, as computed)."""
    return 4 * d * dv + 2 * C * (d + dv)


def bench_prefill(la, lib, torch, w, steps, warmup):
    from causal_linear_attention_attn_amd import inputs

    x = inputs.make_prefill(w, "cuda")
    q, k, v, gamma = x["q"], x["k"], x["v"], x["gamma"]
    B, H, N, d, dv = w.B, w.H, w.N, w.d, w.dv
    o = torch.empty((B, H, N, dv), dtype=w.dtype, device="cuda")
    S = torch.empty((B, H, d, dv), dtype=torch.float32, device="cuda")
    z = torch.empty((B, H, d), dtype=torch.float32, device="cuda")
    ws_bytes = la.workspace_size(q, k, v, gamma=gamma, eps=w.eps)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

    def step():
        la.prefill(q, k, v, gamma=gamma, eps=w.eps, o=o, S_out=S, z_out=z,
                   workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    with KernelTimer(lib) as kt:
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        times = kt.collect()
    dt = (t1 - t0) / steps
    kern = {n: sum(v) / len(v) for n, v in times.items()}
    rec = d * dv + d
    nseg = ws_bytes // (B * H * rec * 4) if ws_bytes else 1
    return dict(x=x, o=o, S=S, z=z, dt=dt, kern=kern, ws_bytes=ws_bytes, nseg=nseg)


def bench_decode(la, lib, torch, nsteps, warmup=8):
    from causal_linear_attention_attn_amd import inputs

    w = inputs.WORKLOADS[3]
    B, H, d, dv = w.B, w.H, w.d, w.dv
    x = inputs.make_prefill(w, "cuda")
    _, S, z = la.prefill(x["q"], x["k"], x["v"], eps=w.eps)
    del x
    dec = inputs.make_decode(w, "cuda", steps=nsteps)
    o = torch.empty((B, H, dv), dtype=w.dtype, device="cuda")
    # warm-up steps on a scratch copy of the state
    S2, z2 = S.clone(), z.clone()
    for t in range(min(warmup, nsteps)):
        la.decode_step(dec["q"][t], dec["k"][t], dec["v"][t], S2, z2, eps=w.eps, o=o)
    del S2, z2
    torch.cuda.synchronize()
    with KernelTimer(lib) as kt:
        t0 = time.perf_counter()
        for t in range(nsteps):
            la.decode_step(dec["q"][t], dec["k"][t], dec["v"][t], S, z, eps=w.eps, o=o)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        times = kt.collect()
    ks = times.get("linear_decode", [])
    kavg = sum(ks) / len(ks) if ks else float("nan")
    step_bytes = 2 * (S.numel() + z.numel()) * 4 + (3 * B * H * d + B * H * dv) * 2
    dt = (t1 - t0) / nsteps
    return {
        "workload": w.name, "steps": nsteps,
        "steps_per_s": 1.0 / dt, "tokens_per_s": B / dt, "ms_per_step": dt * 1e3,
        "kernel_ms": kavg, "bytes_per_step": step_bytes,
        "achieved_GBs": step_bytes / (kavg * 1e-3) / 1e9,
        "hbm_frac": step_bytes / (kavg * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "loop_GBs": step_bytes / dt / 1e9,
    }


def cpu_baseline(res, w, target_s=20.0):
    """Time the fp64 oracle on a bounded sample of the same inputs (whole
    heads, all N tokens) on one host core, and report its parity error."""
    import numpy as np

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    import oracle

    x = res["x"]
    H = w.H
    q, k, v = (x[n][0].cpu() for n in ("q", "k", "v"))  # batch 0: [H, N, d]
    gamma = None if x["gamma"] is None else x["gamma"].cpu()
    # sample: the first `nh` heads of batch 0, sized from a short probe
    probe_tok = 256
    t = time.perf_counter()
    oracle.linear_prefill(q[None, :1, :probe_tok], k[None, :1, :probe_tok],
                          v[None, :1, :probe_tok], eps=w.eps,
                          gamma=None if gamma is None else gamma[:1])
    per_ht = (time.perf_counter() - t) / probe_tok
    nh = int(max(1, min(H, target_s / (per_ht * w.N))))
    ctx = threadpool_limits(1) if threadpool_limits else None
    t0 = time.perf_counter()
    ro, _, _ = oracle.linear_prefill(q[None, :nh], k[None, :nh], v[None, :nh],
                                     eps=w.eps, gamma=None if gamma is None else gamma[:nh])
    el = time.perf_counter() - t0
    if ctx:
        ctx.__exit__(None, None, None)
    got = res["o"][0, :nh].detach().cpu().double().numpy()
    diff = np.abs(got - ro[0]).max(axis=-1)
    scale = np.abs(ro[0]).max(axis=-1)
    err = float((diff / np.where(scale > 0, scale, 1.0)).max())
    head_tokens = nh * w.N
    return {
        "value": head_tokens / H / el, "unit": "tokens/s", "cores": 1,
        "kind": "oracle",
        "sample": f"batch 0, heads 0..{nh - 1} of {H}, all {w.N} tokens "
                  f"({head_tokens} head-tokens, {el:.1f} s); tokens/s = "
                  f"head-tokens/s / H",
        "parity_max_row_rel_err": err,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path shards by (batch, head) with no communication, so N "
              "GPUs would each run this same single-GPU step.", file=sys.stderr)
        sys.exit(2)
    import torch

    import causal_linear_attention_attn_amd as la
    from causal_linear_attention_attn_amd import _lib, inputs

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    lib = _lib.load()
    w = inputs.WORKLOADS[args.workload]
    res = bench_prefill(la, lib, torch, w, args.steps, args.warmup)
    B, H, N, d, dv = w.B, w.H, w.N, w.d, w.dv
    head_tokens = B * H * N
    tok_s = B * N / res["dt"]

    line = {
        "metric": METRIC, "value": tok_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": res["dt"] * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
        "data": "synthetic (seeded normal draws, see inputs.py)",
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "d": d, "dv": dv,
                   "rule": w.rule, "fmap": w.fmap, "decay": w.decay,
                   "eps": w.eps, "head_tokens_per_step": head_tokens},
        "kernels_ms": res["kern"],
        "plan": {"segments_per_sequence": res["nseg"], "workspace_bytes": res["ws_bytes"]},
    }
    if w.rule == "linear":
        kname = "linear_chunk"
        bpht = (2 * d + dv) * 2 + dv * 2  # q, k, v read + o written, bf16
        flops_pht = chunk_flops_per_head_token(d, dv, 64)
    else:
        kname = "delta_seq"
        bpht = (2 * d + dv) * 2 + 4 + dv * 2
        flops_pht = 0
    kms = res["kern"].get(kname)
    if kms:
        achieved = head_tokens * bpht / (kms * 1e-3) / 1e9
        line["roofline"] = {
            "kernel": kname, "bound": "hbm", "achieved": achieved,
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
            "traffic": None, "bytes_per_launch": head_tokens * bpht,
            "kernel_ms": kms,
        }
        if flops_pht:
            tf = head_tokens * flops_pht / (kms * 1e-3) / 1e12
            line["mfma"] = {"kernel": kname, "chunk": 64,
                            "flops_per_launch": head_tokens * flops_pht,
                            "achieved_tflops": tf, "peak_tflops": BF16_PEAK_TFLOPS,
                            "frac": tf / BF16_PEAK_TFLOPS}
        step_bytes = head_tokens * bpht
        line["step_hbm_frac"] = step_bytes / res["dt"] / 1e9 / HBM_PEAK_GBS
    if not args.no_decode:
        line["decode"] = bench_decode(la, lib, torch, args.decode_steps)
    if not args.no_cpu_baseline and w.rule == "linear":
        line["cpu_baseline"] = cpu_baseline(res, w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
