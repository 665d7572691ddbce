#!/usr/bin/env python3
"""Benchmark of the causal linear attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2..8]
                    [--no-decode] [--no-extra] [--no-train] [--no-cpu-baseline]

Prints ONE JSON line.  A "step" is one la_prefill call over the whole batch
of the workload (default: B=4 H=16 N=4096 d=dv=64 bf16 q, k, v, elu+1,
gamma=1, eps=1e-6, bf16 output) with inputs already resident in HBM.
Steps are replayed from HIP graphs holding 8 consecutive la_prefill calls
each, issued back to back on one stream as a serving loop issues them (so
neither host-side argument marshalling nor the per-graph launch is timed per
step); `value` is prefill tokens/s, B*N tokens per step, and
`ms_one_step_alone` the wall time of one step replayed alone from a one-step
graph.  Alongside:
  roofline      the dominant kernel against HBM peak: algorithmic bytes per
                launch (q, k, v read once, o written once) over its average
                duration, from the HIP event pair the library hands to each
                of its kernel dispatches (stamped at kernel start and end on
                the launch stream; eager run of the same step); `traffic` is
                the HBM bytes per launch from committed rocprofv3 byte-counter
                summaries of the same kernel source, else null;
  mfma          the same kernel's chunk-form matrix flops against the bf16
                dense matrix peak;
  decode        the decode-step loop (B=256 H=32 d=dv=128, state built by a
                1024-token prefill, then 1024 single-token steps with fresh
                q, k, v): steps/s and state GB/s against HBM peak;
  workloads     the long-context decay prefill (B=1 H=32 N=131072 d=128), the
                gated delta-rule prefill (B=2 H=16 N=8192 d=128), the same
                with a per-token state decay alpha in (0.9, 1), the main
                workload with a per-key-channel decay (GLA), and the main
                workload behind a width-4 short convolution of q, k, v (conv
                cache in and out), each with its kernels' times and HBM
                fraction;
  train         a training step of the main workload: the prefill keeping
                each token's denominator, then la_backward (dq, dk, dv) for a
                seeded dL/do; tokens/s of the forward+backward step, the
                backward kernels' times, and the dominant backward kernel
                against HBM peak (its algorithmic bytes: q, k, v, o, dL/do
                and the denominators read once, its gradients written once);
  train_gla     the same training step with GLA's per-channel decay (the
                B=4 H=16 N=4096 d=64 workload with alpha), dalpha included;
  train_delta   a training step of the gated delta-rule workload: the
                prefill, then la_delta_backward (dq, dk, dv, dg) for a
                seeded dL/do, with the backward kernels' times and the
                dominant one against HBM peak;
  cpu_baseline  the fp64 oracle on the host cores for the main workload and
                (in `decode` and `workloads`) the decode loop, the
                long-context prefill and the gated delta prefill: a
                process pool over (b, h) shards with one BLAS thread each,
                on a bounded sample of each workload (same shapes, recipe
                and seeds, drawn on the CPU generator), run in a child
                process before this one touches the GPU; a reported
                baseline, not a target (parity is the tests' job).
--gpus N with N > 1 exits with a message: the benchmark runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
METRIC = "prefill tokens/sec + % bf16 MFMA peak; decode state GB/s vs HBM peak"
LINEAR_CHUNK = 64              # chunk length of the bf16 prefill kernels
DELTA_CHUNK = 64


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2, choices=[2, 3, 4, 5, 6, 7, 8],
                    help="3 runs the decode-step loop alone")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-train", action="store_true")
    ap.add_argument("--no-train-gla", action="store_true",
                    help="skip the training step with GLA's per-channel decay")
    ap.add_argument("--no-train-delta", action="store_true",
                    help="skip only the gated-delta training leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB five "
                         "times (a calibration point for hardware byte counters)")
    ap.add_argument("--pmc-summary", metavar="DIR", default=None,
                    help="only summarise rocprofv3 FETCH_SIZE / WRITE_SIZE runs "
                         "kept under DIR/{fetch,write,copy_fetch,copy_write} for "
                         "--workload as markdown (no GPU needed)")
    ap.add_argument("--cpu-baseline-child", metavar="WIDS", default=None,
                    help=argparse.SUPPRESS)  # internal: the CPU baseline's child process
    ap.add_argument("--sq-summary", metavar="DIR", default=None,
                    help="condense rocprofv3 --pmc passes (pass1.. under DIR) of the "
                         "shader / address-unit counter groups for --workload")
    ap.add_argument("--stats-summary", metavar="DIR", default=None,
                    help="only summarise a rocprofv3 --kernel-trace --stats run "
                         "kept under DIR as markdown (no GPU needed)")
    return ap.parse_args()


def copy_probe(torch, mib):
    """Five device copies of MIB MiB (runtime blit kernel) and five
    elementwise passes b = a * 1 (16-byte vector loads and stores): each
    reads and writes exactly MIB MiB, a known size for scaling counters."""
    n = mib * 1024 * 1024 // 4
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    for _ in range(5):
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n * 4, "copies": 5}), flush=True)


# ---------------------------------------------------------------------------
# Hardware byte counters.  rocprofv3 runs of this script under
# --pmc FETCH_SIZE and --pmc WRITE_SIZE (KiB per dispatch), one counter per
# run, plus the same two counters over --copy-probe, are condensed by
# --pmc-summary into a markdown table whose last lines are machine-readable
# records.  A record is tied to a hash of the kernel's source files; the
# benchmark reports a kernel's traffic only while that hash still matches.

CSRC = os.path.join(ROOT, "causal_linear_attention_attn_amd", "csrc")
_DELTA_SRC = ("la_prefill_delta.hip", "la_delta_common.hpp")
_DELTA_BWD_SRC = ("la_backward_delta.hip", "la_delta_common.hpp")
KERNEL_SRC = {
    "linear_chunk": ("la_prefill_linear.hip",), "linear_summary": ("la_prefill_linear.hip",),
    "linear_scan": ("la_prefill_linear.hip",), "delta_prep": _DELTA_SRC,
    "delta_seq": _DELTA_SRC, "linear_decode": ("la_decode.hip",),
    "delta_bwd_prep": _DELTA_BWD_SRC, "delta_bwd_state": _DELTA_BWD_SRC,
    "delta_bwd_rev": _DELTA_BWD_SRC, "delta_bwd_grad": _DELTA_BWD_SRC,
    "delta_decode": ("la_decode.hip",), "linear_bwd_dq": ("la_backward_linear.hip",),
    "linear_bwd_dkv": ("la_backward_linear.hip",), "linear_bwd_rscan": ("la_backward_linear.hip",),
    "conv_qkv": ("la_conv.hip",), "conv_cache": ("la_conv.hip",), "conv_dx": ("la_conv.hip",),
    "conv_dw": ("la_conv.hip",), "conv_dw_reduce": ("la_conv.hip",),
}
PROFILES = os.path.join(ROOT, "profiles")
COPY_PROBE_MIB = 256


def kernel_src_hash(kname):
    import hashlib

    h = hashlib.sha256()
    for f in (*KERNEL_SRC[kname], "la_common.hpp", "la_internal.hpp"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def library_kernel_name(raw):
    """Name the library's own timer uses for a rocprofv3 kernel name
    (mangled or demangled), or None for kernels that are not ours."""
    if "la" not in raw:
        return None
    if "bwd_rscan_kernel" in raw:
        return "linear_bwd_rscan"
    if "bwd_dq_kernel" in raw or "bwd_dq_ch_kernel" in raw:
        return "linear_bwd_dq"
    if "bwd_dkv_kernel" in raw or "bwd_dkv_ch_kernel" in raw:
        return "linear_bwd_dkv"
    if "prep_kernel" in raw:  # its last template flag: the backward's records
        import re

        m = re.search(r"Lb([01])ELb([01])ELb([01])EEEv", raw) or \
            re.search(r", (true|false), (true|false), (true|false)>", raw)
        bwd = m is not None and m.group(3) in ("1", "true")
        return "delta_bwd_prep" if bwd else "delta_prep"
    for fn, name in (("chunk_kernel", "linear_chunk"), ("summary_kernel", "linear_summary"),
                     ("scan_kernel", "linear_scan"), ("seq_kernel", "delta_seq"),
                     ("seq2_kernel", "delta_seq"), ("bstate_kernel", "delta_bwd_state"),
                     ("brev_kernel", "delta_bwd_rev"), ("bgrad_kernel", "delta_bwd_grad"),
                     ("conv_qkv_kernel", "conv_qkv"), ("conv_cache_kernel", "conv_cache"),
                     ("conv_dx_kernel", "conv_dx"), ("conv_dw_partial_kernel", "conv_dw"),
                     ("conv_dw_reduce_kernel", "conv_dw_reduce")):
        if fn in raw:
            return name
    if "decode_kernel" in raw:  # template flags <T, VEC, DELTA, CV>
        import re

        m = re.search(r"Lb([01])ELb([01])EEEv", raw) or \
            re.search(r", (true|false), (true|false)>", raw)
        delta = m is not None and m.group(1) in ("1", "true")
        return "delta_decode" if delta else "linear_decode"
    return None


def _counter_rows(path):
    import csv
    import glob

    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {path}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _per_dispatch(rows, counter, keyfn):
    """Average KiB per dispatch of COUNTER for each key."""
    tot, disp = {}, {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        k = keyfn(r["Kernel_Name"])
        if k is None:
            continue
        tot[k] = tot.get(k, 0.0) + float(r["Counter_Value"])
        disp.setdefault(k, set()).add(r["Dispatch_Id"])
    return {k: (tot[k] / len(disp[k]), len(disp[k])) for k in tot}


def pmc_commands(d, wid):
    run = f"python3 bench.py {bench_args_for_counters(wid)}"
    cp = f"python3 bench.py --copy-probe {COPY_PROBE_MIB}"
    return [
        f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/fetch -o fetch -- {run}",
        f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/write -o write -- {run}",
        f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/copy_fetch -o cf -- {cp}",
        f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/copy_write -o cw -- {cp}",
        f"python3 bench.py --pmc-summary {d} --workload {wid}",
    ]


def bench_args_for_counters(wid):
    """The bench.py run a workload's counters come from: its own kernels only
    (the main workload with its training step, the gated-delta workloads
    with theirs)."""
    if wid == 3:
        return "--workload 3 --decode-steps 16 --no-cpu-baseline"
    own = {2: " --no-train-delta --no-train-gla", 5: "", 7: " --no-train-delta"}.get(
        wid, " --no-train")
    return (f"--workload {wid} --steps 5 --warmup 2 --no-decode --no-extra --no-cpu-baseline"
            + own)


def pmc_summary(d, wid):
    """Markdown table of HBM bytes per dispatch for the library's kernels of
    one workload, scaled by the counters' reading of a copy of known size."""
    from causal_linear_attention_attn_amd import inputs

    w = inputs.WORKLOADS[wid]
    probe = COPY_PROBE_MIB * 1024.0  # KiB read and written by each copy

    def copy_key(raw):
        if "copyBuffer" in raw:
            return "blit copy"
        if "MulFunctor" in raw:
            return "elementwise b = a * 1"
        return None

    cf = _per_dispatch(_counter_rows(os.path.join(d, "copy_fetch")), "FETCH_SIZE", copy_key)
    cw = _per_dispatch(_counter_rows(os.path.join(d, "copy_write")), "WRITE_SIZE", copy_key)
    ref = "elementwise b = a * 1" if "elementwise b = a * 1" in cf else "blit copy"
    f_fac, w_fac = probe / cf[ref][0], probe / cw[ref][0]
    kf = _per_dispatch(_counter_rows(os.path.join(d, "fetch")), "FETCH_SIZE",
                       library_kernel_name)
    kw = _per_dispatch(_counter_rows(os.path.join(d, "write")), "WRITE_SIZE",
                       library_kernel_name)
    alg = None
    if wid != 3:
        alg = w.B * w.H * w.N * bytes_per_head_token(w)
    out = [f"# HBM traffic per dispatch: {w.name}", "",
           "Commands (repository root, TMPDIR=/tmp, one counter per run):", ""]
    out += ["    " + c for c in pmc_commands(d, wid)]
    out += ["", f"Calibration: each probe copy reads and writes {COPY_PROBE_MIB} MiB "
            f"({probe:.0f} KiB).", "",
            "| probe kernel | FETCH_SIZE KiB | WRITE_SIZE KiB |", "|---|---|---|"]
    for k in sorted(cf):
        out.append(f"| {k} | {cf[k][0]:.0f} | {cw.get(k, (float('nan'),))[0]:.0f} |")
    out += ["", f"Scale factors (from the {ref} probe): FETCH_SIZE x {f_fac:.3f}, "
            f"WRITE_SIZE x {w_fac:.3f}.", "",
            "| kernel | dispatches | FETCH KiB | WRITE KiB | scaled read MB | "
            "scaled write MB | scaled total MB | algorithmic MB |",
            "|---|---|---|---|---|---|---|---|"]
    recs = []
    for k in sorted(kf):
        fk, n = kf[k]
        wk = kw.get(k, (float("nan"), 0))[0]
        rd, wr = fk * 1024 * f_fac, wk * 1024 * w_fac
        a = alg if k in ("linear_chunk", "delta_seq") else None
        if wid == 3 and k == "linear_decode":
            a = decode_step_bytes(w)
        if k in ("linear_bwd_dq", "linear_bwd_dkv"):
            a = w.B * w.H * w.N * bwd_bytes_per_head_token(w, k)
        if k.startswith("delta_bwd_"):
            a = w.B * w.H * w.N * delta_bwd_bytes_per_head_token(w, k)
        out.append(f"| {k} | {n} | {fk:.0f} | {wk:.0f} | {rd / 1e6:.1f} | {wr / 1e6:.1f} | "
                   f"{(rd + wr) / 1e6:.1f} | {'' if a is None else f'{a / 1e6:.1f}'} |")
        recs.append({"workload": w.name, "kernel": k, "src": kernel_src_hash(k),
                     "read_bytes": rd, "write_bytes": wr, "traffic_bytes": rd + wr})
    out += ["", "Machine-readable records (bench.py reports `traffic` from these while "
            "the kernel source hash matches):", ""]
    out += [f"<!-- traffic {json.dumps(r)} -->" for r in recs]
    print("\n".join(out))


SQ_PASSES = (
    "SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_INSTS_VALU SQ_INSTS_LDS SQ_INSTS_MFMA "
    "SQ_INSTS_SALU SQ_INSTS_VMEM GRBM_GUI_ACTIVE",
    "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_ANY SQ_WAIT_INST_LDS SQ_WAIT_ANY "
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE",
    "TA_TA_BUSY_sum TA_BUFFER_READ_WAVEFRONTS_sum TCP_TOTAL_CACHE_ACCESSES_sum "
    "TCP_TCC_READ_REQ_sum TCC_HIT_sum TCC_MISS_sum GRBM_GUI_ACTIVE",
)
SIMDS = 1024  # 256 CUs x 4 SIMDs
XCDS = 8


def sq_summary(d, wid):
    """Markdown table of shader, address-unit and L2 counters per dispatch
    for the library's kernels of one workload (one rocprofv3 --pmc pass per
    group of counters, in subdirectories pass1.. of D), with the derived
    fractions and source-hash records."""
    from causal_linear_attention_attn_amd import inputs

    w = inputs.WORKLOADS[wid]
    seen = {}  # (kernel, counter) -> per-dispatch averages of the passes holding it
    for i in range(1, len(SQ_PASSES) + 1):
        sub = os.path.join(d, f"pass{i}")
        if not os.path.isdir(sub):
            continue
        rows = _counter_rows(sub)
        for c in sorted({r["Counter_Name"] for r in rows}):
            for k, (v, _) in _per_dispatch(rows, c, library_kernel_name).items():
                seen.setdefault((k, c), []).append(v)
    names = sorted({c for _, c in seen})
    vals = {}
    for (k, c), v in seen.items():
        vals.setdefault(k, {})[c] = sum(v) / len(v)
    kernels = sorted(vals)
    run = f"python3 bench.py {bench_args_for_counters(wid)}"
    out = [f"# Shader and memory-unit counters per dispatch: {w.name}", "",
           "Commands (repository root, TMPDIR=/tmp, one pass per counter group):", ""]
    for i, ctr in enumerate(SQ_PASSES, 1):
        out.append(f"    rocprofv3 --pmc {ctr} --output-format csv -d {d}/pass{i} -o sq -- {run}")
    out += [f"    python3 bench.py --sq-summary {d} --workload {wid}", "",
            "| counter | " + " | ".join(kernels) + " |", "|---|" + "---|" * len(kernels)]
    for c in names:
        out.append(f"| {c} | " + " | ".join(f"{vals[k].get(c, float('nan')):.0f}"
                                            for k in kernels) + " |")
    out += ["", "Derived (GRBM_GUI_ACTIVE is summed over the 8 XCDs; SQ counters over all "
            f"{SIMDS} SIMDs):", ""]
    recs = []
    for k in kernels:
        v = vals[k]
        cyc = v.get("GRBM_GUI_ACTIVE", 0.0) / XCDS
        parts = []
        if cyc and "SQ_VALU_MFMA_BUSY_CYCLES" in v:
            parts.append(f"matrix-core busy {v['SQ_VALU_MFMA_BUSY_CYCLES'] / SIMDS / cyc:.1%} "
                         "of the kernel's cycles per SIMD")
        if "SQ_LDS_BANK_CONFLICT" in v and v.get("SQ_LDS_IDX_ACTIVE"):
            parts.append(f"LDS bank-conflict cycles {v['SQ_LDS_BANK_CONFLICT'] / v['SQ_LDS_IDX_ACTIVE']:.0%}"
                         " of LDS-busy cycles")
        if v.get("SQ_WAVE_CYCLES"):
            wc = v["SQ_WAVE_CYCLES"]
            if "SQ_WAIT_ANY" in v:
                parts.append(f"waves waiting {v['SQ_WAIT_ANY'] / wc:.0%}")
            if "SQ_ACTIVE_INST_ANY" in v:
                parts.append(f"issuing {v['SQ_ACTIVE_INST_ANY'] / wc:.0%}")
            if "SQ_ACTIVE_INST_VALU" in v:
                parts.append(f"VALU {v['SQ_ACTIVE_INST_VALU'] / wc:.0%} of wave cycles")
        if cyc and "TA_TA_BUSY_sum" in v:
            parts.append(f"address units busy {v['TA_TA_BUSY_sum'] / 256 / cyc:.0%} of the "
                         "kernel's cycles per CU")
        if v.get("TCC_HIT_sum") is not None and v.get("TCC_MISS_sum") is not None:
            tot = v["TCC_HIT_sum"] + v["TCC_MISS_sum"]
            if tot:
                parts.append(f"L2 hit rate {v['TCC_HIT_sum'] / tot:.0%}")
        if parts:
            out.append(f"- {k}: " + "; ".join(parts) + ".")
        recs.append({"workload": w.name, "kernel": k, "src": kernel_src_hash(k),
                     "counters": {c: v[c] for c in sorted(v)}})
    out += ["", "Machine-readable records (per dispatch, with the kernel source hash):", ""]
    out += [f"<!-- counters {json.dumps(r)} -->" for r in recs]
    print("\n".join(out))


def stats_summary(d):
    """Markdown table of the library's kernels from a rocprofv3 --stats run."""
    import csv
    import glob

    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    out = ["| kernel (library name) | rocprofv3 name | calls | average us | min us | "
           "max us |", "|---|---|---|---|---|---|"]
    with open(files[0], newline="") as fh:
        for r in csv.DictReader(fh):
            k = library_kernel_name(r["Name"])
            if k is None:
                continue
            out.append(f"| {k} | `{r['Name'][:90]}` | {r['Calls']} | "
                       f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                       f"{float(r['MaxNs']) / 1e3:.2f} |")
    print("\n".join(out))


def traffic_record(wname, kname):
    """HBM bytes per launch for KNAME on workload WNAME from the committed
    counter summaries, or None when there is none for the current source."""
    import glob

    want = kernel_src_hash(kname)
    for f in sorted(glob.glob(os.path.join(PROFILES, "*.md"))):
        with open(f) as fh:
            for line in fh:
                if not line.startswith("<!-- traffic "):
                    continue
                r = json.loads(line[len("<!-- traffic "):line.rindex("-->")])
                if r["workload"] == wname and r["kernel"] == kname and r["src"] == want:
                    return r["traffic_bytes"], os.path.basename(f)
    return None, None


class KernelTimer:
    """Kernel durations from the HIP events the library hands to each of its
    dispatches (start and end of the kernel itself)."""

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


def bytes_per_head_token(w):
    """Algorithmic HBM bytes: q, k, v read once, o written once (plus the
    fp32 gate, and the fp32 decay when given, for the delta rule)."""
    e = w.dtype.itemsize
    b = (2 * w.d + w.dv) * e + w.dv * e
    if w.rule == "delta":
        b += 4 + (4 if w.decay == "alpha" else 0)
    elif w.decay == "channel":
        b += 4 * w.d  # fp32 decay per key channel
    return b


def flops_per_head_token(w):
    """Matrix flops of the chunk form per head-token, as the workload
    table counts them.  LINEAR (chunk C): state read 2 d dv, state update
    2 d dv, scores and weighted sum 2 C (d + dv).  DELTA (chunk C): the
    three state products (K S, Q S, the update) 6 d dv, the chunk-local
    products 2 C (3 d + 2 dv) and the triangular inverse C^2 / 3 (full
    tiles counted: 181 589 at d = dv = 128, C = 64)."""
    d, dv = w.d, w.dv
    if w.rule == "linear":
        C = LINEAR_CHUNK
        return 4 * d * dv + 2 * C * (d + dv)
    C = DELTA_CHUNK
    return 6 * d * dv + 2 * C * (3 * d + 2 * dv) + (C * C) // 3


def make_step(la, torch, w, x):
    B, H, N, d, dv = w.B, w.H, w.N, w.d, w.dv
    q, k, v, gamma = x["q"], x["k"], x["v"], x["gamma"]
    o = torch.empty((B, H, N, dv), dtype=w.dtype, device="cuda")
    S = torch.empty((B, H, d, dv), dtype=torch.float32, device="cuda")
    if w.rule == "delta":
        g, al = x["g"], x.get("alpha")
        ws_bytes = la.workspace_size(q, k, v, rule="delta", g=g)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

        def step():
            la.prefill(q, k, v, rule="delta", g=g, alpha=al, o=o, S_out=S, workspace=ws)
    else:
        z = torch.empty((B, H, d), dtype=torch.float32, device="cuda")
        al = x.get("alpha")
        cw, cin = x.get("conv_weight"), x.get("conv_cache")
        cout = None if cin is None else torch.empty_like(cin)
        ws_bytes = la.workspace_size(q, k, v, gamma=gamma, eps=w.eps, alpha=al,
                                     conv_weight=cw)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

        def step():
            la.prefill(q, k, v, gamma=gamma, alpha=al, eps=w.eps, o=o, S_out=S, z_out=z,
                       workspace=ws, conv_weight=cw, conv_cache=cin, conv_cache_out=cout)
    return step, o, ws_bytes


def time_kernels(lib, torch, step, reps):
    with KernelTimer(lib) as kt:
        for _ in range(reps):
            step()
        torch.cuda.synchronize()
        times = kt.collect()
    return {n: sum(v) / len(v) for n, v in times.items()}


GRAPH_STEPS = 8  # consecutive steps per captured HIP graph


def _capture(torch, step, n):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            step()
    return g


def time_graph(torch, step, steps, warmup, latency=False):
    """Wall time per step over exactly `steps` steps, replayed from HIP graphs
    that each hold up to GRAPH_STEPS consecutive steps (issued back to back
    on one stream, as a serving or training loop issues them; the host-side
    launch of a graph is then paid once per GRAPH_STEPS steps).  With
    latency=True also the wall time of one step alone (a one-step graph,
    replayed `steps` times), returned second."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    n = max(1, min(GRAPH_STEPS, steps))
    g = _capture(torch, step, n)
    rem = steps % n
    g_rem = _capture(torch, step, rem) if rem else None
    for _ in range(max(1, warmup // n)):
        g.replay()
    if g_rem is not None:  # a graph's first replay also uploads it
        g_rem.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps // n):
        g.replay()
    if g_rem is not None:
        g_rem.replay()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    if not latency:
        return dt
    g1 = _capture(torch, step, 1)
    for _ in range(warmup):
        g1.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g1.replay()
    torch.cuda.synchronize()
    return dt, (time.perf_counter() - t0) / steps


def dominant(kern):
    return max(kern.items(), key=lambda kv: kv[1])


def prefill_summary(w, kern, dt):
    """Per-workload figures: throughput, the dominant kernel against HBM and
    matrix peaks, and the whole step against HBM peak."""
    head_tokens = w.B * w.H * w.N
    bpl = head_tokens * bytes_per_head_token(w)
    fpl = head_tokens * flops_per_head_token(w)
    kname, kms = dominant(kern)
    achieved = bpl / (kms * 1e-3) / 1e9
    tflops = fpl / (kms * 1e-3) / 1e12
    traffic, tsrc = traffic_record(w.name, kname)
    return {
        "tokens_per_s": w.B * w.N / dt, "ms_per_step": dt * 1e3,
        "kernels_ms": kern,
        "roofline": {"kernel": kname, "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "traffic_profile": tsrc, "bytes_per_launch": bpl,
                     "kernel_ms": kms},
        "mfma": {"kernel": kname, "flops_per_launch": fpl,
                 "achieved_tflops": tflops, "peak_tflops": BF16_PEAK_TFLOPS,
                 "frac": tflops / BF16_PEAK_TFLOPS},
        "step_hbm_frac": bpl / dt / 1e9 / HBM_PEAK_GBS,
    }


def bench_workload(la, lib, torch, w, steps, warmup):
    from causal_linear_attention_attn_amd import inputs

    x = inputs.make_prefill(w, "cuda")
    step, o, ws_bytes = make_step(la, torch, w, x)
    for _ in range(max(1, warmup // 4)):
        step()
    torch.cuda.synchronize()
    kern = time_kernels(lib, torch, step, max(3, steps // 4))
    dt, lat = time_graph(torch, step, steps, warmup, latency=True)
    out = prefill_summary(w, kern, dt)
    out["ms_one_step_alone"] = lat * 1e3
    out["workload"] = w.name
    out["workspace_bytes"] = ws_bytes
    return out, x, o


def bwd_bytes_per_head_token(w, kname):
    """Algorithmic bytes of one backward kernel per head-token: q, k, v, o,
    dL/do and den read once; its gradients written once (with GLA's
    per-channel decay also alpha read, and dalpha written by dk/dv; fp32)."""
    e = w.dtype.itemsize
    rd = (2 * w.d + 3 * w.dv) * e + 4
    b = rd + (w.d * e if kname == "linear_bwd_dq" else (w.d + w.dv) * e)
    if w.decay == "channel":
        b += 4 * w.d * (1 if kname == "linear_bwd_dq" else 2)
    return b


def bench_train(la, lib, torch, w, steps, warmup):
    """Training step of the main workload: prefill keeping the per-token
    denominators, then the backward (dq, dk, dv) for a seeded dL/do."""
    from causal_linear_attention_attn_amd import inputs

    x = inputs.make_prefill(w, "cuda")
    do = inputs.make_grad_out(w, "cuda")
    q, k, v, gamma, al = x["q"], x["k"], x["v"], x["gamma"], x.get("alpha")
    B, H, N, d, dv = w.B, w.H, w.N, w.d, w.dv
    o = torch.empty((B, H, N, dv), dtype=w.dtype, device="cuda")
    den = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    wsf = torch.empty(max(la.workspace_size(q, k, v, gamma=gamma, alpha=al, eps=w.eps,
                                            den_out=den), 1),
                      dtype=torch.uint8, device="cuda")

    def fwd():
        la.prefill(q, k, v, gamma=gamma, alpha=al, eps=w.eps, o=o, den_out=den, workspace=wsf,
                   return_state=False)

    def bwd():  # the forward's segment states are reused from its workspace
        return la.backward(q, k, v, o, den, do, gamma=gamma, alpha=al, state_grad=False,
                           fwd_workspace=wsf)

    def step():
        fwd()
        bwd()

    for _ in range(max(1, warmup // 4)):
        step()
    torch.cuda.synchronize()
    kern = time_kernels(lib, torch, bwd, max(3, steps // 4))
    dt = time_graph(torch, step, steps, warmup)
    head_tokens = B * H * N
    bk = {n: t for n, t in kern.items() if n.startswith("linear_bwd")}
    kname, kms = dominant(bk)
    bpl = head_tokens * bwd_bytes_per_head_token(w, kname)
    achieved = bpl / (kms * 1e-3) / 1e9
    traffic, tsrc = traffic_record(w.name, kname)
    return {
        "workload": w.name + "_forward_backward", "tokens_per_s": B * N / dt,
        "ms_per_step": dt * 1e3, "backward_kernels_ms": kern,
        "backward_ms": sum(kern.values()),
        "roofline": {"kernel": kname, "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "traffic_profile": tsrc, "bytes_per_launch": bpl,
                     "kernel_ms": kms},
    }


def delta_bwd_bytes_per_head_token(w, kname):
    """Algorithmic bytes of one delta-rule backward kernel per head-token:
    the inputs and gradients it reads or writes (q, k, v, dL/do rows, the
    gate and decay; workspace records excluded)."""
    e, d, dv = w.dtype.itemsize, w.d, w.dv
    gd = 4 + (4 if w.decay == "alpha" else 0)  # g (and alpha), fp32
    return {"delta_bwd_prep": 2 * d * e + gd,
            "delta_bwd_state": (d + dv) * e,
            "delta_bwd_rev": (2 * d + dv) * e + dv * e,
            "delta_bwd_grad": (2 * d + 2 * dv) * e + gd + 2 * d * e + gd}[kname]


def delta_train_bytes_per_head_token(w):
    """The training step's algorithmic bytes: the forward's (q, k, v, g, alpha
    read, o written) and the backward's (q, k, v, g, alpha, dL/do read; dq,
    dk, dv, dg, dalpha written)."""
    e, d, dv = w.dtype.itemsize, w.d, w.dv
    gd = 4 + (4 if w.decay == "alpha" else 0)
    return bytes_per_head_token(w) + (2 * d + 2 * dv) * e + gd + (2 * d + dv) * e + gd


def bench_train_delta(la, lib, torch, w, steps, warmup):
    """Training step of a gated-delta workload: the prefill, then
    la_delta_backward for a seeded dL/do."""
    from causal_linear_attention_attn_amd import inputs

    x = inputs.make_prefill(w, "cuda")
    do = inputs.make_grad_out(w, "cuda")
    q, k, v, g, al = x["q"], x["k"], x["v"], x["g"], x.get("alpha")
    o = torch.empty((w.B, w.H, w.N, w.dv), dtype=w.dtype, device="cuda")
    wsf = torch.empty(max(la.workspace_size(q, k, v, rule="delta", g=g), 1), dtype=torch.uint8,
                      device="cuda")
    wsb = torch.empty(max(la.delta_backward_workspace_size(q, k, v), 1), dtype=torch.uint8,
                      device="cuda")

    def fwd():
        la.prefill(q, k, v, rule="delta", g=g, alpha=al, o=o, workspace=wsf, return_state=False)

    def bwd():
        return la.delta_backward(q, k, v, g, do, alpha=al, state_grad=False, workspace=wsb)

    def step():
        fwd()
        bwd()

    for _ in range(max(1, warmup // 4)):
        step()
    torch.cuda.synchronize()
    kern = time_kernels(lib, torch, bwd, max(3, steps // 4))
    dt = time_graph(torch, step, steps, warmup)
    head_tokens = w.B * w.H * w.N
    kname, kms = dominant(kern)
    bpl = head_tokens * delta_bwd_bytes_per_head_token(w, kname)
    achieved = bpl / (kms * 1e-3) / 1e9
    traffic, tsrc = traffic_record(w.name, kname)
    step_bytes = head_tokens * delta_train_bytes_per_head_token(w)
    return {
        "workload": w.name + "_forward_backward", "tokens_per_s": w.B * w.N / dt,
        "ms_per_step": dt * 1e3, "backward_kernels_ms": kern,
        "backward_ms": sum(kern.values()),
        "step_hbm_frac": step_bytes / dt / 1e9 / HBM_PEAK_GBS,
        "roofline": {"kernel": kname, "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "traffic_profile": tsrc, "bytes_per_launch": bpl,
                     "kernel_ms": kms},
    }


def decode_step_bytes(w):
    """Algorithmic bytes of one decode step: state S and z read and written
    once; q, k, v read and o written once."""
    e = w.dtype.itemsize
    nbh = w.B * w.H
    return 2 * nbh * (w.d * w.dv + w.d) * 4 + nbh * (2 * w.d + 2 * w.dv) * e


def bench_decode(la, lib, torch, nsteps, warmup=8):
    from causal_linear_attention_attn_amd import inputs

    w = inputs.WORKLOADS[3]
    B, H, d, dv = w.B, w.H, w.d, w.dv
    x = inputs.make_prefill(w, "cuda")
    _, S, z = la.prefill(x["q"], x["k"], x["v"], eps=w.eps)
    del x
    dec = inputs.make_decode(w, "cuda", steps=nsteps)
    o = torch.empty((B, H, dv), dtype=w.dtype, device="cuda")
    S2, z2 = S.clone(), z.clone()  # warm-up steps on a scratch copy
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
    step_bytes = decode_step_bytes(w)
    dt = (t1 - t0) / nsteps
    traffic, tsrc = traffic_record(w.name, "linear_decode")
    return {
        "workload": w.name, "steps": nsteps,
        "steps_per_s": 1.0 / dt, "tokens_per_s": B / dt, "ms_per_step": dt * 1e3,
        "kernel_ms": kavg, "bytes_per_step": step_bytes,
        "roofline": {"kernel": "linear_decode", "bound": "hbm",
                     "achieved": step_bytes / (kavg * 1e-3) / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": step_bytes / (kavg * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "traffic": traffic, "traffic_profile": tsrc},
        "loop_GBs": step_bytes / dt / 1e9,
    }


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on the host cores, per workload, on a bounded
# sample of the workload (same shapes and input recipe).  It runs in a child
# process started before this process touches the GPU; the child never uses
# the GPU, so it can fork a pool of workers over (b, h) shards, each with one
# BLAS thread, that inherit the sample arrays.
CPU_MAX_WORKERS = 16  # the host's CPU share per GPU
CPU_BASELINE_WORKLOADS = (2, 3, 4, 5)
_CPU = {}             # the current sample (fp64, heads flattened to [1, BH, ...])


def _cpu_sample(w):
    """Fill _CPU with a bounded sample of workload w; returns (description,
    work units covered, unit name, units of the whole workload).  Inputs are
    drawn with the workload's recipe and seeds on the CPU generator."""
    import numpy as np

    from causal_linear_attention_attn_amd import inputs

    def flat(t):
        t = t.double().numpy()
        return t.reshape(1, t.shape[0] * t.shape[1], *t.shape[2:])

    _CPU.clear()
    _CPU["wid"] = w.wid
    if w.wid == 3:  # decode loop: 16 of the 256 sequences, all heads
        nb = 16
        x = inputs.make_prefill(w, "cpu", B=nb)
        dec = inputs.make_decode(w, "cpu", B=nb)
        for n in ("q", "k", "v"):
            _CPU[n] = flat(x[n])
            d = dec[n].double().numpy()  # [steps, B, H, dim]
            _CPU["dec_" + n] = d.reshape(d.shape[0], 1, nb * w.H, d.shape[-1])
        heads = nb * w.H
        desc = (f"{nb} of {w.B} sequences x {w.H} heads ({heads} of {w.B * w.H} states): "
                f"the {w.N}-token prefill recurrence, its check against the closed form "
                f"phi(K)^T V, sum phi(k) (gamma = 1), then {w.decode_steps} decode steps")
        return desc, heads, "head-states", w.B * w.H
    N = 16384 if w.wid == 4 else w.N  # the long-context workload: its first 16384 tokens
    x = inputs.make_prefill(w, "cpu", N=N)
    for n in ("q", "k", "v", "g", "alpha"):
        if x.get(n) is not None:
            _CPU[n] = flat(x[n])
    if x.get("gamma") is not None:
        _CPU["gamma"] = np.tile(x["gamma"].double().numpy(), w.B)
    heads = w.B * w.H
    desc = f"all {heads} heads x {N} of {w.N} tokens" if N < w.N else \
        f"the whole workload ({heads} heads x {N} tokens)"
    return desc, heads * N, "head-tokens", w.B * w.H * w.N


def _cpu_shard(job):
    """Oracle over heads [lo, hi) of the current sample, one BLAS thread.
    Returns (seconds, largest closed-form error of the decode prefill)."""
    lo, hi = job
    from threadpoolctl import threadpool_limits

    import numpy as np

    import oracle

    x = _CPU
    sl = lambda n: x[n][:, lo:hi]  # noqa: E731
    err = 0.0
    with threadpool_limits(1):
        t0 = time.perf_counter()
        if x["wid"] == 3:
            q, k, v = sl("q"), sl("k"), sl("v")
            _, S, z = oracle.linear_prefill(q, k, v, eps=1e-6)
            fk = oracle.phi_elu1(k)
            S_cf = np.einsum("bhnr,bhnd->bhrd", fk, v)
            err = max(float(np.abs(S - S_cf).max() / np.abs(S_cf).max()),
                      float(np.abs(z - fk.sum(2)).max() / np.abs(fk.sum(2)).max()))
            t0 = time.perf_counter()  # the decode steps alone are the measured unit
            for t in range(x["dec_q"].shape[0]):
                _, S, z = oracle.linear_decode_step(x["dec_q"][t][:, lo:hi],
                                                    x["dec_k"][t][:, lo:hi],
                                                    x["dec_v"][t][:, lo:hi], S, z, eps=1e-6)
        elif "g" in x:
            oracle.delta_prefill(sl("q"), sl("k"), sl("v"), sl("g"),
                                 alpha=sl("alpha") if "alpha" in x else None)
        else:
            gamma = x["gamma"][lo:hi] if "gamma" in x else None
            oracle.linear_prefill(sl("q"), sl("k"), sl("v"), gamma=gamma, eps=1e-6)
        return time.perf_counter() - t0, err


def _cpu_ready(_):
    return os.getpid()


def cpu_baseline_child(wids):
    """Runs in the child: the oracle over a bounded sample of each workload
    in a fork pool; prints one JSON dict {workload name: cpu_baseline}."""
    import multiprocessing as mp

    import numpy as np
    import torch

    from causal_linear_attention_attn_amd import inputs

    torch.set_num_threads(1)
    cores = min(len(os.sched_getaffinity(0)), CPU_MAX_WORKERS)
    res = {}
    for wid in wids:
        w = inputs.WORKLOADS[wid]
        desc, units, uname, total = _cpu_sample(w)
        nheads = _CPU["q"].shape[1]
        nw = min(cores, nheads)
        bounds = np.linspace(0, nheads, nw + 1).astype(int)
        with mp.get_context("fork").Pool(nw) as pool:
            pool.map(_cpu_ready, range(nw))
            t0 = time.perf_counter()
            out = pool.map(_cpu_shard, list(zip(bounds[:-1].tolist(), bounds[1:].tolist())))
            wall = time.perf_counter() - t0
        r = {"kind": "oracle", "cores": nw, "wall_s": wall,
             "sample": f"{desc}; {nw} worker processes over (b,h) shards, one BLAS thread "
                       f"each, on {len(os.sched_getaffinity(0))} host cores"}
        if wid == 3:  # decode steps of the whole batch per second (the decode
            # loops alone: the slowest worker's)
            dt = max(t for t, _ in out)
            r.update(value=w.decode_steps * units / total / dt, unit="steps/s",
                     decode_s=dt, closed_form_rel_err=max(e for _, e in out))
        else:
            r.update(value=units // w.H / wall, unit="tokens/s")  # B * N tokens
        res[w.name] = r
    print(json.dumps(res), flush=True)


def run_cpu_baseline(wids):
    """The CPU baseline of workloads `wids` from a child process (call before
    anything touches the GPU); {workload name: record}."""
    import subprocess

    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-child",
                        ",".join(str(i) for i in wids)], capture_output=True, text=True,
                       timeout=900)
    if r.returncode != 0:
        raise RuntimeError(f"cpu baseline child failed:\n{r.stderr[-2000:]}")
    return json.loads(r.stdout.strip().splitlines()[-1])


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "heads shard across GPUs with no communication, so each GPU "
              "would run this same single-GPU step on its share.", file=sys.stderr)
        sys.exit(2)
    if args.pmc_summary:
        pmc_summary(args.pmc_summary, args.workload)
        return
    if args.stats_summary:
        stats_summary(args.stats_summary)
        return
    if args.sq_summary:
        sq_summary(args.sq_summary, args.workload)
        return
    if args.cpu_baseline_child:
        cpu_baseline_child([int(i) for i in args.cpu_baseline_child.split(",")])
        return
    # the CPU baseline runs first, in a child process, before this process
    # touches the GPU (rank 0 at N = 1: the only rank here)
    cpu = None
    if not args.no_cpu_baseline and not args.copy_probe:
        wids = [args.workload]
        if args.workload != 3:
            if not args.no_decode:
                wids.append(3)
            if not args.no_extra:
                wids += [i for i in (4, 5) if i != args.workload]
        cpu = run_cpu_baseline([i for i in wids if i in CPU_BASELINE_WORKLOADS])
    import torch

    import causal_linear_attention_attn_amd as la
    from causal_linear_attention_attn_amd import _lib, inputs

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        copy_probe(torch, args.copy_probe)
        return
    lib = _lib.load()
    if args.workload == 3:
        dec = bench_decode(la, lib, torch, args.decode_steps)
        print(json.dumps({
            "metric": "decode state GB/s vs HBM peak", "value": dec["tokens_per_s"],
            "unit": "tokens/s", "n_gpus": 1, "steps": dec["steps"], "warmup": 8,
            "ms_per_step": dec["ms_per_step"], "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic (seeded normal draws; see inputs.py)",
            "config": {"workload": dec["workload"]}, "roofline": dec["roofline"],
            "decode": dec, "cpu_baseline": None if cpu is None else cpu.get(dec["workload"])}),
            flush=True)
        return
    w = inputs.WORKLOADS[args.workload]
    res, x, o = bench_workload(la, lib, torch, w, args.steps, args.warmup)
    line = {
        "metric": METRIC, "value": res["tokens_per_s"], "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"], "ms_one_step_alone": res["ms_one_step_alone"],
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
        "data": "synthetic (seeded normal draws; see inputs.py)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "dv": w.dv, "rule": w.rule, "fmap": w.fmap, "decay": w.decay,
                   "conv": w.conv, "eps": w.eps,
                   "head_tokens_per_step": w.B * w.H * w.N},
        "roofline": res["roofline"], "mfma": res["mfma"],
        "step_hbm_frac": res["step_hbm_frac"], "kernels_ms": res["kernels_ms"],
        "workspace_bytes": res["workspace_bytes"],
    }
    if cpu is not None:
        line["cpu_baseline"] = cpu[w.name]
    del x, o
    if not args.no_decode:
        line["decode"] = bench_decode(la, lib, torch, args.decode_steps)
        if cpu is not None:
            line["decode"]["cpu_baseline"] = cpu.get(line["decode"]["workload"])
    if not args.no_train and w.rule == "linear" and w.decay in ("none", "per_head") \
            and not w.conv:
        line["train"] = bench_train(la, lib, torch, w, max(10, args.steps // 4), 5)
    if not args.no_train and not args.no_train_gla and \
            (w.decay == "channel" or args.workload == 2):
        wg = w if w.decay == "channel" else inputs.WORKLOADS[7]
        line["train_gla"] = bench_train(la, lib, torch, wg, max(10, args.steps // 4), 5)
    if not args.no_train and not args.no_train_delta and \
            (w.rule == "delta" or args.workload == 2):
        wd = w if w.rule == "delta" else inputs.WORKLOADS[5]
        line["train_delta"] = bench_train_delta(la, lib, torch, wd, max(10, args.steps // 10), 3)
    if not args.no_extra:
        extra = {}
        for wid in (4, 5, 6, 7, 8):
            if wid == args.workload:
                continue
            r, xx, oo = bench_workload(la, lib, torch, inputs.WORKLOADS[wid],
                                       max(5, args.steps // 10), 3)
            del xx, oo
            name = r.pop("workload")
            if cpu is not None and name in cpu:
                r["cpu_baseline"] = cpu[name]
            extra[name] = r
        line["workloads"] = extra
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
