#!/usr/bin/env python3
"""Bench: cross-entropy forward+backward on MI355X through the C ABI.

`--workload flce_bf16_4096x6656x202048` benches the fused linear variant instead (one step =
one lce_flce_fwd_bwd call; value = 6 N H V flops per step over the step time, against the dense
bf16 MFMA peak).

One step = one lce_ce_fwd_bwd call (one persistent kernel launch: label count, per-token
loss, reduced loss, argmax/accuracy when the workload asks for it, gradient written in
place) over one batch of synthetic logits already resident in HBM.  The gradient
overwrites its input, so every step gets its own pristine copy, made before the timed
region (the pages' Megatron benchmark likewise clones its inputs outside timing).

Prints ONE JSON line.  `value` is algorithmic HBM throughput (2 N V b + 12 N bytes per
step over the measured step time); the default workload is bf16 [2048, 131072].
`roofline.traffic` comes from the committed rocprofv3 counter summary of the same
workload (profiles/) and is null when the kernel sources changed since it was taken.

`python bench.py --collect-profiles [--workload W]` runs rocprofv3 on this script as child
processes (kernel trace with stats, then FETCH_SIZE, then WRITE_SIZE) and writes the
summary to profiles/; that parent process never touches the GPU.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CE fwd+bwd ms and HBM GB/s (% peak), bf16 logits 2048×131072, 1 GPU"
HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak, published
FLCE_METRIC = "FLCE fwd+bwd ms and bf16 MFMA TFLOP/s (% peak), hidden 4096×6656, weight 202048×6656, 1 GPU"
RESIDENT_METRIC = ("tile-resident FLCE (logits never stored) fwd+bwd ms and bf16 MFMA TFLOP/s at 6·N·H·V "
                   "(% peak), hidden 4096×6656, weight 202048×6656, 1 GPU")
# The pages' CE fwd+bwd latencies for this shape (Megatron-LM PR "Add opt-in Liger vocab-parallel cross
# entropy", Performance (Liger v0.8.5), TP=1 row): another machine, context only, never the target.
H100_CONTEXT = {"hardware": "H100 80GB, BF16, [2048, 131072], TP=1", "liger_ms": 2.041,
                "megatron_native_fused_ms": 3.646, "transformer_engine_ms": 0.711}
CSRC = os.path.join(ROOT, "vocabulary_cross_entropy_row_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
# raw rocprofv3 output of --collect-profiles (CSV files; only the summaries go to profiles/)
RAW_PROFILES = os.environ.get("LCE_PROFILE_RAW_DIR", os.path.join(ROOT, "profiles_raw"))


def call_percentiles(ms, nd: int) -> dict:
    """Median and 10th / 90th percentiles of the per-call times (HIP events)."""
    import numpy as np
    return {"call_ms_median": round(float(np.median(ms)), nd), "call_ms_p10": round(float(np.percentile(ms, 10)), nd),
            "call_ms_p90": round(float(np.percentile(ms, 90)), nd)}


def algorithmic_bytes(w) -> int:
    # one read + one write of the logits, 8 B label read + 4 B loss write per token
    return 2 * w.n * w.V * w.elem_bytes + 12 * w.n


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: as many as 64 GB of pristine input copies hold, 20 to 100; "
                         "20 for the fused-linear workloads)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="ce_bf16_2048x131072")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--collect-profiles", action="store_true")
    ap.add_argument("--path", choices=["fused", "split", "resident"], default="fused",
                    help="split: stats / combine / gradient as separate calls over --tp vocabulary shards; "
                         "resident: the tile-resident fused linear forward + backward (fused-linear workloads)")
    ap.add_argument("--tp", type=int, default=1, help="vocabulary shards of the split path (one GPU)")
    ap.add_argument("--flce-workspace", choices=["default", "wt", "lean"], default="default",
                    help="fused linear workspace: the default layout (one grad_weight pass, grad_hidden reads W in "
                         "place), wt (also room for W^T), or lean (one chunk per grad_weight group)")
    ap.add_argument("--no-pages-protocol", action="store_true",
                    help="skip the extra per-call timing in the pages' protocol (10 warmups, 3 x 50 samples)")
    ap.add_argument("--no-event-pass", action="store_true",
                    help="(profiling runs) skip the event-timed calls of the CE path: the profiler times every "
                         "kernel itself, and the per-call figures are then the back-to-back steps' average")
    return ap.parse_args()


# ---------------------------------------------------------------- CPU baseline

def cpu_baseline(w, x, y, nthreads: int, min_seconds: float = 10.0) -> dict:
    """The oracle as it stands, on the host cores: whole passes over the workload (loss, argmax
    and fp64 gradient of every row, gradients produced in 256-row chunks) repeated until at
    least ``min_seconds`` have elapsed."""
    import numpy as np

    import oracle
    orc = oracle.default()
    chunk = 256
    passes = 0
    t0 = time.perf_counter()
    while True:
        for r0 in range(0, w.n, chunk):
            rows = np.arange(r0, min(w.n, r0 + chunk))
            orc.ce(x, y, V=w.V, label_smoothing=w.label_smoothing, softcap=w.softcap, reduction=w.reduction,
                   grad_out=[w.grad_out], rows=rows, want_grad=True, nthreads=nthreads)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": round(passes * algorithmic_bytes(w) / dt / 1e9, 4), "unit": "GB/s", "cores": nthreads,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"{passes} full passes over the workload ({w.n} rows x {w.V}): fp64 loss, argmax and "
                      f"gradient of every row, OpenMP over rows"}


def split_cpu_baseline(w, x, y, nbytes: int, nthreads: int, min_seconds: float = 10.0) -> dict:
    """The oracle as it stands on the split path's outputs: per 256-row chunk the fp64 loss and gradient
    (row routine) and log-sum-exp, log p_y and entropy (row statistics), repeated over the workload's rows
    until ``min_seconds`` have elapsed; the rate is scaled to the step's algorithmic bytes."""
    import numpy as np

    import oracle
    orc = oracle.default()
    chunk = 256
    rows_done = 0
    t0 = time.perf_counter()
    while True:
        for r0 in range(0, w.n, chunk):
            rows = np.arange(r0, min(w.n, r0 + chunk))
            orc.ce(x, y, V=w.V, label_smoothing=w.label_smoothing, softcap=w.softcap, reduction=w.reduction,
                   grad_out=[w.grad_out], rows=rows, want_grad=True, nthreads=nthreads)
            orc.row_stats(x, y, V=w.V, softcap=w.softcap, rows=rows, nthreads=nthreads)
            rows_done += rows.size
            if time.perf_counter() - t0 >= min_seconds:
                break
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": round(rows_done / w.n * nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": nthreads,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"{rows_done} rows of the workload ({w.n} x {w.V}) in 256-row chunks: fp64 loss, gradient, "
                      f"log-sum-exp, log p_y and entropy, scaled to the step's algorithmic bytes"}


# ---------------------------------------------------------------- the pages' timing protocol

def pages_protocol(call, work, pristine, stream, dev, warmup: int = 10, reps: int = 3, samples: int = 50) -> dict:
    """Per-call latency measured the way the pages measure their CE table (Megatron-LM PR "Add opt-in
    Liger vocab-parallel cross entropy", Performance: 10 warmups, 3 x 50 samples, the median, fresh
    input clones outside the timed region): before every sample the logits are restored from the
    pristine copy and a 512 MB buffer is written, so the 256 MB Infinity Cache holds none of the
    restored logits; both untimed.  Each call is timed with HIP events on its stream."""
    import numpy as np
    import torch
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def sample(ev=None):
        work.copy_(pristine)
        flush.fill_(1)
        if ev:
            ev[0].record(stream)
        call(work)
        if ev:
            ev[1].record(stream)

    for _ in range(warmup):
        sample()
    rep_ms = []
    for _ in range(reps):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(samples)]
        for e in evs:
            sample(e)
        torch.cuda.synchronize()
        rep_ms.append([a.elapsed_time(b) for a, b in evs])
    flat = np.concatenate(rep_ms)
    return {"warmups": warmup, "reps": reps, "samples_per_rep": samples,
            "median_ms": round(float(np.median(flat)), 5), "p10_ms": round(float(np.percentile(flat, 10)), 5),
            "p90_ms": round(float(np.percentile(flat, 90)), 5),
            "rep_medians_ms": [round(float(np.median(r)), 5) for r in rep_ms]}


# ---------------------------------------------------------------- counter summaries

# the sources each measured kernel is compiled from: the persistent row kernel, and for the
# fused variant also its GEMM, transposes and driver
CE_SOURCES = ("ce_device.h", "ce_rows.h", "ce_rows_inst.hip", "ce_rows_mr.h", "ce_rows_mr.hip", "ce_rows_half.h",
              "ce_rows_half.hip", "ce_kernels.hip",
              "lce_internal.h")
FLCE_SOURCES = CE_SOURCES + ("gemm_mfma.h", "flce.hip", "ce_split.hip")


def kernel_source_hash(workload: str = "") -> str:
    files = FLCE_SOURCES if workload.startswith("flce") else CE_SOURCES
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


# the cross-entropy kernels a plain call may run (its profile is named for the one it ran)
CE_KERNELS = ("ce_half_kernel", "ce_rows_mr_kernel", "ce_rows_kernel", "ce_row_generic")


def profile_path(workload: str, resident: bool = False, kernel: str | None = None) -> str:
    if workload.startswith("flce"):
        return os.path.join(PROFILES, f"{'flce_resident_gemm' if resident else 'flce_gemm'}__{workload}.txt")
    if kernel is None:   # whichever cross-entropy kernel's summary exists for this workload
        for k in CE_KERNELS:
            p = os.path.join(PROFILES, f"{k}__{workload}.txt")
            if os.path.exists(p):
                return p
        kernel = CE_KERNELS[-1]
    return os.path.join(PROFILES, f"{kernel}__{workload}.txt")


def read_profile(workload: str, resident: bool = False) -> dict | None:
    try:
        with open(profile_path(workload, resident)) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    kv = {}
    for line in lines:
        if ": " in line and not line.startswith("#"):
            k, v = line.split(": ", 1)
            kv[k.strip()] = v.split()[0] if v.split() else ""
    return kv


def _rocprof(args: list[str], outdir: str, bench_args: list[str], timeout: int) -> None:
    env = dict(os.environ, TMPDIR="/tmp")
    cmd = ["rocprofv3", *args, "-f", "csv", "-d", outdir, "-o", "run", "--",
           sys.executable, os.path.join(ROOT, "bench.py"), *bench_args]
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, cwd="/tmp", env=env, timeout=timeout, check=True, stdout=subprocess.DEVNULL)


def _ours(name: str) -> bool:
    return ("ce_rows_kernel" in name or "ce_rows_mr_kernel" in name or "ce_half_kernel" in name
            or "ce_row_generic" in name)


# VALU counters of the row kernel (one rocprofv3 pass: 3 SQ counters, one GRBM counter)
VALU_COUNTERS = ("SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "VALUBusy", "GRBM_GUI_ACTIVE")
CUS, CLOCK_GHZ = 256, 2.4          # MI355X compute units and peak engine clock
TRANS_SLOWDOWN = 2                 # transcendentals take two issue slots (measured: half rate)


def valu_roofline(valu_insts: float, trans_insts: float, kernel_ns: float) -> dict:
    """The time the kernel's VALU instructions need at the issue rate (one wave64 instruction per CU per
    clock, transcendentals twice as long), and the kernel's fraction of that bound."""
    cycles = (valu_insts - trans_insts) + TRANS_SLOWDOWN * trans_insts   # CU-clocks, summed over CUs
    bound_ns = cycles / CUS / CLOCK_GHZ
    return {"bound_ns": bound_ns, "frac": bound_ns / kernel_ns if kernel_ns > 0 else float("nan")}


def collect_profiles(workload: str) -> int:
    import numpy as np
    import synth
    w = synth.ALL_CE_WORKLOADS[workload]
    raw = os.path.join(RAW_PROFILES, workload)
    os.makedirs(raw, exist_ok=True)
    base = ["--workload", workload, "--no-cpu-baseline", "--no-pages-protocol", "--no-event-pass"]
    _rocprof(["--kernel-trace", "--stats"], os.path.join(raw, "ktrace"), base + ["--steps", "10", "--warmup", "3"], 300)
    _rocprof(["--pmc", "FETCH_SIZE"], os.path.join(raw, "fetch"), base + ["--steps", "5", "--warmup", "2"], 180)
    _rocprof(["--pmc", "WRITE_SIZE"], os.path.join(raw, "write"), base + ["--steps", "5", "--warmup", "2"], 180)
    _rocprof(["--pmc", *VALU_COUNTERS], os.path.join(raw, "valu"), base + ["--steps", "5", "--warmup", "2"], 180)

    stats = list(csv.DictReader(open(os.path.join(raw, "ktrace", "run_kernel_stats.csv"))))
    ours = [r for r in stats if _ours(r["Name"])]
    copy_kib = w.n * w.V * w.elem_bytes / 1024.0          # the pristine copy made before each step

    def counter(sub: str, cname: str):
        rows = [r for r in csv.DictReader(open(os.path.join(raw, sub, "run_counter_collection.csv")))
                if r["Counter_Name"] == cname]
        k = [float(r["Counter_Value"]) for r in rows if _ours(r["Kernel_Name"])]
        # copies of the whole logits buffer (tiny copies of scalars are left out)
        c = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"] and int(r["Grid_Size"]) > 4096]
        return sum(k) / len(k), sum(c) / len(c), len(k), len(c)

    fk, fc, nfk, nfc = counter("fetch", "FETCH_SIZE")
    wk, wc, nwk, nwc = counter("write", "WRITE_SIZE")
    fscale, wscale = copy_kib / fc, copy_kib / wc
    traffic = (fk * fscale + wk * wscale) * 1024.0
    valu = {c: counter("valu", c)[0] for c in VALU_COUNTERS}
    # per dispatch, in launch order: 3 warmup calls, then the 10 back-to-back timed steps (what
    # ms_per_step covers); the profiled runs leave out the event-timed calls
    trace = sorted((r for r in csv.DictReader(open(os.path.join(raw, "ktrace", "run_kernel_trace.csv")))
                    if _ours(r["Kernel_Name"])), key=lambda r: int(r["Start_Timestamp"]))
    durs = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in trace]
    by_phase = []
    if len(durs) == 3 + 10:
        for name, d in (("warmup", durs[:3]), ("timed_steps", durs[3:13])):
            by_phase.append(f"kernel_ns_{name}: avg {np.mean(d):.1f} median {np.median(d):.1f} "
                            f"min {min(d)} max {max(d)}")
    kernel_ns = float(ours[0]["AverageNs"]) if ours else float("nan")
    vr = valu_roofline(valu["SQ_INSTS_VALU"], valu["SQ_INSTS_VALU_TRANS_F32"], kernel_ns)
    b = " ".join(base)
    lines = [
        f"# rocprofv3 summary: the cross-entropy kernel of lce_ce_fwd_bwd, workload {workload}",
        f"# ({w.n} x {w.V} {w.dtype}, eps {w.label_smoothing}, softcap {w.softcap}, argmax {w.want_argmax})",
        f"# made by: python bench.py --collect-profiles --workload {workload}",
        "# which runs, from /tmp with TMPDIR=/tmp:",
        f"#   rocprofv3 --kernel-trace --stats -f csv -d <raw>/ktrace -o run -- python bench.py {b} --steps 10 --warmup 3",
        f"#   rocprofv3 --pmc FETCH_SIZE -f csv -d <raw>/fetch -o run -- python bench.py {b} --steps 5 --warmup 2",
        f"#   rocprofv3 --pmc WRITE_SIZE -f csv -d <raw>/write -o run -- python bench.py {b} --steps 5 --warmup 2",
        f"#   rocprofv3 --pmc {' '.join(VALU_COUNTERS)} -f csv -d <raw>/valu -o run -- python bench.py {b} "
        "--steps 5 --warmup 2",
        "# Counter scale: what each counter reads for the plain copy (__amd_rocclr_copyBuffer) of the",
        f"# pristine logits -- a known {copy_kib:.0f} KiB read + {copy_kib:.0f} KiB write -- divided into that size.",
        "# VALU roofline: wave64 VALU instructions issue at one per CU per clock (4 SIMDs x 16 lanes),",
        "# transcendentals (exp, rcp, log) at half of that (measured on the device); 256 CUs at 2.4 GHz.",
        "#",
        "# kernel trace (--stats), nanoseconds:",
    ]
    for r in stats:
        lines.append(f"#   {r['Name'][:92]:<92} calls {r['Calls']:>4} avg {float(r['AverageNs']):>11.1f} "
                     f"min {r['MinNs']:>9} max {r['MaxNs']:>9}")
    lines += [
        f"kernel: {ours[0]['Name'] if ours else 'n/a'}",
        f"kernel_avg_ns: {float(ours[0]['AverageNs']):.1f}" if ours else "kernel_avg_ns: n/a",
        *by_phase,
        f"fetch_kib_per_dispatch: {fk:.1f}   ({nfk} dispatches)",
        f"copy_fetch_kib_per_dispatch: {fc:.1f}   ({nfc} dispatches)",
        f"fetch_scale: {fscale:.4f}",
        f"write_kib_per_dispatch: {wk:.1f}   ({nwk} dispatches)",
        f"copy_write_kib_per_dispatch: {wc:.1f}   ({nwc} dispatches)",
        f"write_scale: {wscale:.4f}",
        f"traffic_bytes_per_dispatch: {traffic:.0f}",
        f"algorithmic_bytes_per_dispatch: {algorithmic_bytes(w)}",
        f"valu_insts_per_dispatch: {valu['SQ_INSTS_VALU']:.0f}",
        f"valu_trans_f32_insts_per_dispatch: {valu['SQ_INSTS_VALU_TRANS_F32']:.0f}",
        f"valu_busy_pct: {valu['VALUBusy']:.1f}",
        f"grbm_gui_active_per_dispatch: {valu['GRBM_GUI_ACTIVE']:.0f}",
        f"valu_issue_bound_ns: {vr['bound_ns']:.1f}",
        f"valu_roofline_frac: {vr['frac']:.4f}",
        f"kernel_source_sha256_16: {kernel_source_hash(workload)}",
    ]
    os.makedirs(PROFILES, exist_ok=True)
    kname = next((k for k in CE_KERNELS if ours and k in ours[0]["Name"]), CE_KERNELS[-1])
    for k in CE_KERNELS:   # one summary per workload, named for the kernel that ran
        old = profile_path(workload, kernel=k)
        if k != kname and os.path.exists(old):
            os.remove(old)
    path = profile_path(workload, kernel=kname)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(open(path).read(), flush=True)
    return 0


# ---------------------------------------------------------------- fused linear variant

def flce_flops(w) -> int:
    # Z = H W^T, dH = G W, dW = G^T H: three dense contractions of 2 N H V flops each
    return 6 * w.n * w.H * w.V


def flce_cpu_baseline(w, hb, wb, y, nthreads: int) -> dict:
    """The oracle as it stands on a slice of the workload: the first `nthreads` tokens (one per host
    thread) with the full H and V; it forms Z, the per-token CE and both gradients in fp64."""
    import oracle
    k = max(1, nthreads)
    t0 = time.perf_counter()
    oracle.default().flce(hb[:k], wb, y[:k], label_smoothing=w.label_smoothing, softcap=w.softcap,
                          reduction=w.reduction, nthreads=nthreads)
    dt = time.perf_counter() - t0
    return {"value": round(6 * k * w.H * w.V / dt / 1e12, 6), "unit": "TFLOP/s", "cores": nthreads,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"first {k} tokens with the full H={w.H} and V={w.V} (6 k H V flops), fp64 loss, "
                      f"grad_hidden and grad_weight"}


def flce_setup(w, dev):
    import numpy as np
    import torch

    import synth
    hb = synth.flce_hidden_rows(w, np.arange(w.n))
    wb = synth.flce_weight_rows(w, np.arange(w.V))
    y = synth.labels(w)

    def up(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    return hb, wb, y, up(hb), up(wb), torch.from_numpy(y).to(dev)


def bench_flce(args, w) -> int:
    import numpy as np
    import torch

    import vocabulary_cross_entropy_row_amd as lce
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hb, wb, y, hidden, weight, labels = flce_setup(w, dev)
    print(f"# inputs resident: hidden {tuple(hidden.shape)}, weight {tuple(weight.shape)}", file=sys.stderr,
          flush=True)
    # a plain copy of known size: the reference that scales the traffic counters (untimed)
    ref_src = torch.empty(256 << 20, dtype=torch.int32, device=dev)
    torch.empty_like(ref_src).copy_(ref_src)
    grad_out = torch.full((1,), w.grad_out, dtype=torch.float32, device=dev)
    loss_tok = torch.empty(w.n, dtype=torch.float32, device=dev)
    loss_out = torch.empty(1, dtype=torch.float32, device=dev)
    grad_hidden = torch.empty((w.n, w.H), dtype=torch.bfloat16, device=dev)
    grad_weight = torch.empty((w.V, w.H), dtype=torch.float32, device=dev)
    counts = torch.empty(3, dtype=torch.int64, device=dev)
    nchunks = -(-w.n // w.chunk)
    default_wsb = lce.lce_flce_workspace_bytes(w.n, w.H, w.V, w.chunk)
    wsb = {"default": default_wsb, "wt": default_wsb + (2 * w.H * w.V + 255) // 256 * 256,
           "lean": lce.lce_flce_workspace_bytes_grouped(w.n, w.H, w.V, w.chunk, 1)}[args.flce_workspace]
    del nchunks
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    resident = args.path == "resident"
    if resident:
        f = lambda: torch.empty(w.n, dtype=torch.float32, device=dev)  # noqa: E731
        rows = lce.SplitRows(f(), f(), loss_tok, loss_out, f(), f(), torch.empty(w.n, dtype=torch.int64, device=dev),
                             counts)
        stats_ws = torch.empty(lce.lce_flce_stats_bytes(w.n, w.V), dtype=torch.uint8, device=dev)
    mid = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]

    def step(i=None):
        if not resident:
            lce.lce_flce_fwd_bwd(hidden, weight, labels, label_smoothing=w.label_smoothing, softcap=w.softcap,
                                 reduction=w.reduction, grad_out=grad_out, chunk_tokens=w.chunk, loss_tok=loss_tok,
                                 loss_out=loss_out, grad_hidden=grad_hidden, grad_weight=grad_weight, counts=counts,
                                 workspace=ws, stream=stream)
            return
        lce.lce_flce_forward(hidden, weight, labels, label_smoothing=w.label_smoothing, softcap=w.softcap,
                             reduction=w.reduction, workspace=stats_ws, out=rows, stream=stream)
        if i is not None:
            mid[i].record(stream)
        lce.lce_flce_backward(hidden, weight, labels, rows, label_smoothing=w.label_smoothing, softcap=w.softcap,
                              reduction=w.reduction, grad_out=grad_out, chunk_tokens=w.chunk, grad_hidden=grad_hidden,
                              grad_weight=grad_weight, workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # device memory a step allocates beyond what the caller already holds (inputs, outputs, workspace):
    # the binding allocates nothing when every buffer is passed, so this is expected to be 0
    base_alloc = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    step()
    torch.cuda.synchronize()
    step_extra = torch.cuda.max_memory_allocated(dev) - base_alloc
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
        print(f"# step {i} issued", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call_ms = [a.elapsed_time(b) for a, b in ev]
    ms_per_step = wall * 1e3 / args.steps
    call_ms = float(np.mean(per_call_ms))
    flops = flce_flops(w)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (call_ms * 1e-3) / 1e12
    prof = read_profile(w.name, resident)
    traffic = None
    if prof and prof.get("kernel_source_sha256_16") == kernel_source_hash(w.name):
        traffic = int(prof["traffic_bytes_per_dispatch"])
    out = {
        "metric": RESIDENT_METRIC if resident else FLCE_METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "n": w.n, "H": w.H, "V": w.V, "chunk_tokens": w.chunk,
                   "hidden_scale": w.hidden_scale, "w_sigma": w.w_sigma, "ignore_frac": w.ignore_frac,
                   "softcap": w.softcap, "label_smoothing": w.label_smoothing, "reduction": w.reduction,
                   "workspace_layout": args.flce_workspace, "workspace_bytes": wsb, "parallelism": "none (1 GPU)"},
        "memory": {"extra_device_bytes": wsb + (int(stats_ws.numel()) + 6 * 4 * w.n if resident else 0),
                   "workspace_bytes": wsb,
                   "forward_stats_bytes": int(stats_ws.numel()) if resident else 0,
                   "allocated_by_the_step_bytes": int(step_extra),
                   "bf16_logits_bytes_for_comparison": 2 * w.n * w.V,
                   "grad_weight_fp32_bytes": 4 * w.V * w.H,
                   "note": "extra device memory beyond the inputs (hidden, weight, labels) and the outputs "
                           "(grad_hidden, fp32 grad_weight, losses, counts)"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                     "kernel": ("lce_flce_forward + lce_flce_backward" if resident else "lce_flce_fwd_bwd call") +
                               " (all GEMM, CE and transpose launches), HIP events per step",
                     "call_ms_mean": round(call_ms, 4), "call_ms_min": round(min(per_call_ms), 4),
                     "call_ms_max": round(max(per_call_ms), 4), **call_percentiles(per_call_ms, 4),
                     "algorithmic_flops": flops},
        "cpu_baseline": None,
    }
    if resident:
        fwd_ms = float(np.mean([a.elapsed_time(m) for (a, _), m in zip(ev, mid)]))
        out["phase_ms"] = {"forward": round(fwd_ms, 4), "backward": round(call_ms - fwd_ms, 4)}
        out["executed_flops"] = 8 * w.n * w.H * w.V   # the backward forms the logits again
        out["executed_tflops"] = round(8 * w.n * w.H * w.V / (call_ms * 1e-3) / 1e12, 2)
    if not args.no_cpu_baseline:
        nthr = len(os.sched_getaffinity(0))
        if os.environ.get("OMP_NUM_THREADS"):
            nthr = min(nthr, int(os.environ["OMP_NUM_THREADS"]))
        out["cpu_baseline"] = flce_cpu_baseline(w, hb, wb, y, nthr)
    print(json.dumps(out), flush=True)
    return 0


def collect_profiles_flce(workload: str, resident: bool = False) -> int:
    import synth
    w = synth.FLCE_WORKLOADS[workload]
    raw = os.path.join(RAW_PROFILES, workload + ("_resident" if resident else ""))
    os.makedirs(raw, exist_ok=True)
    base = ["--workload", workload, "--no-cpu-baseline"] + (["--path", "resident"] if resident else [])
    _rocprof(["--kernel-trace", "--stats"], os.path.join(raw, "ktrace"), base + ["--steps", "3", "--warmup", "1"], 600)
    _rocprof(["--pmc", "FETCH_SIZE"], os.path.join(raw, "fetch"), base + ["--steps", "1", "--warmup", "1"], 600)
    _rocprof(["--pmc", "WRITE_SIZE"], os.path.join(raw, "write"), base + ["--steps", "1", "--warmup", "1"], 600)
    _rocprof(["--pmc", "TCC_HIT_sum", "TCC_MISS_sum"], os.path.join(raw, "l2"), base + ["--steps", "1", "--warmup", "1"],
             600)
    stats = list(csv.DictReader(open(os.path.join(raw, "ktrace", "run_kernel_stats.csv"))))
    calls = 5   # the trace run's calls: 1 warmup, the memory-measuring call, 3 steps
    ref_kib = (256 << 20) * 4 / 1024.0
    ours = ("gemm_nt_kernel", "transpose_bf16_kernel", "splitk_fold_kernel", "ce_rows_kernel", "ce_count_kernel",
            "loss_fold_kernel", "fill_zero_f32_kernel", "ce_row_generic", "ce_combine")

    def counter(sub: str, cname: str):
        rows = list(csv.DictReader(open(os.path.join(raw, sub, "run_counter_collection.csv"))))
        rows = [r for r in rows if r["Counter_Name"] == cname]
        k = [float(r["Counter_Value"]) for r in rows if any(o in r["Kernel_Name"] for o in ours)]
        c = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        # per call: the run makes 3 calls (1 warmup, the memory-measuring call, 1 step); the reference
        # copy is the largest copy
        return sum(k) / 3.0, max(c), len(k)

    fk, fc, nfk = counter("fetch", "FETCH_SIZE")
    wk, wc, nwk = counter("write", "WRITE_SIZE")
    fscale, wscale = ref_kib / fc, ref_kib / wc
    traffic = (fk * fscale + wk * wscale) * 1024.0

    def per_gemm(sub: str, cname: str) -> dict:
        """Counter per GEMM launch kind (the kernel's template arguments name its output mode), averaged
        over that kind's launches."""
        rows = [r for r in csv.DictReader(open(os.path.join(raw, sub, "run_counter_collection.csv")))
                if r["Counter_Name"] == cname and "gemm_nt_kernel" in r["Kernel_Name"]]
        acc = {}
        for r in rows:
            key = r["Kernel_Name"].split("(")[0].replace("void lce::gemm::", "")
            tot, cnt = acc.get(key, (0.0, 0))
            acc[key] = (tot + float(r["Counter_Value"]), cnt + 1)
        return {k: (t / c, c) for k, (t, c) in acc.items()}

    gemm_fetch = per_gemm("fetch", "FETCH_SIZE")
    gemm_hit = per_gemm("l2", "TCC_HIT_sum")
    gemm_miss = per_gemm("l2", "TCC_MISS_sum")
    b = " ".join(base)
    total_ns = sum(float(r["TotalDurationNs"]) for r in stats if any(o in r["Name"] for o in ours)) / calls
    what = ("tile-resident fused linear cross-entropy (lce_flce_forward + lce_flce_backward)" if resident
            else "fused linear cross-entropy (lce_flce_fwd_bwd)")
    lines = [
        f"# rocprofv3 summary: {what}, workload {workload}",
        f"# (hidden {w.n} x {w.H}, weight {w.V} x {w.H} bf16, chunk {w.chunk}, softcap {w.softcap})",
        f"# made by: python bench.py --collect-profiles --workload {workload}" + (" --path resident" if resident else ""),
        "# which runs, from /tmp with TMPDIR=/tmp:",
        f"#   rocprofv3 --kernel-trace --stats -f csv -d <raw>/ktrace -o run -- python bench.py {b} --steps 3 --warmup 1",
        f"#   rocprofv3 --pmc FETCH_SIZE -f csv -d <raw>/fetch -o run -- python bench.py {b} --steps 1 --warmup 1",
        f"#   rocprofv3 --pmc WRITE_SIZE -f csv -d <raw>/write -o run -- python bench.py {b} --steps 1 --warmup 1",
        f"#   rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum -f csv -d <raw>/l2 -o run -- python bench.py {b} --steps 1 "
        "--warmup 1",
        "# Counter scale: what each counter reads for a plain 1 GiB device copy (__amd_rocclr_copyBuffer)",
        "# made once before timing, divided into its known size.  Traffic is per step (one call, or",
        "# forward + backward), summed over all of its kernels.",
        "#",
        "# kernel trace (--stats), nanoseconds (per-call share = total / calls):",
    ]
    for r in stats:
        lines.append(f"#   {r['Name'][:80]:<80} calls {r['Calls']:>5} avg {float(r['AverageNs']):>12.1f} "
                     f"per-call-share {float(r['TotalDurationNs']) / calls / 1e6:>8.3f} ms")
    gemm = [r for r in stats if "gemm_nt_kernel" in r["Name"]]
    gemm_ns = sum(float(r["TotalDurationNs"]) for r in gemm) / calls
    if resident:
        # the stats GEMM (epilogue mode 3) is one launch per forward: 2 n H V flops
        st = [r for r in gemm if "gemm_nt_kernel<3" in r["Name"]]
        if st:
            st_ns = float(st[0]["AverageNs"])
            lines += [f"stats_gemm_kernel: {st[0]['Name']}", f"stats_gemm_avg_ns: {st_ns:.1f}",
                      f"stats_gemm_tflops: {2 * w.n * w.H * w.V / (st_ns * 1e-9) / 1e12:.1f}"]
        lines.append("gemm_flops_executed_per_step: " + str(8 * w.n * w.H * w.V) + "   (the backward forms the logits again)")
    lines += [
        f"call_kernel_ns: {total_ns:.0f}",
        f"gemm_kernel_ns_per_call: {gemm_ns:.0f}",
        f"gemm_tflops: {flce_flops(w) / (gemm_ns * 1e-9) / 1e12:.1f}",
        f"call_tflops_kernels_only: {flce_flops(w) / (total_ns * 1e-9) / 1e12:.1f}",
        f"fetch_kib_per_call: {fk:.1f}   ({nfk} dispatches)",
        f"copy_fetch_kib: {fc:.1f}",
        f"fetch_scale: {fscale:.4f}",
        f"write_kib_per_call: {wk:.1f}   ({nwk} dispatches)",
        f"copy_write_kib: {wc:.1f}",
        f"write_scale: {wscale:.4f}",
        f"traffic_bytes_per_dispatch: {traffic:.0f}",
        f"algorithmic_flops_per_call: {flce_flops(w)}",
        "# per GEMM launch kind (averaged over its launches): duration, FETCH_SIZE scaled to bytes, L2 hits / misses",
    ]
    for r in gemm:
        key = r["Name"].split("(")[0].replace("void lce::gemm::", "")
        f_kib = gemm_fetch.get(key, (float("nan"), 0))[0]
        hit, miss = gemm_hit.get(key, (float("nan"), 0))[0], gemm_miss.get(key, (float("nan"), 0))[0]
        lines.append(f"gemm: {key}  avg_ns {float(r['AverageNs']):.0f}  calls {r['Calls']}  "
                     f"fetch_bytes {f_kib * fscale * 1024.0:.4g}  l2_hit {hit:.4g}  l2_miss {miss:.4g}  "
                     f"l2_hit_rate {hit / (hit + miss) if hit + miss > 0 else float('nan'):.3f}")
    lines.append(f"kernel_source_sha256_16: {kernel_source_hash(workload)}")
    os.makedirs(PROFILES, exist_ok=True)
    with open(profile_path(workload, resident), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(open(profile_path(workload, resident)).read(), flush=True)
    return 0


# ---------------------------------------------------------------- split path

SPLIT_METRIC = "split CE (stats, combine, gradient) ms and HBM GB/s (% peak), bf16 logits 2048×131072, 1 GPU"


def bench_split(args, w) -> int:
    """One step = lce_ce_stats on every shard + lce_ce_combine + lce_ce_grad on every shard, each shard its
    own contiguous [N, V / tp] tensor as a rank of a vocabulary-parallel layout holds it (with one shard a
    forward / deferred-backward pair).  Algorithmic bytes: one read for the statistics and one read + write
    for the gradient, 3 N V b, plus the records and row outputs."""
    import numpy as np
    import torch

    import vocabulary_cross_entropy_row_amd as lce
    import synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    y = synth.labels(w)
    x = synth.logits(w, y)
    tp = args.tp
    if w.V % (8 * tp):
        print(f"V = {w.V} does not split into {tp} shards of whole 16-byte vectors", file=sys.stderr)
        return 2
    ws = w.V // tp
    full = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    pristine = [full[:, k * ws:(k + 1) * ws].contiguous() for k in range(tp)]   # shard k: columns [k ws, (k+1) ws)
    del full
    labels = torch.from_numpy(y).to(dev)
    nbuf = args.warmup + args.steps
    bufs = [[p.clone() for p in pristine] for _ in range(nbuf)]
    stats = torch.empty((tp, w.n, 8), dtype=torch.float32, device=dev)
    grad_out = torch.full((1,), w.grad_out, dtype=torch.float32, device=dev)
    fv = lambda: torch.empty(w.n, dtype=torch.float32, device=dev)  # noqa: E731
    rows_out = lce.SplitRows(fv(), fv(), fv(), torch.empty(1, dtype=torch.float32, device=dev), fv(), fv(),
                             torch.empty(w.n, dtype=torch.int64, device=dev), torch.empty(3, dtype=torch.int64, device=dev))
    stream = torch.cuda.current_stream()
    ev = {k: [] for k in ("stats", "combine", "grad")}

    def step(buf, timed):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if timed else [None] * 4
        mark = (lambda i: e[i].record(stream)) if timed else (lambda i: None)  # noqa: E731
        mark(0)
        for k in range(tp):
            lce.lce_ce_stats(buf[k], labels, v_offset=k * ws, softcap=w.softcap, stats=stats[k], stream=stream)
        mark(1)
        rows = lce.lce_ce_combine(stats, labels, w.V, label_smoothing=w.label_smoothing, reduction=w.reduction,
                                  out=rows_out, stream=stream)
        mark(2)
        for k in range(tp):
            lce.lce_ce_grad(buf[k], labels, w.V, rows, v_offset=k * ws,
                            label_smoothing=w.label_smoothing, softcap=w.softcap, reduction=w.reduction,
                            grad_out=grad_out, stream=stream)
        mark(3)
        if timed:
            ev["stats"].append((e[0], e[1]))
            ev["combine"].append((e[1], e[2]))
            ev["grad"].append((e[2], e[3]))
        return e

    for i in range(args.warmup):
        step(bufs[i], False)
    # the timed steps: back to back, nothing between the calls
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(bufs[args.warmup + i], False)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    # phase and call durations: the same steps again on restored logits, HIP events between the phases
    for i in range(args.steps):
        for b, p in zip(bufs[args.warmup + i], pristine):
            b.copy_(p)
    torch.cuda.synchronize()
    whole = [step(bufs[args.warmup + i], True) for i in range(args.steps)]
    torch.cuda.synchronize()
    call_ms = float(np.mean([a[0].elapsed_time(a[3]) for a in whole]))
    phase = {k: round(float(np.mean([a.elapsed_time(b) for a, b in v])), 5) for k, v in ev.items()}
    nbytes = 3 * w.n * w.V * w.elem_bytes + w.n * (8 + tp * 32 * 2 + 4 * 6)
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (call_ms * 1e-3) / 1e9
    out = {
        "metric": SPLIT_METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "n": w.n, "V": w.V, "shards": tp, "shard_V": ws, "logits_dtype": w.dtype,
                   "shard_layout": "contiguous [n, V / tp] per shard",
                   "parallelism": f"vocabulary split into {tp} shards on one GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "traffic_scope": "every kernel of one step (rocprofv3 FETCH_SIZE + WRITE_SIZE, profiles/)",
                     "kernel": "stats + combine + gradient calls of one step, HIP events", "phase_ms": phase,
                     "stats_GBps": round(w.n * w.V * w.elem_bytes / (phase["stats"] * 1e-3) / 1e9, 1),
                     "grad_GBps": round(2 * w.n * w.V * w.elem_bytes / (phase["grad"] * 1e-3) / 1e9, 1),
                     "algorithmic_bytes": nbytes},
        "cpu_baseline": None,
    }
    prof = read_split_profile(w.name, tp)
    if prof:
        out["roofline"]["rocprof_kernel_ns"] = {k: float(v) for k, v in prof.items() if k.endswith("_avg_ns")}
        if "traffic_bytes_per_step" in prof:
            out["roofline"]["traffic"] = int(float(prof["traffic_bytes_per_step"]))
    if not args.no_cpu_baseline:
        nthr = len(os.sched_getaffinity(0))
        if os.environ.get("OMP_NUM_THREADS"):
            nthr = min(nthr, int(os.environ["OMP_NUM_THREADS"]))
        out["cpu_baseline"] = split_cpu_baseline(w, x, y, nbytes, nthr)
    print(json.dumps(out), flush=True)
    return 0


SPLIT_SOURCES = ("ce_device.h", "lce_internal.h", "ce_split.hip", "ce_kernels.hip")


def split_profile_path(workload: str, tp: int) -> str:
    return os.path.join(PROFILES, f"ce_split__{workload}_tp{tp}.txt")


def split_source_hash() -> str:
    h = hashlib.sha256()
    for f in SPLIT_SOURCES:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def read_split_profile(workload: str, tp: int) -> dict | None:
    try:
        lines = open(split_profile_path(workload, tp)).read().splitlines()
    except OSError:
        return None
    kv = {}
    for line in lines:
        if ": " in line and not line.startswith("#"):
            k, v = line.split(": ", 1)
            kv[k.strip()] = v.split()[0] if v.split() else ""
    if kv.get("kernel_source_sha256_16") != split_source_hash():
        return None
    return kv


SPLIT_KERNELS = ("ce_stats_kernel", "ce_combine", "ce_grad_kernel", "ce_count_kernel", "loss_fold_kernel")


def collect_profiles_split(workload: str, tp: int) -> int:
    """Kernel trace of the split path's three kernels (stats per shard, combine, gradient per shard),
    then FETCH_SIZE and WRITE_SIZE of every kernel a step launches, scaled like the fused path's."""
    import synth
    w = synth.ALL_CE_WORKLOADS[workload]
    raw = os.path.join(RAW_PROFILES, f"{workload}_split_tp{tp}")
    os.makedirs(raw, exist_ok=True)
    base = ["--workload", workload, "--no-cpu-baseline", "--path", "split", "--tp", str(tp)]
    _rocprof(["--kernel-trace", "--stats"], os.path.join(raw, "ktrace"), base + ["--steps", "10", "--warmup", "3"], 300)
    _rocprof(["--pmc", "FETCH_SIZE"], os.path.join(raw, "fetch"), base + ["--steps", "5", "--warmup", "2"], 180)
    _rocprof(["--pmc", "WRITE_SIZE"], os.path.join(raw, "write"), base + ["--steps", "5", "--warmup", "2"], 180)
    stats = list(csv.DictReader(open(os.path.join(raw, "ktrace", "run_kernel_stats.csv"))))
    copy_kib = w.n * (w.V // tp) * w.elem_bytes / 1024.0   # the pristine copy of one shard (one per shard and step)

    def counter(sub: str, cname: str):
        rows = [r for r in csv.DictReader(open(os.path.join(raw, sub, "run_counter_collection.csv")))
                if r["Counter_Name"] == cname]
        ours = sum(float(r["Counter_Value"]) for r in rows if any(k in r["Kernel_Name"] for k in SPLIT_KERNELS))
        c = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"] and int(r["Grid_Size"]) > 4096]
        return ours / 12.0, sum(c) / len(c)   # 2 warmup steps, 5 timed back to back, 5 again with events

    fk, fc = counter("fetch", "FETCH_SIZE")
    wk, wc = counter("write", "WRITE_SIZE")
    traffic = (fk * copy_kib / fc + wk * copy_kib / wc) * 1024.0
    b = " ".join(base)
    lines = [
        f"# rocprofv3 summary: split cross-entropy (lce_ce_stats per shard, lce_ce_combine, lce_ce_grad per shard),",
        f"# workload {workload} ({w.n} x {w.V} {w.dtype}) as {tp} vocabulary shards of {w.V // tp} columns",
        f"# made by: python bench.py --collect-profiles --workload {workload} --path split --tp {tp}",
        "# which runs, from /tmp with TMPDIR=/tmp:",
        f"#   rocprofv3 --kernel-trace --stats -f csv -d <raw>/ktrace -o run -- python bench.py {b} --steps 10 --warmup 3",
        f"#   rocprofv3 --pmc FETCH_SIZE -f csv -d <raw>/fetch -o run -- python bench.py {b} --steps 5 --warmup 2",
        f"#   rocprofv3 --pmc WRITE_SIZE -f csv -d <raw>/write -o run -- python bench.py {b} --steps 5 --warmup 2",
        "# Counter scale: what each counter reads for the plain copy (__amd_rocclr_copyBuffer) of a pristine",
        f"# shard -- a known {copy_kib:.0f} KiB read + {copy_kib:.0f} KiB write -- divided into that size.",
        "# Each shard is its own contiguous [n, V / tp] tensor.",
        "# kernel trace (--stats), nanoseconds per launch (13 steps; stats and grad launch once per shard):",
    ]
    for r in stats:
        lines.append(f"#   {r['Name'][:92]:<92} calls {r['Calls']:>4} avg {float(r['AverageNs']):>11.1f} "
                     f"min {r['MinNs']:>9} max {r['MaxNs']:>9}")
    for key, sub in (("stats", "ce_stats_kernel"), ("combine", "ce_combine"), ("grad", "ce_grad_kernel")):
        rs = [r for r in stats if sub in r["Name"]]
        if rs:
            ns = sum(float(r["TotalDurationNs"]) for r in rs) / sum(int(r["Calls"]) for r in rs)
            lines.append(f"{key}_avg_ns: {ns:.1f}")
    shard_bytes = w.n * (w.V // tp) * w.elem_bytes
    lines += [f"stats_bytes_per_launch: {shard_bytes}", f"grad_bytes_per_launch: {2 * shard_bytes}",
              f"fetch_kib_per_step: {fk:.1f}", f"fetch_scale: {copy_kib / fc:.4f}",
              f"write_kib_per_step: {wk:.1f}", f"write_scale: {copy_kib / wc:.4f}",
              f"traffic_bytes_per_step: {traffic:.0f}",
              f"kernel_source_sha256_16: {split_source_hash()}"]
    os.makedirs(PROFILES, exist_ok=True)
    with open(split_profile_path(workload, tp), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(open(split_profile_path(workload, tp)).read(), flush=True)
    return 0


# ---------------------------------------------------------------- the bench

def main() -> int:
    args = parse()
    import synth
    if args.collect_profiles:
        if args.path == "split":
            return collect_profiles_split(args.workload, args.tp)
        if args.workload in synth.FLCE_WORKLOADS:
            return collect_profiles_flce(args.workload, args.path == "resident")
        return collect_profiles(args.workload)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: there is no multi-GPU path (token rows would shard "
              "across GPUs with no exchange but the valid count and the loss sum). Run with --gpus 1.",
              file=sys.stderr)
        return 2

    if args.workload in synth.FLCE_WORKLOADS:
        if args.steps is None:
            args.steps = 20
        return bench_flce(args, synth.FLCE_WORKLOADS[args.workload])
    if args.path == "split":
        if args.steps is None:
            args.steps = 20
        return bench_split(args, synth.ALL_CE_WORKLOADS[args.workload])

    import numpy as np
    import torch

    import vocabulary_cross_entropy_row_amd as lce

    w = synth.ALL_CE_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    y = synth.labels(w)
    x = synth.logits(w, y)
    if w.dtype == "bf16":
        pristine = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        pristine = torch.from_numpy(x).to(dev)
    labels = torch.from_numpy(y).to(dev)
    if args.steps is None:
        # each timed step gets its own pristine copy; enough steps that the fixed cost of the
        # first launch and the final synchronisation (~0.1 ms) is spread thin
        per_buf = w.n * w.V * w.elem_bytes
        args.steps = int(min(100, max(20, 64e9 // per_buf - args.warmup)))
    # the warmup calls, the back-to-back timed steps and the event-timed calls each get their own
    # pristine copy, all made here, so no bulk restore runs between the two timed passes
    nbuf = args.warmup + (1 if args.no_event_pass else 2) * args.steps
    bufs = [torch.empty_like(pristine) for _ in range(nbuf)]
    for b in bufs:
        b.copy_(pristine)
    grad_out = torch.full((1,), w.grad_out, dtype=torch.float32, device=dev)
    loss_tok = torch.empty(w.n, dtype=torch.float32, device=dev)
    loss_out = torch.empty(1, dtype=torch.float32, device=dev)
    argmax = torch.empty(w.n, dtype=torch.int64, device=dev) if w.want_argmax else None
    counts = torch.empty(3, dtype=torch.int64, device=dev)
    ws = torch.zeros(lce.lce_ce_workspace_bytes(w.n, w.V), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(buf):
        lce.lce_ce_fwd_bwd(buf, labels, label_smoothing=w.label_smoothing, softcap=w.softcap,
                           reduction=w.reduction, grad_out=grad_out, loss_tok=loss_tok, loss_out=loss_out,
                           argmax_out=argmax, counts=counts, workspace=ws, stream=stream)

    for i in range(args.warmup):
        step(bufs[i])
    torch.cuda.synchronize()

    # the timed steps: back to back, nothing between the calls
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(bufs[args.warmup + i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    # per-call durations (the roofline's): as many calls again on their own pristine copies, HIP
    # events around each call on the stream it runs on
    if args.no_event_pass:
        per_call_ms = [ms_per_step]
    else:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            ev[i][0].record(stream)
            step(bufs[args.warmup + args.steps + i])
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        per_call_ms = [a.elapsed_time(b) for a, b in ev]
    call_ms = float(np.mean(per_call_ms))
    # context, after the timed region: a plain device copy of the same logits (one read + one write of
    # N V b bytes, the same traffic as one call), HIP events around each copy
    cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
    for a_, b_ in cev:
        a_.record(stream)
        bufs[0].copy_(pristine)
        b_.record(stream)
    torch.cuda.synchronize()
    copy_ms = float(np.median([a_.elapsed_time(b_) for a_, b_ in cev]))
    pages = None if args.no_pages_protocol else pages_protocol(step, bufs[0], pristine, stream, dev)

    nbytes = algorithmic_bytes(w)
    prof = read_profile(w.name)
    traffic = None
    if prof and prof.get("kernel_source_sha256_16") == kernel_source_hash(w.name):
        traffic = int(prof["traffic_bytes_per_dispatch"])
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (call_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "n": w.n, "V": w.V, "logits_dtype": w.dtype, "sigma": w.sigma,
                   "ignore_frac": w.ignore_frac, "label_smoothing": w.label_smoothing, "softcap": w.softcap,
                   "reduction": w.reduction, "grad_out": w.grad_out, "argmax": w.want_argmax,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "lce_ce_fwd_bwd call = one persistent row-kernel launch, HIP events per call",
                     "call_ms_mean": round(call_ms, 5), "call_ms_min": round(min(per_call_ms), 5),
                     "call_ms_max": round(max(per_call_ms), 5), **call_percentiles(per_call_ms, 5),
                     "algorithmic_bytes": nbytes,
                     "copy_GBps_same_bytes": round(2 * w.n * w.V * w.elem_bytes / (copy_ms * 1e-3) / 1e9, 1),
                     "workspace_bytes": int(ws.numel())},
        "cpu_baseline": None,
    }
    if pages is not None:
        pages["GBps_at_median"] = round(nbytes / (pages["median_ms"] * 1e-3) / 1e9, 1)
        pages["frac_at_median"] = round(nbytes / (pages["median_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        out["pages_protocol"] = pages
    if prof and traffic is not None and "valu_roofline_frac" in prof:
        out["valu"] = {"bound": "alu", "issue_bound_ms": round(float(prof["valu_issue_bound_ns"]) * 1e-6, 5),
                       "kernel_ms_rocprof": round(float(prof["kernel_avg_ns"]) * 1e-6, 5),
                       "frac": float(prof["valu_roofline_frac"]), "valu_busy_pct": float(prof["valu_busy_pct"]),
                       "source": os.path.relpath(profile_path(w.name), ROOT)}
    if w.n == 2048 and w.V == 131072 and w.dtype == "bf16":
        out["context_other_hardware"] = H100_CONTEXT
    if not args.no_cpu_baseline:
        nthr = len(os.sched_getaffinity(0))
        if os.environ.get("OMP_NUM_THREADS"):
            nthr = min(nthr, int(os.environ["OMP_NUM_THREADS"]))
        out["cpu_baseline"] = cpu_baseline(w, x, y, nthr)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
