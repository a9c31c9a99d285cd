#!/usr/bin/env python3
"""Bench: cross-entropy forward+backward on MI355X through the C ABI.

One step = one lce_ce_fwd_bwd call (count kernel + row kernel: per-token loss, reduced
loss, argmax/accuracy when the workload asks for it, gradient written in place) over one
batch of synthetic logits already resident in HBM.  The gradient overwrites its input, so
every step gets its own pristine copy, made before the timed region (the pages' Megatron
benchmark likewise clones its inputs outside timing).

Prints ONE JSON line.  `value` is algorithmic HBM throughput (2 N V b + 12 N bytes per
step over the measured step time), the default workload is bf16 [2048, 131072].
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CE fwd+bwd ms and HBM GB/s (% peak), bf16 logits 2048×131072, 1 GPU"
HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published


def algorithmic_bytes(w) -> int:
    # one read + one write of the logits, 8 B label read + 4 B loss write per token
    return 2 * w.n * w.V * w.elem_bytes + 12 * w.n


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="ce_bf16_2048x131072")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def cpu_baseline(w, x, y, nthreads: int) -> dict:
    """The oracle as it stands, on the host cores, over the whole workload (grads in chunks)."""
    import numpy as np

    import oracle
    orc = oracle.default()
    chunk = 256
    t0 = time.perf_counter()
    for r0 in range(0, w.n, chunk):
        rows = np.arange(r0, min(w.n, r0 + chunk))
        orc.ce(x, y, V=w.V, label_smoothing=w.label_smoothing, softcap=w.softcap, reduction=w.reduction,
               grad_out=[w.grad_out], rows=rows, want_grad=True, nthreads=nthreads)
    dt = time.perf_counter() - t0
    return {"value": round(algorithmic_bytes(w) / dt / 1e9, 4), "unit": "GB/s", "cores": nthreads,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"the whole workload ({w.n} rows x {w.V}), fp64 loss+argmax+gradient, "
                      f"{chunk}-row chunks, OpenMP over rows"}


def main() -> int:
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(rows shard with no exchange; see the design notes). Run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import synth
    import vocabulary_cross_entropy_row_amd as lce

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    y = synth.labels(w)
    x = synth.logits(w, y)
    if w.dtype == "bf16":
        pristine = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        pristine = torch.from_numpy(x).to(dev)
    labels = torch.from_numpy(y).to(dev)
    nbuf = args.warmup + args.steps
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

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(bufs[args.warmup + i])
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call_ms = [a.elapsed_time(b) for a, b in ev]
    ms_per_step = wall * 1e3 / args.steps
    call_ms = float(np.mean(per_call_ms))

    nbytes = algorithmic_bytes(w)
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
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "lce_ce_fwd_bwd call (count + row kernel), HIP events per call",
                     "call_ms_mean": round(call_ms, 5), "call_ms_min": round(min(per_call_ms), 5),
                     "call_ms_max": round(max(per_call_ms), 5), "algorithmic_bytes": nbytes},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        nthr = len(os.sched_getaffinity(0))
        if os.environ.get("OMP_NUM_THREADS"):
            nthr = min(nthr, int(os.environ["OMP_NUM_THREADS"]))
        out["cpu_baseline"] = cpu_baseline(w, x, y, nthr)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
