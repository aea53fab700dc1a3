#!/usr/bin/env python3
"""Benchmark of the FlashAttention-2 forward pass on one MI355X.

One step = one fa2_fwd call (the whole forward pass: Q/K/V staging, both MFMA
products, the online softmax, masking, P handoff and the epilogue) over the
B=4, H=8, S=4096, D=64 non-causal fp16 workload, inputs already resident in HBM.
Prints one JSON line:

    value      FLOP rate, 4*B*H*S^2*D FLOPs (halved when causal) / average step time
    roofline   the kernel against the MI355X dense fp16 MFMA peak (2516.6 TFLOP/s),
               its duration taken with HIP events on the launch stream
    cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same
               workload on this host's cores (a reported baseline, not a target)

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload 2] [--causal]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_F16_PEAK_TFLOPS = 2516.6   # MI355X dense fp16 MFMA, 256 CUs x 2.4 GHz x 4096 FLOP/clk/CU
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = [os.path.join(ROOT, "attention_forward_fa2_amd", "csrc", f)
                  for f in ("fa2_fwd_kernel.hip", "fa2_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa2_fwd_B4H8S4096D64_noncausal_traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: int, causal: bool):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, or None if the counters were taken on other kernel source."""
    if workload != 2 or causal or not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return float(t["hbm_bytes_per_launch"])


def cpu_baseline(q, k, v, causal, scale, stride):
    """Time the fp64 oracle on every `stride`-th query row of the workload."""
    import numpy as np
    import oracle
    B, H, S, D = q.shape
    rows = np.arange(0, B * H * S, stride, dtype=np.int64)
    _, _, secs = oracle.timed_rows(q, k, v, causal, scale, rows)
    if causal:
        flops = float(np.sum(4.0 * D * ((rows % S) + 1)))
    else:
        flops = 4.0 * D * S * len(rows)
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle", "seconds": secs,
            "sample": (f"all {len(rows)} query rows of the workload" if stride == 1 else
                       f"every {stride}th query row ({len(rows)} of {B * H * S} rows) of the workload")
                      + ", fp64 oracle, FLOPs counted as 4*D per admitted key"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--causal", action="store_true", help="run the causal variant of the workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-stride", type=int, default=1, help="oracle sample: every n-th row (1 = all rows)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run 10 plain device-to-device copies of MIB MiB "
                         "(the reference kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    if args.copy_calibration:
        import torch
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                          "copies": 10}), flush=True)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the forward pass here has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import attention_forward_fa2_amd as fa2
    from fa2_inputs import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    causal = bool(args.causal) or w.causal_modes == (True,)
    if causal not in w.causal_modes:
        raise SystemExit(f"workload {args.workload} is not run in this mode")
    dev = torch.device("cuda:0")
    log(f"bench: workload {args.workload} ({w.name}) causal={causal} steps={args.steps} warmup={args.warmup}")
    q, k, v = make_inputs(args.workload)
    qt, kt, vt = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    o = torch.empty_like(qt)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    ptrs = (qt.data_ptr(), kt.data_ptr(), vt.data_ptr(), o.data_ptr(), lse.data_ptr())

    def step():
        st = fa2.fa2_fwd(*ptrs, w.B, w.H, w.S, w.D, int(causal), w.scale, sp)
        if st != 0:
            raise fa2.FA2Error(st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("bench: warmup done")

    # Per-launch events on the launch stream give the kernel duration; the outer
    # pair gives the step time.
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / args.steps
    kern_ms = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    kern_avg_ms = sum(kern_ms) / len(kern_ms)
    log(f"bench: {ms_per_step * 1e3:.1f} us/step, kernel avg {kern_avg_ms * 1e3:.1f} us "
        f"(min {kern_ms[0] * 1e3:.1f}, median {kern_ms[len(kern_ms) // 2] * 1e3:.1f})")

    flops = w.flops(causal)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kern_avg_ms * 1e-3) / 1e12
    traffic = measured_traffic(args.workload, causal)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                "traffic": traffic}

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a sample")
        cpu = cpu_baseline(q, k, v, causal, float(np.float32(w.scale)), args.cpu_stride)
        log(f"bench: oracle {cpu['seconds']:.1f} s on {cpu['cores']} threads")

    rec = {
        "metric": "FA2 fwd TFLOP/s (4*B*H*S^2*D, 1/2 causal) and % of MI355X FP16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"attention fwd {w.name} {'causal' if causal else 'non-causal'}",
                   "B": w.B, "H": w.H, "S": w.S, "D": w.D, "causal": causal, "scale": w.scale,
                   "inputs": "fp16 iid normal, seeds 1000*w+{0,1,2}",
                   "pct_of_fp16_mfma_peak": round(100 * value / MFMA_F16_PEAK_TFLOPS, 2)},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
