"""Benchmark: achieved HBM GB/s and logits rows/s of the FP8 E4M3 LM head.

Workload (default): the 1.27 GB FP8 head -- vocab 155136 x hidden 8192 E4M3
weights (N(0, 0.015) draws quantized per row on the device, F32 row scales),
BF16 activations from N(0, 1) -- decoded at rows 1, 2, 4, 8 and 16. One step
is one pass of the head path over that batch: five qhead_fp8_rowscale calls,
each one weight pass. The weights are resident in HBM before timing starts.

value = algorithmic bytes of the step / step time, where a launch's
algorithmic bytes are W + row scales + R * (2 * hidden + 2 * vocab) (weights
once per launch, activations in, logits out). Launch durations come from HIP
events recorded on the launch stream around every call.

Prints one JSON line (see the repository's design notes for field meanings).
Other workloads for local measurements: --workload w8a8 (the 129280 x 7168
head, W8A8 at rows 1 and 16) or --rows to change the row sweep.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "fp8_gemv_155136x8192_counters.json")
KERNEL_SOURCES = [os.path.join(ROOT, "quantized_weight_decode_amd", "csrc", f)
                  for f in ("fp8_gemv.hip", "qhead_device.h")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--rows", type=str, default="1,2,4,8,16")
    ap.add_argument("--workload", choices=["fp8", "w8a8"], default="fp8")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target duration of the oracle CPU baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only copy 1 GiB device to device (for rocprofv3 FETCH_SIZE/WRITE_SIZE "
                         "calibration) and exit")
    return ap.parse_args()


def build_head(cfg_index: int, qh, torch):
    """Generate the seeded head chunk by chunk and quantize it on the device."""
    import synth

    cfg = synth.CONFIGS[cfg_index]
    dev = torch.device("cuda:0")
    codes = torch.empty((cfg.vocab, cfg.hidden), dtype=torch.uint8, device=dev)
    scales = torch.empty((cfg.vocab,), dtype=torch.float32, device=dev)
    for lo, hi, wf in synth.iter_weight_chunks(cfg_index):
        wd = torch.from_numpy(wf).to(dev)
        qh.quantize_fp8_rows(wd, codes=codes[lo:hi], scales=scales[lo:hi])
        del wd
    torch.cuda.synchronize()
    return cfg, codes, scales


def algorithmic_bytes(fmt: str, V: int, H: int, R: int) -> int:
    w = V * H + 4 * V
    act = R * (2 * H + 2 * V)
    if fmt == "w8a8":
        # quantized activations written and read back once per call
        act += 2 * R * (H + 4)
    return w + act


def cpu_baseline(cfg_index: int, rows: list[int], target_s: float):
    """The oracle timed on a bounded sample of the same workload (vocab rows
    [0, n) of the same head, the same row sweep); returns GB/s of that sample
    in the workload's algorithmic bytes."""
    import oracle
    import synth

    cfg = synth.CONFIGS[cfg_index]
    x = synth.activations_bf16(cfg_index, max(rows), max_rows=max(rows))

    def run(n: int) -> float:
        wf = synth.weight_rows_f32(cfg_index, 0, n)
        w, s = oracle.prep_fp8_rows(wf)
        vidx = np.arange(n, dtype=np.int64)
        t0 = time.perf_counter()
        for R in rows:
            if cfg.fmt == "w8a8":
                xq, sa = oracle.quant_act_e4m3(x[:R])
                oracle.w8a8_ref(w, s, xq, sa, vidx)
            else:
                oracle.fp8_rowscale_ref(w, s, x[:R], vidx)
        return time.perf_counter() - t0

    n = 256
    t = run(n)
    n = int(min(cfg.vocab, max(n, n * target_s / max(t, 1e-3))))
    t = run(n)
    fmt = "w8a8" if cfg.fmt == "w8a8" else "fp8"
    bytes_ = sum(algorithmic_bytes(fmt, n, cfg.hidden, R) for R in rows)
    return {
        "value": round(bytes_ / t / 1e9, 4),
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"vocab rows [0, {n}) of the same head, rows {rows}, {t:.1f} s "
                  f"(binary64 dequantize-then-dot, OpenMP)",
        "rows_per_s_full_head": round(sum(rows) * n / cfg.vocab / t, 6),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported "
              "(the head shards by vocab across GPUs; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        # A plain copy of known size: the counters of this one kernel give the
        # factor between FETCH_SIZE / WRITE_SIZE readings and bytes moved.
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n}), flush=True)
        return

    import quantized_weight_decode_amd as qh

    rows = [int(r) for r in args.rows.split(",")]
    cfg_index = 2 if args.workload == "fp8" else 3
    t_prep = time.perf_counter()
    cfg, codes, scales = build_head(cfg_index, qh, torch)
    t_prep = time.perf_counter() - t_prep
    V, H = cfg.vocab, cfg.hidden
    import synth

    xall = synth.activations_bf16(cfg_index, max(rows), max_rows=max(rows))
    dev = torch.device("cuda:0")
    xs = {R: torch.from_numpy(xall[:R].view(np.int16)).to(dev).view(torch.bfloat16) for R in rows}
    outs = {R: torch.empty((R, V), dtype=torch.bfloat16, device=dev) for R in rows}
    ws = qh.w8a8_workspace(H, dev) if args.workload == "w8a8" else None

    def call(R):
        if args.workload == "w8a8":
            qh.w8a8(codes, scales, xs[R], out=outs[R], workspace=ws)
        else:
            qh.fp8_rowscale(codes, scales, xs[R], out=outs[R])

    for _ in range(args.warmup):
        for R in rows:
            call(R)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in rows] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for k in range(args.steps):
        for i, R in enumerate(rows):
            evs[k][i][0].record(stream)
            call(R)
            evs[k][i][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0

    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    per_rows = {}
    for i, R in enumerate(rows):
        d = np.array([evs[k][i][0].elapsed_time(evs[k][i][1]) for k in range(args.steps)])
        b = algorithmic_bytes(args.workload, V, H, R)
        per_rows[str(R)] = {"us_median": round(float(np.median(d)) * 1e3, 2),
                            "us_min": round(float(d.min()) * 1e3, 2),
                            "GBps": round(b / (np.median(d) * 1e-3) / 1e9, 1),
                            "pct_peak": round(b / (np.median(d) * 1e-3) / 1e9 / HBM_PEAK_GBS * 100,
                                              1),
                            "rows_per_s": round(R / (np.median(d) * 1e-3), 1)}
    step_bytes = sum(algorithmic_bytes(args.workload, V, H, R) for R in rows)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    launch_ms = np.array([[evs[k][i][0].elapsed_time(evs[k][i][1]) for i in range(len(rows))]
                          for k in range(args.steps)])
    mean_launch_bytes = step_bytes / len(rows)
    achieved = mean_launch_bytes / (launch_ms.mean() * 1e-3) / 1e9

    traffic = None
    if os.path.exists(PROFILE_COUNTERS) and args.workload == "fp8" and rows == [1, 2, 4, 8, 16]:
        with open(PROFILE_COUNTERS) as f:
            prof = json.load(f)
        if prof.get("kernel_source_hash") == kernel_source_hash():
            traffic = prof.get("hbm_bytes_per_launch")

    line = {
        "metric": "achieved HBM GB/s (% of peak) & logits rows/sec, 1.27 GB FP8 head, rows 1..16"
        if args.workload == "fp8" else "achieved HBM GB/s, W8A8 head 129280x7168",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 x bf16 -> f32 acc, bf16 out" if args.workload == "fp8"
        else "fp8e4m3 x fp8e4m3 -> f32 acc, bf16 out",
        "data": "synthetic (seeded N(0,0.015) weights quantized per row to E4M3, N(0,1) BF16 x)",
        "config": {"workload": cfg.label, "vocab": V, "hidden": H, "rows_per_step": rows,
                   "launches_per_step": len(rows), "weight_bytes": V * H,
                   "pct_of_hbm_peak": round(value / HBM_PEAK_GBS * 100, 2),
                   "rows_per_s": round(sum(rows) / (ms_per_step * 1e-3), 1),
                   "per_rows": per_rows, "wall_s_timed": round(wall, 3),
                   "head_prep_s": round(t_prep, 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "fp8_gemv_kernel (mean over the step's launches)",
                     "avg_launch_us": round(float(launch_ms.mean()) * 1e3, 2)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg_index, rows, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
