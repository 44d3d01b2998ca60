"""Benchmark: achieved HBM GB/s and logits rows/s of the quantized LM head.

Workload (default, --workload fp8): the 1.27 GB FP8 head -- vocab 155136 x
hidden 8192 E4M3 weights (N(0, 0.015) draws quantized per row on the device,
F32 row scales), BF16 activations from N(0, 1) -- decoded at rows 1, 2, 4, 8
and 16. One step is one pass of the head path over that batch: five
qhead_fp8_rowscale calls, each one weight pass. The weights are resident in
HBM before timing starts.

value = algorithmic bytes of the step / step time, where a call's
algorithmic bytes are the weight bytes once per weight pass plus R * (2 *
hidden + 2 * vocab) (activations in, logits out) plus, for W8A8 and Q6_K, the
quantized activations written and read back once. Call durations come from
HIP events recorded on the launch stream around every call.

Other workloads:
  --workload fp8_rows64   the same head at 64 rows (four 16-row passes)
  --workload fp8_32000    32000 x 4096 FP8 head, outlier channels, rows 1, 2,
                          3, 4, 8, 16 and 40 (16 + 16 + 8)
  --workload fp8_8192     8192 x 1024 FP8 head, one row
  --workload w8a8         129280 x 7168 W8A8 head, calls of 1, 16, 128 and
                          300 rows (activation quantization + GEMV per call)
  --workload nvfp4        129280 x 7168 NVFP4 W4A16 at rows 1, 2, 4, 8, 16
  --workload q6k          129280 x 7168 Q6_K with q8_1 activations, rows 1..8
  --workload dequant      load-time NVFP4 -> BF16 of that head
  --workload w8a8_silu    W8A8 down projection of bf16(silu(gate) * up),
                          output 7168 x FFN width 18432, calls of 1, 16, 128
Heads smaller than 768 MiB are held in several copies that the calls rotate
over (at least 768 MiB in all, three times the 256 MiB last-level cache), so
that no call finds its weights in a cache, as when a decode step walks the
layers of a model.
--rows changes the row sweep. Prints one JSON line; config.read_ceiling is
the library's plain streaming read (qhead_stream_read) over the same weight
bytes, and every row count's pct_read_ceiling compares its GB/s with it.
Every row count also carries its roofs: the HBM time of its bytes at 8 TB/s
and the issue time of its VALU (or MFMA) work at the chip's peak rate (see
compute_roof_us); pct_of_bound is the larger roof over the measured time.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from dataclasses import dataclass

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402  (seeded input shapes; no method arithmetic)

HBM_PEAK_GBS = 8000.0
CSRC = os.path.join(ROOT, "quantized_weight_decode_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
ROTATE_BYTES = 768 << 20   # weight copies rotated up to this many bytes
# MI355X: 256 CUs x 4 SIMDs at 2.4 GHz; a SIMD issues one wave64 VALU
# instruction every 4 cycles (64 lane-operations per CU per cycle) and a
# 16x16x32 BF16 MFMA every 16 cycles.
CUS, SIMDS_PER_CU, CLOCK_HZ = 256, 4, 2.4e9
VALU_LANE_OPS_PER_S = CUS * 64 * CLOCK_HZ
MFMA_16X16X32_CYCLES = 16


@dataclass(frozen=True)
class Workload:
    cfg: int
    rows: str
    kernel: str
    sources: tuple
    counters: str
    metric: str
    dtype: str
    data: str


_W002 = "synthetic (seeded N(0,0.02) weights quantized on the device, N(0,1) BF16 x)"
_FP8_SRC = ("fp8_gemv.hip", "qhead_device.h")
_FP8_DTYPE = "fp8e4m3 x bf16 -> f32 acc, bf16 out"
_W8_SRC = ("w8a8_gemv.hip", "act_quant.hip", "quant_common.h", "qhead_device.h", "lds_dma.h")
WORKLOADS = {
    "fp8": Workload(
        synth.FP8_155136X8192, "1,2,4,8,16", "fp8_gemv_kernel", _FP8_SRC,
        "fp8_gemv_155136x8192_counters.json",
        "achieved HBM GB/s (% of peak) & logits rows/sec, 1.27 GB FP8 head, rows 1..16",
        _FP8_DTYPE,
        "synthetic (seeded N(0,0.015) weights quantized per row to E4M3, N(0,1) BF16 x)"),
    "fp8_rows64": Workload(
        synth.FP8_155136X8192, "64", "fp8_gemv_kernel", _FP8_SRC,
        "fp8_gemv_155136x8192_rows64_counters.json",
        "achieved HBM GB/s & logits rows/sec, 1.27 GB FP8 head, 64 rows in 16-row passes",
        _FP8_DTYPE,
        "synthetic (seeded N(0,0.015) weights quantized per row to E4M3, N(0,1) BF16 x)"),
    "fp8_32000": Workload(
        synth.FP8_32000X4096, "1,2,3,4,8,16,40", "fp8_gemv_kernel", _FP8_SRC,
        "fp8_gemv_32000x4096_counters.json",
        "achieved HBM GB/s & logits rows/sec, FP8 head 32000x4096, rows 1..16 and 40",
        _FP8_DTYPE,
        "synthetic (seeded N(0,0.02) weights quantized per row to E4M3, N(0,1) BF16 x with "
        "41 outlier channels x20)"),
    "fp8_8192": Workload(
        synth.FP8_8192X1024, "1", "fp8_gemv_kernel", _FP8_SRC,
        "fp8_gemv_8192x1024_counters.json",
        "achieved HBM GB/s & logits rows/sec, FP8 head 8192x1024, one row",
        _FP8_DTYPE, _W002),
    "w8a8": Workload(
        synth.W8A8_129280X7168, "1,16,128,300",
        "w8a8_valu_kernel / w8a8_mfma_kernel + quant_act_e4m3_kernel (per call)", _W8_SRC,
        "w8a8_129280x7168_counters.json",
        "achieved HBM GB/s, W8A8 head 129280x7168, calls of 1/16/128/300 rows",
        "fp8e4m3 x fp8e4m3 (exact products, bf16 operands) -> f32 acc, bf16 out", _W002),
    "nvfp4": Workload(
        synth.NVFP4_Q6K_129280X7168, "1,2,4,8,16", "nvfp4_gemv_kernel",
        ("nvfp4_gemv.hip", "qhead_device.h"),
        "nvfp4_gemv_129280x7168_counters.json",
        "achieved HBM GB/s, NVFP4 W4A16 head 129280x7168, rows 1..16",
        "e2m1 x e4m3 block scale x bf16 -> f32 acc, bf16 out", _W002),
    "q6k": Workload(
        synth.NVFP4_Q6K_129280X7168, "1,2,4,8", "q6k_gemv_kernel + quant_q8_1_kernel (per call)",
        ("q6k_gemv.hip", "act_quant.hip", "quant_common.h", "qhead_device.h", "lds_dma.h"),
        "q6k_gemv_129280x7168_counters.json",
        "achieved HBM GB/s, Q6_K head 129280x7168 with q8_1 activations, rows 1..8",
        "int6 x int8 -> i32 dot4, f32 scales, bf16 out", _W002),
    "w8a8_silu": Workload(
        synth.SILU_DOWN_7168X18432, "1,16,128",
        "w8a8_valu_split_kernel / w8a8_mfma_kernel + silu_slice_max/quant kernels (per call)",
        ("w8a8_gemv.hip", "silu_quant.hip", "quant_common.h", "qhead_device.h", "lds_dma.h"),
        "w8a8_silu_7168x18432_counters.json",
        "achieved HBM GB/s, W8A8 SiLU down projection 7168x18432, calls of 1/16/128 rows",
        "bf16 silu(gate)*up -> fp8e4m3 x fp8e4m3 -> f32 acc, bf16 out",
        "synthetic (seeded N(0,0.02) weights quantized per row on the device, gate N(0,1.5^2) "
        "and up N(0,1) BF16)"),
    "dequant": Workload(
        synth.NVFP4_Q6K_129280X7168, "0", "dequant_fp4_kernel<false>",
        ("dequant.hip", "qhead_device.h"),
        "dequant_nvfp4_129280x7168_counters.json",
        "achieved HBM GB/s, load-time NVFP4 -> BF16 of the 129280x7168 head",
        "e2m1 x e4m3 x f32 global -> bf16", _W002),
}
FP8_FAMILY = ("fp8", "fp8_rows64", "fp8_32000", "fp8_8192")
E4M3_HEADS = FP8_FAMILY + ("w8a8", "w8a8_silu")
# rows per weight pass (the library's row chunks)
PASS_ROWS = {"fp8": 16, "w8a8": 128, "nvfp4": 16, "q6k": 8}


def fmt_of(name: str) -> str:
    if name in FP8_FAMILY:
        return "fp8"
    if name in ("w8a8", "w8a8_silu"):
        return "w8a8"
    return name


def weight_copies(name: str, V: int, H: int) -> int:
    """Copies of the weights the calls rotate over (at least ROTATE_BYTES)."""
    wbytes = algorithmic_bytes(name, V, H, 0)
    return max(1, min(128, -(-ROTATE_BYTES // wbytes)))


def compute_roof_us(name: str, V: int, H: int, R: int):
    """(issue time in us, "valu" or "mfma") of the arithmetic one call of R
    rows must issue, at the chip's peak issue rate, from the kernels' inner
    loops per weight byte and pass (the rest -- trees, stores, quantizers --
    is left out, so this is a lower bound of the compute time):
      FP8 W8A16, W8A8 below 16 rows: per BF16 pair of weights one half-rate
        convert (2 lane-slots) and one v_dot2_f32_bf16 per row: (R + 2) / 2
        lane-slots per weight byte;
      W8A8 at 16..128 rows: 32 * ceil(R / 16) 16x16x32 BF16 MFMAs per 16 vocab
        rows and 256 k, 16 cycles each on one of the 1024 SIMDs;
      NVFP4: per byte (one pair) a 2-slot convert, R dot2 and R / 8 block FMAs,
        plus about 0.3 slots of block-scale decode: 2.3 + 1.125 R;
      Q6_K: per 16 weights 24 slots of 6-bit decode and scale, and per row
        4 v_dot4_i32_i8, a convert, a multiply and an FMA: 1.5 + 0.4375 R
        lane-slots per weight;
    None for the dequant (no arithmetic to speak of)."""
    fmt = fmt_of(name)
    if fmt == "dequant" or R == 0:
        return None
    step = PASS_ROWS[fmt]
    chunks = [min(step, R - d) for d in range(0, R, step)]
    valu = mfma_cycles = 0.0
    for m in chunks:
        if fmt in ("fp8", "w8a8") and not (fmt == "w8a8" and m >= 16):
            valu += V * H / 2 * (m + 2)
        elif fmt == "w8a8":
            mfma_cycles += -(-V // 16) * -(-H // 256) * 32 * -(-m // 16) * MFMA_16X16X32_CYCLES
        elif fmt == "nvfp4":
            valu += V * H / 2 * (2.3 + 1.125 * m)
        elif fmt == "q6k":
            valu += V * H * (1.5 + 0.4375 * m)
    valu_us = valu / VALU_LANE_OPS_PER_S * 1e6
    mfma_us = mfma_cycles / (CUS * SIMDS_PER_CU * CLOCK_HZ) * 1e6
    return valu_us + mfma_us, ("mfma" if mfma_us > valu_us else "valu")


def kernel_source_hash(wl: Workload) -> str:
    h = hashlib.sha256()
    for name in wl.sources:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rows", type=str, default=None)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="fp8")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target duration of the oracle CPU baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only copy 1 GiB device to device (for rocprofv3 FETCH_SIZE/WRITE_SIZE "
                         "calibration) and exit")
    return ap.parse_args()


def nvfp4_global(amax: float) -> float:
    """The head's NVFP4 global multiplier: fl32(amax / 2688), 2688 = 6 * 448."""
    return float(np.float32(amax) / np.float32(2688.0))


def build_head(name: str, cfg, qh, torch):
    """Generate the seeded head chunk by chunk and quantize it on the device;
    E4M3 heads smaller than ROTATE_BYTES are cloned into rotation copies."""
    dev = torch.device("cuda:0")
    V, H = cfg.vocab, cfg.hidden
    if name in E4M3_HEADS:
        codes = torch.empty((V, H), dtype=torch.uint8, device=dev)
        scales = torch.empty((V,), dtype=torch.float32, device=dev)
        for lo, hi, wf in synth.iter_weight_chunks(cfg.index):
            wd = torch.from_numpy(wf).to(dev)
            qh.quantize_fp8_rows(wd, codes=codes[lo:hi], scales=scales[lo:hi])
            del wd
        torch.cuda.synchronize()
        copies = [(codes, scales)] + [(codes.clone(), scales.clone())
                                      for _ in range(weight_copies(name, V, H) - 1)]
        torch.cuda.synchronize()
        return {"copies": copies}
    wf = torch.empty((V, H), dtype=torch.float32, device=dev)
    for lo, hi, chunk in synth.iter_weight_chunks(cfg.index):
        wf[lo:hi].copy_(torch.from_numpy(chunk))
    if name == "q6k":
        head = {"blocks": qh.quantize_q6k_rows(wf)}
    else:
        g = nvfp4_global(float(wf.abs().max().item()))
        wp, bs = qh.quantize_nvfp4_rows(wf, g)
        head = {"wp": wp, "bs": bs, "g": g}
    torch.cuda.synchronize()
    del wf
    torch.cuda.empty_cache()
    return head


def algorithmic_bytes(name: str, V: int, H: int, R: int) -> int:
    """Bytes one call must move: weights once per weight pass (one pass per
    PASS_ROWS rows), activations in, logits out, and quantized activations
    written and read back where the format has them. R = 0 gives the bytes of
    one weight pass."""
    fmt = fmt_of(name)
    passes = max(1, -(-R // PASS_ROWS[fmt])) if fmt in PASS_ROWS else 1
    io = R * (2 * H + 2 * V)
    if fmt == "fp8":
        return passes * (V * H + 4 * V) + io
    if name == "w8a8":
        return passes * (V * H + 4 * V) + io + 2 * R * (H + 4)
    if name == "w8a8_silu":
        # gate and up read (2 x 2 bytes per value) instead of one BF16 x
        return passes * (V * H + 4 * V) + io + R * 2 * H + 2 * R * (H + 4)
    if name == "nvfp4":
        return passes * (V * H // 2 + V * H // 16) + io
    if name == "q6k":
        return passes * V * (H // 256) * 210 + io + 2 * R * (H // 32) * 36
    if name == "dequant":
        return V * H // 2 + V * H // 16 + 2 * V * H
    raise ValueError(name)


def measure_read_ceiling(name: str, head, qh, torch, stream, warmup: int = 3,
                         timed: int = 10) -> dict:
    """The streaming-read yardstick on the workload's own weight bytes: the
    library's plain read kernel (qhead_stream_read) over the main weight
    buffer, median of `timed` calls (rotating over the weight copies where
    the workload rotates them, so that no read is served from cache)."""
    if "copies" in head:
        bufs = [w for w, _ in head["copies"]]
    else:
        bufs = [head["blocks" if name == "q6k" else "wp"]]
    nbytes = bufs[0].numel() * bufs[0].element_size()
    out = torch.zeros((qh.STREAM_READ_WORDS,), dtype=torch.int32, device=bufs[0].device)
    # every call rewrites the words of the workgroups it launches: the raw
    # entry point is timed, without the binding's clear of the output
    fn, sptr = qh.lib().qhead_stream_read, stream.cuda_stream

    def read(i):
        st = fn(bufs[i % len(bufs)].data_ptr(), nbytes, out.data_ptr(), sptr)
        if st != 0:
            raise RuntimeError(f"qhead_stream_read: {qh.status_string(st)}")

    for i in range(warmup):
        read(i)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(timed)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        read(i)
        b.record(stream)
    torch.cuda.synchronize()
    us = float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e3
    return {"GBps": round(nbytes / (us * 1e-6) / 1e9, 1), "us_median": round(us, 2),
            "bytes": nbytes, "kernel": "stream_read_kernel (qhead_stream_read)"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(name: str, cfg, rows: list[int], target_s: float):
    """The oracle timed on a bounded sample of the same workload (vocab rows
    [0, n) of the same head, the same row sweep); returns GB/s of that sample
    in the workload's algorithmic bytes."""
    import oracle
    import synth

    x = synth.activations_bf16(cfg.index, max(max(rows), 1), max_rows=max(max(rows), 1))
    if name == "w8a8_silu":
        gate, up = synth.gate_up_bf16(cfg.index, max(rows), max_rows=max(rows))

    def run(n: int) -> float:
        wf = synth.weight_rows_f32(cfg.index, 0, n)
        vidx = np.arange(n, dtype=np.int64)
        if name in E4M3_HEADS:
            w, s = oracle.prep_fp8_rows(wf)
        elif name == "q6k":
            blocks = oracle.prep_q6k_rows(wf)
        else:
            g = oracle.nvfp4_global(float(np.abs(wf).max()))
            wp, bs = oracle.prep_nvfp4_rows(wf, g)
        t0 = time.perf_counter()
        for R in rows:
            if name in FP8_FAMILY:
                oracle.fp8_rowscale_ref(w, s, x[:R], vidx)
            elif name == "w8a8":
                xq, sa = oracle.quant_act_e4m3(x[:R])
                oracle.w8a8_ref(w, s, xq, sa, vidx)
            elif name == "w8a8_silu":
                xq, sa, _ = oracle.quant_act_silu_e4m3(gate[:R], up[:R])
                oracle.w8a8_ref(w, s, xq, sa, vidx)
            elif name == "nvfp4":
                oracle.nvfp4_ref(wp, bs, g, x[:R], vidx)
            elif name == "q6k":
                oracle.q6k_ref(blocks, oracle.quant_q8_1(x[:R]), cfg.hidden, vidx)
            else:
                oracle.dequant_nvfp4_bf16(wp, bs, g)
        return time.perf_counter() - t0

    # Size the sample in two steps (about 1 s, then the target): a tiny first
    # run overstates the time per vocab row (thread start-up, fixed costs).
    n, t = 256, 0.0
    for goal in (1.0, target_s):
        t = run(n)
        n = int(min(cfg.vocab, max(n, n * goal / max(t, 1e-3))))
    t = run(n)
    bytes_ = sum(algorithmic_bytes(name, n, cfg.hidden, R) for R in rows)
    what = "NVFP4 -> BF16 of those rows" if name == "dequant" else f"rows {rows}"
    return {
        "value": round(bytes_ / t / 1e9, 4),
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "nproc": os.cpu_count(),
        "cores_available": len(os.sched_getaffinity(0)),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"vocab rows [0, {n}) of the same head, {what}, {t:.1f} s "
                  f"(binary64 oracle, OpenMP)",
        "rows_per_s_full_head": round(sum(rows) * n / cfg.vocab / t, 6),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the head would be split by vocab rows across GPUs, one launch per GPU)", file=sys.stderr)
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
    import synth

    name = args.workload
    wl = WORKLOADS[name]
    cfg = synth.CONFIGS[wl.cfg]
    rows = [int(r) for r in (args.rows or wl.rows).split(",")]
    if name == "dequant":
        rows = [0]
    t_prep = time.perf_counter()
    head = build_head(name, cfg, qh, torch)
    t_prep = time.perf_counter() - t_prep
    V, H = cfg.vocab, cfg.hidden

    dev = torch.device("cuda:0")
    nx = max(max(rows), 1)
    xall = synth.activations_bf16(cfg.index, nx, max_rows=nx)
    xs = {R: torch.from_numpy(xall[:R].view(np.int16)).to(dev).view(torch.bfloat16) for R in rows}
    if name == "w8a8_silu":
        g_all, u_all = synth.gate_up_bf16(cfg.index, nx, max_rows=nx)
        gd = torch.from_numpy(g_all.view(np.int16)).to(dev).view(torch.bfloat16)
        ud = torch.from_numpy(u_all.view(np.int16)).to(dev).view(torch.bfloat16)
    ncall = [0]
    if name == "dequant":
        outs = {0: torch.empty((V, H), dtype=torch.bfloat16, device=dev)}
    else:
        outs = {R: torch.empty((R, V), dtype=torch.bfloat16, device=dev) for R in rows}
    ws = None
    if name in ("w8a8", "w8a8_silu"):
        ws = qh.w8a8_workspace(H, dev)
    elif name == "q6k":
        ws = torch.empty((qh.q6k_workspace_bytes(H),), dtype=torch.uint8, device=dev)

    def call(R):
        if "copies" in head:
            w, sc = head["copies"][ncall[0] % len(head["copies"])]
            ncall[0] += 1
        if name in FP8_FAMILY:
            qh.fp8_rowscale(w, sc, xs[R], out=outs[R])
        elif name == "w8a8":
            qh.w8a8(w, sc, xs[R], out=outs[R], workspace=ws)
        elif name == "w8a8_silu":
            qh.w8a8_silu(w, sc, gd[:R], ud[:R], out=outs[R], workspace=ws)
        elif name == "nvfp4":
            qh.nvfp4(head["wp"], head["bs"], xs[R], head["g"], out=outs[R])
        elif name == "q6k":
            qh.q6k(head["blocks"], xs[R], out=outs[R], workspace=ws)
        else:
            qh.dequant_nvfp4_bf16(head["wp"], head["bs"], head["g"], out=outs[0])

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
    launch_ms = np.array([[evs[k][i][0].elapsed_time(evs[k][i][1]) for i in range(len(rows))]
                          for k in range(args.steps)])
    per_rows = {}
    for i, R in enumerate(rows):
        d = launch_ms[:, i]
        b = algorithmic_bytes(name, V, H, R)
        gbs = b / (np.median(d) * 1e-3) / 1e9
        us = float(np.median(d)) * 1e3
        hbm_us = b / (HBM_PEAK_GBS * 1e9) * 1e6
        roof = compute_roof_us(name, V, H, R)
        entry = {
            "us_median": round(us, 2),
            "us_min": round(float(d.min()) * 1e3, 2),
            "us_p90": round(float(np.percentile(d, 90)) * 1e3, 2),
            "GBps": round(gbs, 1),
            "pct_peak": round(gbs / HBM_PEAK_GBS * 100, 1),
            "rows_per_s": round(R / (np.median(d) * 1e-3), 1),
            "weight_passes": max(1, -(-R // PASS_ROWS.get(fmt_of(name), 1 << 30))),
            "hbm_roof_us": round(hbm_us, 2)}
        bound, bound_us = "hbm", hbm_us
        if roof is not None:
            entry[f"{roof[1]}_roof_us"] = round(roof[0], 2)
            if roof[0] > hbm_us:
                bound, bound_us = roof[1], roof[0]
        entry["bound"] = bound
        entry["pct_of_bound"] = round(bound_us / us * 100, 1)
        per_rows["head" if name == "dequant" else str(R)] = entry
    step_bytes = sum(algorithmic_bytes(name, V, H, R) for R in rows)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    mean_launch_bytes = step_bytes / len(rows)
    achieved = mean_launch_bytes / (launch_ms.mean() * 1e-3) / 1e9

    read_ceiling = measure_read_ceiling(name, head, qh, torch, stream)
    for v in per_rows.values():
        v["pct_read_ceiling"] = round(v["GBps"] / read_ceiling["GBps"] * 100, 1)

    traffic = None
    counters = os.path.join(PROFILES, wl.counters)
    if os.path.exists(counters) and rows == [int(r) for r in wl.rows.split(",")]:
        with open(counters) as f:
            prof = json.load(f)
        if prof.get("kernel_source_hash") == kernel_source_hash(wl):
            traffic = prof.get("hbm_bytes_per_launch")

    config = {"workload": cfg.label if name != "dequant" else
              f"nvfp4 -> bf16 dequant of the {V}x{H} head",
              "vocab": V, "hidden": H, "rows_per_step": rows if name != "dequant" else [],
              "launches_per_step": len(rows), "weight_bytes": algorithmic_bytes(name, V, H, 0),
              "pct_of_hbm_peak": round(value / HBM_PEAK_GBS * 100, 2),
              "weight_copies": len(head.get("copies", [None])),
              "per_rows": per_rows, "read_ceiling": read_ceiling,
              "wall_s_timed": round(wall, 3),
              "head_prep_s": round(t_prep, 1)}
    if name != "dequant":
        config["rows_per_s"] = round(sum(rows) / (ms_per_step * 1e-3), 1)
    line = {
        "metric": wl.metric,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": wl.data,
        "config": config,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": f"{wl.kernel} (mean over the step's calls)",
                     "avg_launch_us": round(float(launch_ms.mean()) * 1e3, 2),
                     # per call: the binding roof (HBM, or the VALU / MFMA issue
                     # time where that is longer) and the fraction of it reached
                     "per_rows": {k: {"bound": v["bound"], "frac": round(v["pct_of_bound"] / 100, 4),
                                      "frac_hbm": round(v["pct_peak"] / 100, 4)}
                                  for k, v in per_rows.items()}},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(name, cfg, rows, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
