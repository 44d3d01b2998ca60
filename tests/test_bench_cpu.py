"""Host-side checks of bench.py (no GPU): the multi-GPU refusal, the
algorithmic byte counts each workload is measured against, and the workload
table that names the kernel sources behind each profile summary."""

import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_algorithmic_bytes():
    V, H = 155136, 8192
    # FP8 head: codes once, one F32 scale per row, BF16 activations in and logits out
    assert bench.algorithmic_bytes("fp8", V, H, 1) == V * H + 4 * V + 2 * H + 2 * V
    assert bench.algorithmic_bytes("fp8", V, H, 16) - bench.algorithmic_bytes("fp8", V, H, 0) \
        == 16 * (2 * H + 2 * V)
    # W8A8 adds the E4M3 activations and their scale, written then read back
    assert bench.algorithmic_bytes("w8a8", V, H, 4) - bench.algorithmic_bytes("fp8", V, H, 4) \
        == 2 * 4 * (H + 4)
    V, H = 129280, 7168
    # NVFP4: half a byte per weight plus one E4M3 scale per 16 weights
    assert bench.algorithmic_bytes("nvfp4", V, H, 0) == V * H // 2 + V * H // 16
    # Q6_K: 210 bytes per 256 weights; q8_1 blocks of 36 bytes per 32 values, twice
    assert bench.algorithmic_bytes("q6k", V, H, 0) == V * (H // 256) * 210
    assert bench.algorithmic_bytes("q6k", V, H, 1) - bench.algorithmic_bytes("q6k", V, H, 0) \
        == 2 * H + 2 * V + 2 * (H // 32) * 36
    # dequant: read codes and scales, write BF16
    assert bench.algorithmic_bytes("dequant", V, H, 0) == V * H // 2 + V * H // 16 + 2 * V * H


def test_workload_table():
    for name, wl in bench.WORKLOADS.items():
        cfg = synth.CONFIGS[wl.cfg]
        assert cfg.vocab > 0 and cfg.hidden > 0, name
        for src in wl.sources:
            assert os.path.exists(os.path.join(bench.CSRC, src)), (name, src)
        assert len(bench.kernel_source_hash(wl)) == 16
        assert os.path.exists(os.path.join(ROOT, "profiles", wl.counters)), name
    # the default workload is the 1.27 GB FP8 head at rows 1..16
    fp8 = bench.WORKLOADS["fp8"]
    cfg = synth.CONFIGS[fp8.cfg]
    assert (cfg.vocab, cfg.hidden) == (155136, 8192)
    assert [int(r) for r in fp8.rows.split(",")] == [1, 2, 4, 8, 16]


def test_compute_roofs():
    """The per-call compute roofs bench.py reports next to the HBM roof: the
    VALU issue time of (R + 2)/2 lane-slots per FP8 weight byte at 64
    lane-operations per CU per cycle, and for W8A8 at 16+ rows the matrix-unit
    time of 32 * ceil(R/16) 16-cycle MFMAs per 16 vocab rows and 256 k."""
    V, H = 155136, 8192
    rate = 256 * 64 * 2.4e9
    us, unit = bench.compute_roof_us("fp8", V, H, 16)
    assert unit == "valu" and abs(us - V * H / 2 * 18 / rate * 1e6) < 1e-6
    us64, _ = bench.compute_roof_us("fp8_rows64", V, H, 64)
    assert abs(us64 - 4 * us) < 1e-6  # four 16-row passes
    V, H = 129280, 7168
    us, unit = bench.compute_roof_us("w8a8", V, H, 128)
    mfma = (V // 16) * (H // 256) * 32 * 8 * 16 / (1024 * 2.4e9) * 1e6
    assert unit == "mfma" and abs(us - mfma) < 1e-6
    us1, unit1 = bench.compute_roof_us("w8a8", V, H, 1)
    assert unit1 == "valu" and abs(us1 - V * H / 2 * 3 / rate * 1e6) < 1e-6
    # 300 rows = 128 + 128 + 44: three passes, the last of 3 row tiles
    us300, _ = bench.compute_roof_us("w8a8", V, H, 300)
    assert abs(us300 - mfma * (8 + 8 + 3) / 8) < 1e-6
    assert bench.compute_roof_us("dequant", V, H, 0) is None


def test_weight_copies_exceed_the_cache():
    for name in bench.E4M3_HEADS:
        cfg = synth.CONFIGS[bench.WORKLOADS[name].cfg]
        n = bench.weight_copies(name, cfg.vocab, cfg.hidden)
        wbytes = bench.algorithmic_bytes(name, cfg.vocab, cfg.hidden, 0)
        assert n == 1 or n * wbytes >= bench.ROTATE_BYTES, name
        assert n * wbytes >= min(bench.ROTATE_BYTES, wbytes)
    cfg = synth.CONFIGS[synth.FP8_32000X4096]
    assert bench.weight_copies("fp8_32000", cfg.vocab, cfg.hidden) >= 3
