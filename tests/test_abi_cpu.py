"""C-ABI checks that need no GPU: the library loads, exports every function
include/qhead.h declares, rejects invalid arguments before touching the
device, and plans row chunks as the pages' chunk loops do (16 rows per FP8
W8A16 pass, 128 per W8A8 call, 16 per NVFP4 pass, 8 per Q6_K pass)."""

import ctypes
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def qh():
    lib = os.path.join(ROOT, "quantized_weight_decode_amd", "libqhead.so")
    if not os.path.exists(lib):
        subprocess.run(["python", os.path.join(ROOT, "quantized_weight_decode_amd", "build.py")],
                       check=True)
    import quantized_weight_decode_amd as m

    return m


# fake device addresses: never dereferenced, the calls return before any HIP call
A16 = 0x10000
A256 = 0x20000
MIS = 0x10001


def test_exports_every_declared_function(qh):
    names = qh.header_functions()
    assert len(names) == 23
    for n in names:
        assert hasattr(qh.lib(), n), n
    out = subprocess.run(["nm", "-D", "--defined-only", qh.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert set(names) <= exported


def test_status_strings(qh):
    for st in range(-8, 1):
        assert qh.status_string(st) and qh.status_string(st) != "unknown status"
    assert qh.status_string(-99) == "unknown status"


def test_plan_chunks(qh):
    assert qh.plan_chunks(qh.FMT_FP8, 40) == [16, 16, 8]
    assert qh.plan_chunks(qh.FMT_FP8, 64) == [16, 16, 16, 16]
    assert qh.plan_chunks(qh.FMT_FP8, 16) == [16]
    assert qh.plan_chunks(qh.FMT_FP8, 1) == [1]
    assert qh.plan_chunks(qh.FMT_W8A8, 300) == [128, 128, 44]
    assert qh.plan_chunks(qh.FMT_W8A8, 128) == [128]
    assert qh.plan_chunks(qh.FMT_NVFP4, 8) == [8]
    assert qh.plan_chunks(qh.FMT_NVFP4, 40) == [16, 16, 8]
    assert qh.plan_chunks(qh.FMT_Q6K, 13) == [8, 5]
    assert qh.plan_chunks(qh.FMT_Q6K, 0) == []
    L = qh.lib()
    assert L.qhead_plan_chunks(qh.FMT_FP8, -1, None, 0) == -2
    assert L.qhead_plan_chunks(9, 4, None, 0) == -5
    buf = (ctypes.c_int32 * 2)()
    # a short buffer still returns the full count and fills what fits
    assert L.qhead_plan_chunks(qh.FMT_FP8, 50, buf, 2) == 4
    assert list(buf) == [16, 16]
    assert [qh.max_rows_per_launch(f) for f in range(4)] == [16, 128, 16, 8]
    assert L.qhead_max_rows_per_launch(7) == -5


def test_workspace_sizes(qh):
    assert qh.w8a8_workspace_bytes(7168) >= 128 * 7168 + 128 * 4
    # the GEMV's staged BF16 activations: 64 KiB per 256 of hidden
    assert qh.w8a8_workspace_bytes(7168) >= 128 * 7168 + 28 * 65536
    assert qh.w8a8_workspace_bytes(7169) >= qh.w8a8_workspace_bytes(7168) + 65536
    assert qh.w8a8_workspace_bytes(7168) % 256 == 0
    assert qh.w8a8_workspace_bytes(0) == 0
    assert qh.q6k_workspace_bytes(7168) >= 8 * (7168 // 32) * 36
    assert qh.q6k_workspace_bytes(-5) == 0


def test_fp8_validation(qh):
    f = qh.lib().qhead_fp8_rowscale
    assert f(None, A16, A16, 1, 16, 8, A16, None) == -1
    assert f(A16, A16, A16, -1, 16, 8, A16, None) == -2
    assert f(A16, A16, A16, 1, 24, 8, A16, None) == -2   # hidden % 16
    assert f(A16, A16, A16, 1, 16, 0, A16, None) == -2
    assert f(MIS, A16, A16, 1, 16, 8, A16, None) == -3
    assert f(A16, A16, A16 + 8, 1, 16, 8, A16, None) == -3
    assert f(A16, A16, A16, 1, 16, 8, MIS, None) == -3
    assert f(A16, A16, A16, 0, 16, 8, A16, None) == 0     # rows = 0: no launch


def test_w8a8_validation(qh):
    L = qh.lib()
    ws = qh.w8a8_workspace_bytes(64)
    f = L.qhead_w8a8
    assert f(A16, A16, A16, 1, 64, 8, A16, None, ws, None) == -4
    assert f(A16, A16, A16, 1, 64, 8, A16, A256, ws - 1, None) == -4
    assert f(A16, A16, A16, 1, 64, 8, A16, A256 + 16, ws, None) == -3
    assert f(A16, A16, A16, 1, 65, 8, A16, A256, ws, None) == -2
    assert f(A16, A16, A16, 0, 64, 8, A16, A256, ws, None) == 0
    g = L.qhead_quant_act_e4m3
    assert g(A16, 2, 64, None, A16, None) == -1
    assert g(A16, 2, 64, A16 + 4, A16, None) == -3
    assert g(A16, 0, 64, A16, A16, None) == 0
    h = L.qhead_w8a8_gemv
    assert h(A16, A16, A16, None, 1, 64, 8, A16, None) == -1
    assert h(A16, A16, A16 + 8, A16, 1, 64, 8, A16, None) == -3  # xq 16-byte aligned
    assert h(A16, A16, A16, A16, 0, 64, 8, A16, None) == 0


def test_nvfp4_validation(qh):
    f = qh.lib().qhead_nvfp4
    assert f(A16, A16, A16, 1, 48, 8, A16, 1.0, None) == -2   # hidden % 32
    assert f(A16, A16 + 1, A16, 1, 64, 8, A16, 1.0, None) == -3
    assert f(A16, None, A16, 1, 64, 8, A16, 1.0, None) == -1
    assert f(A16, A16, A16, 0, 64, 8, A16, 1.0, None) == 0


def test_q6k_validation(qh):
    L = qh.lib()
    ws = qh.q6k_workspace_bytes(512)
    f = L.qhead_q6k
    assert f(A16, A16, A16, 1, 512, 8, A16, A256, ws, None) == -5   # scales must be NULL
    assert f(A16, None, A16, 1, 384, 8, A16, A256, ws, None) == -2  # hidden % 256
    assert f(A16, None, A16, 1, 512, 8, A16, A256, ws - 1, None) == -4
    assert f(A16 + 1, None, A16, 1, 512, 8, A16, A256, ws, None) == -3
    assert f(A16, None, A16, 0, 512, 8, A16, A256, ws, None) == 0
    g = L.qhead_quant_q8_1
    assert g(A16, 1, 48, A16, None) == -2
    assert g(A16, 1, 64, A16 + 2, None) == -3
    assert g(A16, 0, 64, A16, None) == 0
    h = L.qhead_q6k_gemv
    assert h(A16, A16 + 2, 1, 256, 8, A16, None) == -3
    assert h(A16, A16, 0, 256, 8, A16, None) == 0


def test_q6k_static_scratch_validation(qh):
    """The fixed-scratch Q6_K entry point rejects what qhead_q6k rejects, and
    hidden beyond its scratch (QHEAD_ERR_SCRATCH), before any HIP call."""
    L = qh.lib()
    f = L.qhead_q6k_static_scratch
    big = qh.Q6K_STATIC_MAX_HIDDEN
    assert f(A16, A16, A16, 1, 512, 8, A16, None) == -5   # scales must be NULL
    assert f(A16, None, A16, 1, 384, 8, A16, None) == -2  # hidden % 256
    assert f(A16, None, A16, -1, 512, 8, A16, None) == -2
    assert f(None, None, A16, 1, 512, 8, A16, None) == -1
    assert f(A16 + 1, None, A16, 1, 512, 8, A16, None) == -3
    assert f(A16, None, A16, 1, big + 256, 8, A16, None) == -8
    assert f(A16, None, A16, 0, big + 256, 8, A16, None) == 0  # rows == 0: nothing to do
    assert f(A16, None, A16, 0, 512, 8, A16, None) == 0
    assert "scratch" in qh.status_string(-8)


def test_quantize_fp8_rows_validation(qh):
    f = qh.lib().qhead_quantize_fp8_rows
    assert f(A16, 8, 24, A16, A16, None) == -2
    assert f(A16 + 4, 8, 16, A16, A16, None) == -3
    assert f(A16, 0, 16, A16, A16, None) == 0


def test_silu_validation(qh):
    L = qh.lib()
    m = L.qhead_silu_mul_bf16
    assert m(A16, A16, -1, A16, None) == -2
    assert m(A16, None, 8, A16, None) == -1
    assert m(A16, A16, 8, MIS, None) == -3
    assert m(None, None, 0, None, None) == 0
    f = L.qhead_quant_act_silu_e4m3
    assert f(A16, A16, 64, 2, 24, A16, A16, None) == -2     # hidden % 16
    assert f(A16, A16, 48, 2, 64, A16, A16, None) == -2     # ld < hidden
    assert f(A16, A16, 68, 2, 64, A16, A16, None) == -2     # ld % 8
    assert f(A16, None, 64, 2, 64, A16, A16, None) == -1
    assert f(A16, A16 + 8, 64, 2, 64, A16, A16, None) == -3
    assert f(A16, A16, 64, 2, 64, A16 + 4, A16, None) == -3
    assert f(None, None, 64, 0, 64, None, None, None) == 0   # rows = 0: no launch
    ws = qh.w8a8_workspace_bytes(64)
    g = L.qhead_w8a8_silu
    assert g(A16, A16, A16, A16, 64, 1, 64, 8, A16, A256, ws - 1, None) == -4
    assert g(A16, A16, A16, A16, 56, 1, 64, 8, A16, A256, ws, None) == -2
    assert g(A16, A16, A16, None, 64, 1, 64, 8, A16, A256, ws, None) == -1
    assert g(A16, A16, A16, A16 + 2, 64, 1, 64, 8, A16, A256, ws, None) == -3
    assert g(A16, A16, A16, A16, 64, 1, 64, 8, A16, A256 + 64, ws, None) == -3
    assert g(None, None, None, None, 64, 0, 64, 8, None, None, 0, None) == 0


def test_quantize_nvfp4_q6k_rows_validation(qh):
    L = qh.lib()
    f = L.qhead_quantize_nvfp4_rows
    assert f(A16, 8, 24, 1.0, A16, A16, None) == -2      # hidden % 16
    assert f(A16, -1, 32, 1.0, A16, A16, None) == -2
    assert f(A16, 8, 32, 1.0, A16, None, None) == -1
    assert f(A16 + 4, 8, 32, 1.0, A16, A16, None) == -3
    assert f(A16, 8, 32, 1.0, A16 + 4, A16, None) == -3
    assert f(None, 0, 32, 1.0, None, None, None) == 0    # vocab = 0: no launch
    g = L.qhead_quantize_q6k_rows
    assert g(A16, 8, 384, A16, None) == -2              # hidden % 256
    assert g(A16, 8, 256, None, None) == -1
    assert g(A16, 8, 256, A16 + 1, None) == -3
    assert g(None, 0, 256, None, None) == 0


def test_dequant_validation(qh):
    L = qh.lib()
    f = L.qhead_dequant_nvfp4_bf16
    assert f(A16, A16, 4, 48, 1.0, A16, None) == -2      # cols % 32
    assert f(A16, A16, -1, 64, 1.0, A16, None) == -2
    assert f(A16, None, 4, 64, 1.0, A16, None) == -1
    assert f(A16 + 8, A16, 4, 64, 1.0, A16, None) == -3
    assert f(A16, A16 + 1, 4, 64, 1.0, A16, None) == -3
    assert f(A16, A16, 4, 64, 1.0, A16 + 2, None) == -3
    assert f(None, None, 0, 64, 1.0, None, None) == 0
    g = L.qhead_dequant_fp4_e8m0_bf16
    assert g(A16, A16, 96, 5, A16, None) == -2           # 96 values do not split in 5 groups
    assert g(A16, A16, 96, 4, A16, None) == -2           # groups of 24 (not a multiple of 16)
    assert g(A16, A16, 96, 0, A16, None) == -2
    assert g(A16, A16, 96, 3, None, None) == -1
    assert g(A16 + 4, A16, 96, 3, A16, None) == -3
    assert g(A16, A16, 96, 3, A16 + 8, None) == -3
    assert g(None, None, 0, 3, None, None) == 0


def test_stream_read_validation(qh):
    f = qh.lib().qhead_stream_read
    assert f(A16, 40, A16, None) == -2                   # not a multiple of 16
    assert f(A16, -16, A16, None) == -2
    assert f(None, 64, A16, None) == -1
    assert f(A16, 64, None, None) == -1
    assert f(A16 + 8, 64, A16, None) == -3
    assert f(A16, 64, A16 + 2, None) == -3
    assert f(None, 0, None, None) == 0


def test_header_is_plain_c(qh, tmp_path):
    """A C99 program includes include/qhead.h (-pedantic -Werror), links the
    library and calls its host-side entry points."""
    exe = tmp_path / "c_abi_smoke"
    libdir = os.path.dirname(qh.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_smoke.c"),
                    "-L", libdir, "-lqhead", f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True)
    run = subprocess.run([str(exe)], capture_output=True, text=True)
    assert run.returncode == 0, run.stdout + run.stderr


def test_binding_rejects_host_tensors(qh):
    import torch

    w = torch.zeros((8, 16), dtype=torch.uint8)
    with pytest.raises(ValueError):
        qh.fp8_rowscale(w, torch.zeros(8), torch.zeros((1, 16), dtype=torch.bfloat16))


def test_binding_rejects_wrong_shapes(qh):
    """Every wrapper checks its tensors' shapes before any pointer reaches the
    library (the library reads and writes by the sizes passed, so a short
    tensor would be overrun). Host tensors serve here: the shape check comes
    before the device check, and the message names the shape."""
    import torch

    u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
    V, H, R = 8, 512, 2
    w = torch.zeros((V, H), dtype=u8)
    s = torch.zeros(V, dtype=f32)
    x = torch.zeros((R, H), dtype=bf)
    xq = torch.zeros((R, H), dtype=u8)
    sa = torch.zeros(R, dtype=f32)
    shape_msg = r"shape|elements|exceeds"
    cases = [
        lambda: qh.fp8_rowscale(w, s[:V - 1], x),
        lambda: qh.fp8_rowscale(w, s, x[:, :H - 16]),
        lambda: qh.fp8_rowscale(w, s, x, out=torch.zeros((R, V - 1), dtype=bf)),
        lambda: qh.fp8_rowscale(w, s, x, out=torch.zeros((R + 1, V), dtype=bf)),
        lambda: qh.quant_act_e4m3(x, xq=xq[:1]),
        lambda: qh.quant_act_e4m3(x, xscale=sa[:1]),
        lambda: qh.w8a8_gemv(w, s, xq, sa[:1]),
        lambda: qh.w8a8_gemv(w, s, xq[:, :H - 32], sa),
        lambda: qh.w8a8(w, s, x, workspace=torch.zeros(4, dtype=u8)),
        lambda: qh.w8a8_silu(w, s, x, x[:, :H - 16]),
        lambda: qh.quant_act_silu_e4m3(x, x, hidden=H + 16),
        lambda: qh.silu_mul_bf16(x, x, out=torch.zeros((R, H - 1), dtype=bf)),
        lambda: qh.nvfp4(torch.zeros((V, H // 2), dtype=u8), torch.zeros((V, H // 32), dtype=u8),
                         x, 1.0),
        lambda: qh.nvfp4(torch.zeros((V, H // 2), dtype=u8), torch.zeros((V, H // 16), dtype=u8),
                         x[:, :H // 2], 1.0),
        lambda: qh.quant_q8_1(x, q8=torch.zeros(R * (H // 32) * 36 - 1, dtype=u8)),
        lambda: qh.q6k_gemv(torch.zeros((V, 2 * 210), dtype=u8),
                            torch.zeros((R, H // 32 * 36), dtype=u8), H + 256),
        lambda: qh.q6k_gemv(torch.zeros((V, 2 * 210), dtype=u8),
                            torch.zeros((R, H // 32 * 36 - 36), dtype=u8), H),
        lambda: qh.q6k(torch.zeros((V, 3 * 210), dtype=u8), x),
        lambda: qh.q6k_static_scratch(torch.zeros((V, 1 * 210), dtype=u8), x),
        lambda: qh.quantize_fp8_rows(torch.zeros((V, H)), codes=w[:, :H - 1]),
        lambda: qh.quantize_fp8_rows(torch.zeros((V, H)), scales=s[:1]),
        lambda: qh.quantize_nvfp4_rows(torch.zeros((V, H)), 1.0,
                                       block_scale=torch.zeros((V, H // 8), dtype=u8)),
        lambda: qh.quantize_q6k_rows(torch.zeros((V, H)),
                                     blocks=torch.zeros((V, 210), dtype=u8)),
        lambda: qh.dequant_nvfp4_bf16(torch.zeros((V, H // 2), dtype=u8),
                                      torch.zeros((V, H // 16 - 1), dtype=u8), 1.0),
        lambda: qh.dequant_fp4_e8m0_bf16(torch.zeros(H // 2, dtype=u8),
                                         torch.zeros(H // 32, dtype=u8),
                                         out=torch.zeros(H - 2, dtype=bf)),
    ]
    for call in cases:
        with pytest.raises(ValueError, match=shape_msg):
            call()
    # the same call with matching shapes gets as far as the device check
    with pytest.raises(ValueError, match="device|CUDA|cuda"):
        qh.fp8_rowscale(w, s, x)
