"""GPU parity of the FP8 head (W8A16), the W8A8 head and the activation
quantizer against the CPU oracle, through the C ABI (Python binding).

Bars: logits within |gpu - ref| <= 2^-7 |ref| + 1e-4 sum|x w|; quantizer bytes
and scales bit-exact; exact dyadic cases bit-exact; every row's logits
bit-identical across row counts and chunkings.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import (DEV, assert_within_bound, bf16_bits_to_f64, dev_bf16, dev_f32, dev_u8,
                         fp8_head, host_bits, log, sample_vidx, x_rows)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qh():
    import quantized_weight_decode_amd as m

    assert torch.cuda.is_available()
    return m


def _fp8_small(V, H, cfg=synth.FP8_8192X1024, seed_rows=None):
    wf = synth.weight_rows_f32(cfg, 0, V, vocab=V, hidden=H)
    return oracle.prep_fp8_rows(wf)


# ------------------------------------------------------------- exact decode

def test_fp8_every_code_every_byte_position(qh):
    """One-hot activations pick single weights: out = e4m3(code) * s exactly."""
    V, H = 256, 1024
    w = np.zeros((V, H), dtype=np.uint8)
    codes = np.arange(256, dtype=np.uint8)
    codes[[0x7F, 0xFF]] = 0  # NaN codes are never generated
    ks = [0, 1, 2, 3, 4, 7, 8, 15, 16, 17, 500, 511, 512, 1020, 1023]
    for k in ks:
        w[:, k] = codes
    s = np.ones(V, dtype=np.float32)
    s[1::2] = 0.25
    x = np.zeros((len(ks), H), dtype=np.uint16)
    for i, k in enumerate(ks):
        x[i, k] = 0x3F80
    log(f"[case] fp8 one-hot decode V={V} H={H} R={len(ks)}")
    out = qh.fp8_rowscale(dev_u8(w), dev_f32(s), dev_bf16(x))
    torch.cuda.synchronize()
    got = host_bits(out)
    ref, _ = oracle.fp8_rowscale_ref(w, s, x)
    expect = oracle.bf16_rne_array(ref)
    assert np.array_equal(got, expect)


def test_fp8_exact_dyadic_cases_bit_exact(qh):
    """Small-integer x, weights on a coarse dyadic grid, power-of-two scales:
    every partial sum is exact in FP32, so GPU bits equal bf16(ref)."""
    V, H, R = 1000, 2048, 5
    g = np.random.Generator(np.random.PCG64(21))
    grid = [c for c in range(256) if c not in (0x7F, 0xFF) and
            abs(oracle.e4m3_value(c)) <= 8 and (oracle.e4m3_value(c) * 8) % 1 == 0]
    w = g.choice(np.array(grid, dtype=np.uint8), size=(V, H))
    s = (2.0 ** g.integers(-12, 4, size=V)).astype(np.float32)
    xv = g.integers(-4, 5, size=(R, H)).astype(np.float32)
    x = synth.to_bf16_bits(xv)
    log(f"[case] fp8 exact dyadic V={V} H={H} R={R}")
    out = qh.fp8_rowscale(dev_u8(w), dev_f32(s), dev_bf16(x))
    torch.cuda.synchronize()
    ref, _ = oracle.fp8_rowscale_ref(w, s, x)
    assert np.array_equal(host_bits(out), oracle.bf16_rne_array(ref))


# ------------------------------------------------------------------ 8192x1024

def test_fp8_8192x1024_all_logits(qh):
    w, s = _fp8_small(8192, 1024)
    x = x_rows(synth.FP8_8192X1024, 16, max_rows=16)
    wd, sd = dev_u8(w), dev_f32(s)
    ref, ad = oracle.fp8_rowscale_ref(w, s, x)
    outs = {}
    for R in range(1, 17):
        log(f"[case] fp8 8192x1024 R={R}")
        out = qh.fp8_rowscale(wd, sd, dev_bf16(x[:R]))
        torch.cuda.synchronize()
        outs[R] = host_bits(out)
        assert_within_bound(outs[R], ref[:R], ad[:R], f"8192x1024 R={R}")
    # row invariance: a row's bits do not depend on the launch's row count
    for R in range(1, 17):
        assert np.array_equal(outs[R], outs[16][:R]), R


def test_fp8_launch_shape_does_not_change_bits(qh):
    """9..16-row launches take 2-row bands on heads with fewer than
    8 * 4 * 2 * CUs vocab rows and 4-row bands above. The same rows computed
    under both shapes (a head and its leading rows) have identical bits, for
    W8A16 and W8A8, and lie within the bound."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    v_big = 2 * cus * 8 * 4          # 4-row bands: (V + 3) / 4 is not below the limit
    v_small = v_big - 4              # 2-row bands
    H = 1024
    w, s = _fp8_small(v_big, H, cfg=synth.FP8_32000X4096)
    wd, sd = dev_u8(w), dev_f32(s)
    for R in (9, 16):
        x = synth.activations_bf16(synth.FP8_32000X4096, R, hidden=H, max_rows=R)
        xd = dev_bf16(x)
        log(f"[case] fp8 launch shapes V={v_big}/{v_small} R={R}")
        big = host_bits(qh.fp8_rowscale(wd, sd, xd))
        small = host_bits(qh.fp8_rowscale(wd[:v_small], sd[:v_small], xd))
        assert np.array_equal(big[:, :v_small], small), R
        vidx = sample_vidx(v_big, 600, R)
        ref, ad = oracle.fp8_rowscale_ref(w[vidx], s[vidx], x)
        assert_within_bound(big[:, vidx], ref, ad, f"shape check R={R}")
        big8 = host_bits(qh.w8a8(wd, sd, xd))
        small8 = host_bits(qh.w8a8(wd[:v_small], sd[:v_small], xd))
        assert np.array_equal(big8[:, :v_small], small8), R


def test_fp8_edge_shapes(qh):
    """Ragged vocab, hidden not a multiple of the 1024-wide segment or the
    4096-wide LDS tile, a single vocab row, and rows spanning chunk borders."""
    for V, H, rows in [(1001, 1040, 3), (1, 16, 2), (37, 16, 16), (513, 4112, 17),
                       (300, 8208, 9), (4099, 3072, 33), (64, 8192, 1)]:
        log(f"[case] fp8 edge V={V} H={H} rows={rows}")
        wf = synth.weight_rows_f32(synth.FP8_32000X4096, 0, V, vocab=V, hidden=H)
        w, s = oracle.prep_fp8_rows(wf)
        x = synth.activations_bf16(synth.FP8_32000X4096, rows, hidden=H, max_rows=rows,
                                   outlier_channels=0)
        out = qh.fp8_rowscale(dev_u8(w), dev_f32(s), dev_bf16(x))
        torch.cuda.synchronize()
        ref, ad = oracle.fp8_rowscale_ref(w, s, x)
        assert_within_bound(host_bits(out), ref, ad, f"edge V={V} H={H} rows={rows}")


def test_fp8_rows_zero_is_noop(qh):
    """rows = 0 through the C ABI: success, and the output buffer (here one
    row long) is left untouched."""
    w, s = _fp8_small(64, 64)
    wd, sd = dev_u8(w), dev_f32(s)
    x = torch.zeros((1, 64), dtype=torch.bfloat16, device=DEV)
    out = torch.full((1, 64), 7.0, dtype=torch.bfloat16, device=DEV)
    st = qh.lib().qhead_fp8_rowscale(wd.data_ptr(), sd.data_ptr(), x.data_ptr(), 0, 64, 64,
                                     out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    assert torch.all(out == 7.0)
    # the binding passes rows = 0 for an empty x and returns an empty result
    assert qh.fp8_rowscale(wd, sd, x[:0]).shape == (0, 64)


def test_fp8_zero_rows_and_scale(qh):
    V, H = 128, 256
    w, s = _fp8_small(V, H)
    w[5] = 0
    s[5] = 0.0
    s[9] = 0.0
    x = x_rows(synth.FP8_8192X1024, 3, hidden=H, max_rows=3)
    x[1] = 0
    out = host_bits(qh.fp8_rowscale(dev_u8(w), dev_f32(s), dev_bf16(x)))
    torch.cuda.synchronize()
    vals = bf16_bits_to_f64(out)
    assert (vals[:, 5] == 0).all() and (vals[:, 9] == 0).all() and (out[1] == 0).all()


# ------------------------------------------------------------------ 32000x4096

def test_fp8_32000x4096_outliers_sampled(qh):
    w, s, wd, sd = fp8_head(synth.FP8_32000X4096)
    cfg = synth.CONFIGS[synth.FP8_32000X4096]
    x = x_rows(synth.FP8_32000X4096, 40)
    vidx = sample_vidx(cfg.vocab, 3000, 1)
    ref, ad = oracle.fp8_rowscale_ref(w, s, x, vidx)
    outs = {}
    for R in cfg.rows:
        log(f"[case] fp8 32000x4096 R={R}")
        out = qh.fp8_rowscale(wd, sd, dev_bf16(x[:R]))
        torch.cuda.synchronize()
        outs[R] = host_bits(out)
        assert_within_bound(outs[R][:, vidx], ref[:R], ad[:R], f"32000x4096 R={R}")
    for R in cfg.rows:
        assert np.array_equal(outs[R], outs[40][:R]), f"row invariance R={R}"


# ------------------------------------------------------------------ 155136x8192

def test_fp8_155136x8192_full_head_sampled(qh):
    """The 1.27 GB head at rows 1, 2, 4, 8, 16 and 64 (four 16-row passes)."""
    w, s, wd, sd = fp8_head(synth.FP8_155136X8192)
    cfg = synth.CONFIGS[synth.FP8_155136X8192]
    x = x_rows(synth.FP8_155136X8192, 64)
    vidx = sample_vidx(cfg.vocab, 1500, 2)
    ref, ad = oracle.fp8_rowscale_ref(w, s, x, vidx)
    outs = {}
    for R in cfg.rows:
        log(f"[case] fp8 155136x8192 R={R}")
        out = qh.fp8_rowscale(wd, sd, dev_bf16(x[:R]))
        torch.cuda.synchronize()
        outs[R] = host_bits(out)
        assert_within_bound(outs[R][:, vidx], ref[:R], ad[:R], f"155136x8192 R={R}")
    for R in cfg.rows:
        assert np.array_equal(outs[R], outs[64][:R]), f"row invariance R={R}"
    # the 64-row call equals its four 16-row chunks launched separately
    for c in range(4):
        part = host_bits(qh.fp8_rowscale(wd, sd, dev_bf16(x[16 * c:16 * c + 16])))
        assert np.array_equal(part, outs[64][16 * c:16 * c + 16])


def test_quantize_fp8_rows_matches_oracle(qh):
    """Load-time weight quantization on the GPU equals the oracle's bytes."""
    wf = synth.weight_rows_f32(synth.FP8_155136X8192, 5000, 7048)
    wf[3] = 0.0
    log("[case] quantize_fp8_rows 2048x8192")
    codes, scales = qh.quantize_fp8_rows(dev_f32(wf))
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.prep_fp8_rows(wf)
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


# --------------------------------------------------------- act quant, W8A8

def _act_rows_with_specials(H, rows, cfg=synth.W8A8_129280X7168):
    x = synth.activations_bf16(cfg, rows, hidden=H, max_rows=rows)
    x[0] = 0                       # all-zero row
    x[1] = 0x8000                  # all negative zero
    x[2, :] = 0
    x[2, 7] = 0x0001               # a single BF16 subnormal
    x[3] = synth.to_bf16_bits(np.linspace(-448, 448, H, dtype=np.float32)[None, :])[0]
    x[4, ::3] = 0x8000             # scattered negative zeros
    return x


def test_quant_act_e4m3_bit_exact(qh):
    H, rows = 7168, 300
    x = _act_rows_with_specials(H, rows)
    log(f"[case] quant_act_e4m3 rows={rows} H={H}")
    xq, sa = qh.quant_act_e4m3(dev_bf16(x))
    torch.cuda.synchronize()
    xq_ref, sa_ref = oracle.quant_act_e4m3(x)
    assert np.array_equal(sa.cpu().numpy().view(np.uint32), sa_ref.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), xq_ref)


def test_quant_act_e4m3_ties_exhaustive_grid(qh):
    """Rows whose quotients x / sa land on every E4M3 tie and grid point."""
    H = 512
    grid = np.array(sorted(set(oracle.e4m3_table()[:0x7F].tolist())), dtype=np.float64)
    mids = (grid[1:] + grid[:-1]) / 2
    vals = np.concatenate([grid, mids, -grid, -mids])
    vals = np.resize(vals, (2, H)).astype(np.float32)
    # with amax = 448 the scale is exactly 1, so x / sa = x
    vals[:, 0] = 448.0
    x = synth.to_bf16_bits(vals)
    xq, sa = qh.quant_act_e4m3(dev_bf16(x))
    torch.cuda.synchronize()
    xq_ref, sa_ref = oracle.quant_act_e4m3(x)
    assert np.array_equal(sa.cpu().numpy(), sa_ref)
    assert np.array_equal(xq.cpu().numpy(), xq_ref)


def test_w8a8_exact_cases_bit_exact(qh):
    V, H, R = 700, 1024, 6
    g = np.random.Generator(np.random.PCG64(33))
    grid = [c for c in range(256) if c not in (0x7F, 0xFF) and
            abs(oracle.e4m3_value(c)) <= 16 and (oracle.e4m3_value(c) * 4) % 1 == 0]
    w = g.choice(np.array(grid, dtype=np.uint8), size=(V, H))
    xq = g.choice(np.array(grid, dtype=np.uint8), size=(R, H))
    sw = (2.0 ** g.integers(-10, 2, size=V)).astype(np.float32)
    sa = (2.0 ** g.integers(-6, 3, size=R)).astype(np.float32)
    out = qh.w8a8_gemv(dev_u8(w), dev_f32(sw), dev_u8(xq), dev_f32(sa))
    torch.cuda.synchronize()
    ref, _ = oracle.w8a8_ref(w, sw, xq, sa)
    assert np.array_equal(host_bits(out), oracle.bf16_rne_array(ref))


def test_w8a8_129280x7168_full_head(qh):
    """W8A8 on the 129280 x 7168 head at rows 1, 16, 128 and 300 (<= 128-row
    calls); logits within the bound on sampled vocab rows, row-invariant bits."""
    w, s, wd, sd = fp8_head(synth.W8A8_129280X7168)
    cfg = synth.CONFIGS[synth.W8A8_129280X7168]
    x = x_rows(synth.W8A8_129280X7168, 300)
    xq, sa = oracle.quant_act_e4m3(x)
    vidx = sample_vidx(cfg.vocab, 800, 3)
    ref, ad = oracle.w8a8_ref(w, s, xq, sa, vidx)
    ws = qh.w8a8_workspace(cfg.hidden, DEV)
    outs = {}
    for R in cfg.rows:
        log(f"[case] w8a8 129280x7168 R={R}")
        out = qh.w8a8(wd, sd, dev_bf16(x[:R]), workspace=ws)
        torch.cuda.synchronize()
        outs[R] = host_bits(out)
        assert_within_bound(outs[R][:, vidx], ref[:R], ad[:R], f"129280x7168 R={R}")
    for R in cfg.rows:
        assert np.array_equal(outs[R], outs[300][:R]), f"row invariance R={R}"
    # rows 128..255 of the 300-row call equal a separate call on those rows
    sep = host_bits(qh.w8a8(wd, sd, dev_bf16(x[128:256]), workspace=ws))
    assert np.array_equal(sep, outs[300][128:256])


def test_w8a8_two_streams_two_workspaces(qh):
    V, H = 4096, 2048
    w, s = _fp8_small(V, H)
    wd, sd = dev_u8(w), dev_f32(s)
    xa = x_rows(synth.W8A8_129280X7168, 20, hidden=H, max_rows=40)
    xb = synth.to_bf16_bits(synth.activations_f32(synth.W8A8_129280X7168, 40, hidden=H)[20:40] * 3)
    ref_a = host_bits(qh.w8a8(wd, sd, dev_bf16(xa)))
    ref_b = host_bits(qh.w8a8(wd, sd, dev_bf16(xb)))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    ws1, ws2 = qh.w8a8_workspace(H, DEV), qh.w8a8_workspace(H, DEV)
    dxa, dxb = dev_bf16(xa), dev_bf16(xb)
    torch.cuda.synchronize()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            oa = qh.w8a8(wd, sd, dxa, workspace=ws1)
        with torch.cuda.stream(s2):
            ob = qh.w8a8(wd, sd, dxb, workspace=ws2)
        outs.append((oa, ob))
    torch.cuda.synchronize()
    for oa, ob in outs:
        assert np.array_equal(host_bits(oa), ref_a)
        assert np.array_equal(host_bits(ob), ref_b)
