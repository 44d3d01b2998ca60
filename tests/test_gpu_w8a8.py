"""W8A8 GEMV across its two kernels: the VALU kernel (1..15 rows per launch)
and the MFMA kernel (16..128 rows per launch, one weight pass) add the same
BF16 pairs in the same order, so a row's logits must be bit-identical whatever
the row count of the call ("lm_head_fp8_rows.rs" module doc: one weight pass
per 128 rows, W8A8_MAX_ROWS; "w8a8_layer.rs" module doc: a row's bits do not
depend on the row count). Every logit is also checked against the binary64
oracle within |gpu - ref| <= 2^-7 |ref| + 1e-4 sum|x w|."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import (DEV, assert_within_bound, dev_bf16, dev_f32, dev_u8, fp8_head, host_bits,
                         log, sample_vidx, x_rows)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qh():
    import quantized_weight_decode_amd as m

    return m


def _head(V, H, seed=0):
    wf = synth.weight_rows_f32(synth.W8A8_129280X7168, seed, seed + V, vocab=seed + V, hidden=H)
    return oracle.prep_fp8_rows(wf)


@pytest.mark.parametrize("V,H", [(1001, 1040), (37, 16), (513, 4112), (700, 8208), (96, 4096)])
def test_w8a8_every_row_count_small_heads(qh, V, H):
    """Rows 1..128 in one call each (R < 16 on the VALU kernel, R >= 16 on the
    MFMA kernel): all logits within the bound, and every row bit-identical to
    the same row of the 128-row call. Shapes cover a 16-k tail (H % 32 == 16),
    a tail past one 4096-k tile, two tiles plus a tail, vocab tails and a
    single 16-k granule."""
    w, s = _head(V, H)
    x = synth.activations_bf16(synth.W8A8_129280X7168, 128, hidden=H, max_rows=128)
    xq, sa = oracle.quant_act_e4m3(x)
    ref, ad = oracle.w8a8_ref(w, s, xq, sa)
    wd, sd, xqd, sad = dev_u8(w), dev_f32(s), dev_u8(xq), dev_f32(sa)
    log(f"[case] w8a8 every row count V={V} H={H}")
    full = host_bits(qh.w8a8_gemv(wd, sd, xqd, sad))
    torch.cuda.synchronize()
    assert_within_bound(full, ref, ad, f"w8a8 V={V} H={H} R=128")
    for R in range(1, 128):
        out = host_bits(qh.w8a8_gemv(wd, sd, xqd[:R], sad[:R]))
        assert np.array_equal(out, full[:R]), f"V={V} H={H}: row invariance at R={R}"


def test_w8a8_all_codes_valu_equals_mfma(qh):
    """Weights and activations drawn uniformly over all 254 finite E4M3 codes
    (every binade, subnormals, both zeros; unit scales): partial sums span the
    whole range where the accumulation rounds, so any difference between the
    VALU dot2 steps and the MFMA steps shows. Rows at R = 1, 4, 15 (VALU) and
    16, 17, 64, 128 (MFMA) must be bit-identical."""
    V, H = 4099, 7168
    g = np.random.Generator(np.random.PCG64(2024))
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    w = g.choice(codes, size=(V, H))
    xq = g.choice(codes, size=(128, H))
    sw = np.ones(V, np.float32)
    sa = np.ones(128, np.float32)
    wd, sd, xqd, sad = dev_u8(w), dev_f32(sw), dev_u8(xq), dev_f32(sa)
    log("[case] w8a8 all-codes VALU vs MFMA")
    full = host_bits(qh.w8a8_gemv(wd, sd, xqd, sad))
    vidx = sample_vidx(V, 400, 7)
    ref, ad = oracle.w8a8_ref(w, sw, xq, sa, vidx)
    assert_within_bound(full[:, vidx], ref, ad, "w8a8 all codes R=128")
    for R in (1, 4, 15, 16, 17, 64):
        out = host_bits(qh.w8a8_gemv(wd, sd, xqd[:R], sad[:R]))
        assert np.array_equal(out, full[:R]), f"all codes: row invariance at R={R}"


@pytest.mark.parametrize("R", [16, 40, 128])
def test_w8a8_exact_cases_mfma_bit_exact(qh, R):
    """Dyadic values whose every partial sum is exact: the MFMA kernel must
    return the oracle's BF16 rounding of the exact result."""
    V, H = 700, 1024
    g = np.random.Generator(np.random.PCG64(34 + R))
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


@pytest.mark.parametrize("V,H", [(1001, 1040), (20000, 4112), (700, 8208), (37, 16)])
def test_w8a8_staged_image_equals_in_kernel_staging(qh, V, H):
    """qhead_w8a8 stages the activations of its launches with direct weight
    loads from a BF16 image built in its workspace (copied into LDS without
    passing through registers); qhead_w8a8_gemv, which has no workspace,
    converts the codes inside the kernel. Both must stage the same bytes, so
    on the same quantized activations their logits are bit-identical, at row
    counts on every launch shape (narrow heads from 17 rows, wide heads from
    33) including ragged row tiles."""
    w, s = _head(V, H)
    x = synth.activations_bf16(synth.W8A8_129280X7168, 128, hidden=H, max_rows=128)
    wd, sd = dev_u8(w), dev_f32(s)
    ws = qh.w8a8_workspace(H, DEV)
    for R in (17, 32, 33, 40, 48, 49, 64, 65, 80, 97, 113, 128):
        log(f"[case] w8a8 image vs in-kernel staging V={V} H={H} R={R}")
        xd = dev_bf16(x[:R])
        xq, sa = qh.quant_act_e4m3(xd)
        staged = host_bits(qh.w8a8_gemv(wd, sd, xq, sa))
        imaged = host_bits(qh.w8a8(wd, sd, xd, workspace=ws))
        assert np.array_equal(imaged, staged), f"V={V} H={H} R={R}: image path differs"


def test_w8a8_full_head_row_counts_across_kernels(qh):
    """The 129280 x 7168 head: rows of 1-, 4-, 15-, 16-, 17- and 128-row
    calls equal the same rows of the 300-row call (128 + 128 + 44), and the
    sampled logits are within the bound."""
    w, s, wd, sd = fp8_head(synth.W8A8_129280X7168)
    cfg = synth.CONFIGS[synth.W8A8_129280X7168]
    x = x_rows(synth.W8A8_129280X7168, 300)
    ws = qh.w8a8_workspace(cfg.hidden, DEV)
    log("[case] w8a8 129280x7168 R=300")
    full = host_bits(qh.w8a8(wd, sd, dev_bf16(x), workspace=ws))
    torch.cuda.synchronize()
    vidx = sample_vidx(cfg.vocab, 600, 11)
    xq, sa = oracle.quant_act_e4m3(x)
    ref, ad = oracle.w8a8_ref(w, s, xq, sa, vidx)
    assert_within_bound(full[:, vidx], ref, ad, "w8a8 129280x7168 R=300")
    for R in (1, 4, 15, 16, 17, 128):
        log(f"[case] w8a8 129280x7168 R={R}")
        out = host_bits(qh.w8a8(wd, sd, dev_bf16(x[:R]), workspace=ws))
        assert np.array_equal(out, full[:R]), f"row invariance at R={R}"
    # a 44-row call on rows 256..299 (the third chunk of the 300-row call)
    tail = host_bits(qh.w8a8(wd, sd, dev_bf16(x[256:300]), workspace=ws))
    assert np.array_equal(tail, full[256:300])
