"""GPU parity of the NVFP4 (W4A16) head, the q8_1 quantizer and the Q6_K
head against the CPU oracle, through the C ABI (Python binding).

Bars: logits within |gpu - ref| <= 2^-7 |ref| + 1e-4 sum|x w|; q8_1 bytes
bit-exact; one-hot decodes and exact dyadic cases bit-exact; row-invariant
bits across row counts and chunkings.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import (DEV, assert_within_bound, bf16_bits_to_f64, dev_bf16, dev_u8, host_bits,
                         log, nvfp4_head, q6k_head, sample_vidx)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qh():
    import quantized_weight_decode_amd as m

    assert torch.cuda.is_available()
    return m


# ------------------------------------------------------------------ NVFP4

def test_nvfp4_every_nibble_every_block_scale(qh):
    """One-hot x picks single weights: out = e2m1(nibble) * e4m3(scale) * g."""
    V, H = 256, 64
    wp = np.zeros((V, H // 2), dtype=np.uint8)
    for k in range(32):  # nibble k % 16 at k, for both blocks of the first 32 k
        nib = k % 16
        wp[:, k // 2] |= np.uint8(nib if k % 2 == 0 else nib << 4)
    bs = np.zeros((V, H // 16), dtype=np.uint8)
    codes = np.arange(256, dtype=np.uint8)
    codes[[0x7F, 0xFF]] = 0
    bs[:, 0] = codes
    bs[:, 1] = codes[::-1]
    x = np.zeros((32, H), dtype=np.uint16)
    for k in range(32):
        x[k, k] = 0x3F80
    for g in (1.0, 0.25, 8.0):
        log(f"[case] nvfp4 one-hot g={g}")
        out = qh.nvfp4(dev_u8(wp), dev_u8(bs), dev_bf16(x), g)
        torch.cuda.synchronize()
        ref, _ = oracle.nvfp4_ref(wp, bs, g, x)
        assert np.array_equal(host_bits(out), oracle.bf16_rne_array(ref)), g


def test_nvfp4_exact_dyadic_bit_exact(qh):
    V, H, R = 900, 1024, 7
    g = np.random.Generator(np.random.PCG64(41))
    wp = g.integers(0, 256, size=(V, H // 2), dtype=np.uint8)
    pow2 = np.array([0x28, 0x30, 0x38, 0x40, 0x48], dtype=np.uint8)  # 2^-2 .. 2^2
    bs = g.choice(pow2, size=(V, H // 16))
    x = synth.to_bf16_bits(g.integers(-4, 5, size=(R, H)).astype(np.float32))
    out = qh.nvfp4(dev_u8(wp), dev_u8(bs), dev_bf16(x), 0.5)
    torch.cuda.synchronize()
    ref, _ = oracle.nvfp4_ref(wp, bs, 0.5, x)
    assert np.array_equal(host_bits(out), oracle.bf16_rne_array(ref))


def _nvfp4_small(V, H, cfg=synth.NVFP4_Q6K_129280X7168):
    wf = synth.weight_rows_f32(cfg, 0, V, vocab=V, hidden=H)
    g = oracle.nvfp4_global(float(np.abs(wf).max()))
    wp, bs = oracle.prep_nvfp4_rows(wf, g)
    return wp, bs, g


def test_nvfp4_edge_shapes(qh):
    for V, H, rows in [(1, 32, 1), (1001, 2080, 8), (77, 8224, 3), (513, 7168, 13),
                       (4096, 64, 9), (1001, 2080, 4), (1003, 8224, 16), (6, 12320, 4)]:
        log(f"[case] nvfp4 edge V={V} H={H} rows={rows}")
        wp, bs, g = _nvfp4_small(V, H)
        x = synth.activations_bf16(synth.NVFP4_Q6K_129280X7168, rows, hidden=H, max_rows=rows)
        out = qh.nvfp4(dev_u8(wp), dev_u8(bs), dev_bf16(x), g)
        torch.cuda.synchronize()
        ref, ad = oracle.nvfp4_ref(wp, bs, g, x)
        assert_within_bound(host_bits(out), ref, ad, f"nvfp4 edge V={V} H={H} rows={rows}")


def test_nvfp4_zero_global_scale(qh):
    wp, bs, _ = _nvfp4_small(64, 256)
    x = synth.activations_bf16(synth.NVFP4_Q6K_129280X7168, 2, hidden=256, max_rows=2)
    out = host_bits(qh.nvfp4(dev_u8(wp), dev_u8(bs), dev_bf16(x), 0.0))
    assert (bf16_bits_to_f64(out) == 0).all()


def test_nvfp4_129280x7168_full_head(qh):
    """The 129280 x 7168 head at every row count 1..16 (one weight pass each:
    8192-wide tiles up to 8 rows, 4096-wide above) and a 40-row call
    (16 + 16 + 8); sampled logits within the bound, row-invariant bits."""
    wp, bs, g, wpd, bsd = nvfp4_head()
    cfg = synth.CONFIGS[synth.NVFP4_Q6K_129280X7168]
    x = synth.activations_bf16(synth.NVFP4_Q6K_129280X7168, 40, max_rows=40)
    vidx = sample_vidx(cfg.vocab, 1500, 4)
    ref, ad = oracle.nvfp4_ref(wp, bs, g, x, vidx)
    outs = {}
    for R in list(range(1, 17)) + [40]:
        log(f"[case] nvfp4 129280x7168 R={R}")
        out = qh.nvfp4(wpd, bsd, dev_bf16(x[:R]), g)
        torch.cuda.synchronize()
        outs[R] = host_bits(out)
        assert_within_bound(outs[R][:, vidx], ref[:R], ad[:R], f"nvfp4 129280x7168 R={R}")
    for R in outs:
        assert np.array_equal(outs[R], outs[40][:R]), f"row invariance R={R}"


@pytest.mark.parametrize("H", [2048, 6144, 10240, 16416])
def test_nvfp4_row_invariance_across_tile_widths(qh, H):
    """Hidden sizes whose 4096-k reduction groups split differently into the
    8192-wide (<= 8 rows) and 4096-wide (9..16 rows) tiles."""
    V = 700
    wp, bs, g = _nvfp4_small(V, H)
    x = synth.activations_bf16(synth.NVFP4_Q6K_129280X7168, 16, hidden=H, max_rows=16)
    ref, ad = oracle.nvfp4_ref(wp, bs, g, x)
    wpd, bsd = dev_u8(wp), dev_u8(bs)
    outs = {}
    for R in (1, 3, 8, 9, 16):
        log(f"[case] nvfp4 tiles H={H} R={R}")
        outs[R] = host_bits(qh.nvfp4(wpd, bsd, dev_bf16(x[:R]), g))
        assert_within_bound(outs[R], ref[:R], ad[:R], f"nvfp4 H={H} R={R}")
    for R in outs:
        assert np.array_equal(outs[R], outs[16][:R]), f"row invariance H={H} R={R}"


# ------------------------------------------------------------------- q8_1

def test_quant_q8_1_bit_exact(qh):
    H, rows = 7168, 19
    x = synth.activations_bf16(synth.NVFP4_Q6K_129280X7168, rows, hidden=H, max_rows=rows)
    x[0, :64] = 0                        # two all-zero blocks
    x[1, :32] = 0x8000                   # a block of negative zeros
    ties = np.zeros(32, dtype=np.float32)
    ties[:8] = [127.0, 2.5, -3.5, 0.5, 1.5, -0.5, -127.0, 64.0]
    x[2, :32] = synth.to_bf16_bits(ties[None, :])[0]
    x[3, 32:64] = synth.to_bf16_bits(np.full((1, 32), 1e-30, dtype=np.float32))[0]
    log(f"[case] quant_q8_1 rows={rows} H={H}")
    q8 = qh.quant_q8_1(dev_bf16(x))
    torch.cuda.synchronize()
    assert np.array_equal(q8.cpu().numpy(), oracle.quant_q8_1(x))


# ------------------------------------------------------------------- Q6_K

def _q6k_small(V, H, cfg=synth.NVFP4_Q6K_129280X7168):
    wf = synth.weight_rows_f32(cfg, 0, V, vocab=V, hidden=H)
    return oracle.prep_q6k_rows(wf)


def test_q6k_every_q_every_position(qh):
    """Row v holds q = v (all 64 six-bit values) everywhere, scales vary by
    sub-block (including negative), d = 1; one-hot activations of 127 give
    q8 = 127 with d8 = 1, so every logit is exact."""
    V, H = 64, 256
    blocks = np.zeros((V, 210), dtype=np.uint8)
    for v in range(V):
        q = v
        blocks[v, 0:128] = (q & 15) | ((q & 15) << 4)
        hb = (q >> 4) & 3
        blocks[v, 128:192] = hb | (hb << 2) | (hb << 4) | (hb << 6)
        blocks[v, 192:208] = np.array([1, -1, 2, 3, -5, 7, 127, -128, 9, 11, 13, -17, 19, 23,
                                       29, 31], dtype=np.int8).view(np.uint8)
        blocks[v, 208], blocks[v, 209] = 0x00, 0x3C
    ks = [0, 1, 15, 16, 31, 32, 63, 64, 95, 96, 127, 128, 160, 192, 224, 255]
    x = np.zeros((len(ks), H), dtype=np.uint16)
    for i, k in enumerate(ks):
        x[i, k] = synth.to_bf16_bits(np.array([[127.0]], dtype=np.float32))[0, 0]
    q8 = oracle.quant_q8_1(x)
    log("[case] q6k one-hot")
    out = qh.q6k_gemv(dev_u8(blocks), dev_u8(q8), H)
    torch.cuda.synchronize()
    ref, _ = oracle.q6k_ref(blocks, q8, H)
    assert np.array_equal(host_bits(out), oracle.bf16_rne_array(ref))
    # the fused path (quantize inside the call) gives the same bits
    out2 = qh.q6k(dev_u8(blocks), dev_bf16(x))
    assert np.array_equal(host_bits(out2), host_bits(out))


def test_q6k_edge_shapes_and_alignment(qh):
    for V, H, rows in [(1, 256, 1), (333, 768, 8), (70, 8448, 3), (1001, 1280, 11)]:
        log(f"[case] q6k edge V={V} H={H} rows={rows}")
        blocks = _q6k_small(V, H)
        x = synth.activations_bf16(synth.NVFP4_Q6K_129280X7168, rows, hidden=H, max_rows=rows)
        q8 = oracle.quant_q8_1(x)
        ref, ad = oracle.q6k_ref(blocks, q8, H)
        out = qh.q6k(dev_u8(blocks), dev_bf16(x))
        torch.cuda.synchronize()
        assert_within_bound(host_bits(out), ref, ad, f"q6k edge V={V} H={H} rows={rows}")
        # the same blocks at a base address that is 2 mod 4
        big = torch.zeros(blocks.size + 2, dtype=torch.uint8, device=DEV)
        big[2:] = dev_u8(blocks).view(-1)
        shifted = big[2:].view(V, -1)
        assert shifted.data_ptr() % 4 == 2
        out2 = qh.q6k(shifted, dev_bf16(x))
        assert np.array_equal(host_bits(out2), host_bits(out))


def test_q6k_129280x7168_full_head(qh):
    blocks, bd = q6k_head()
    cfg = synth.CONFIGS[synth.NVFP4_Q6K_129280X7168]
    x = synth.activations_bf16(synth.NVFP4_Q6K_129280X7168, 8)
    q8 = oracle.quant_q8_1(x)
    vidx = sample_vidx(cfg.vocab, 1000, 5)
    ref, ad = oracle.q6k_ref(blocks, q8, cfg.hidden, vidx)
    ws = torch.empty((qh.q6k_workspace_bytes(cfg.hidden),), dtype=torch.uint8, device=DEV)
    outs = {}
    for R in range(1, 9):
        log(f"[case] q6k 129280x7168 R={R}")
        out = qh.q6k(bd, dev_bf16(x[:R]), workspace=ws)
        torch.cuda.synchronize()
        outs[R] = host_bits(out)
        assert_within_bound(outs[R][:, vidx], ref[:R], ad[:R], f"q6k 129280x7168 R={R}")
    for R in range(1, 9):
        assert np.array_equal(outs[R], outs[8][:R]), f"row invariance R={R}"
