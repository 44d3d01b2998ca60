"""GPU parity of the load-time kernels against the CPU oracle, through the C
ABI (Python binding): NVFP4 -> BF16 and E2M1/E8M0 -> BF16 dequantization,
and the NVFP4 and Q6_K weight quantizers that build the heads the GEMVs
read. All of these produce bytes, so the bar is bit-exact.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import DEV, dev_f32, dev_u8, host_bits, log, nvfp4_head, q6k_head, sample_vidx

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qh():
    import quantized_weight_decode_amd as m

    assert torch.cuda.is_available()
    return m


def _rand_bytes(seed, shape):
    return np.random.Generator(np.random.PCG64(seed)).integers(0, 256, size=shape, dtype=np.uint8)


def _finite_e4m3(codes):
    codes = codes.copy()
    codes[codes == 0x7F] = 0x7E  # the two NaN codes
    codes[codes == 0xFF] = 0xFE
    return codes


# -------------------------------------------------------- NVFP4 -> BF16

@pytest.mark.parametrize("n,k", [(1, 32), (37, 1056), (300, 7168), (5, 64)])
def test_dequant_nvfp4_bit_exact(qh, n, k):
    wp = _rand_bytes(51 + n, (n, k // 2))
    bs = _finite_e4m3(_rand_bytes(61 + n, (n, k // 16)))
    for g in (1.0, float(np.float32(0.0123)), float(np.float32(1.0 / 3.0)), 0.0):
        log(f"[case] dequant nvfp4 n={n} k={k} g={g}")
        out = qh.dequant_nvfp4_bf16(dev_u8(wp), dev_u8(bs), g)
        torch.cuda.synchronize()
        ref = oracle.dequant_nvfp4_bf16(wp, bs, g)
        assert np.array_equal(host_bits(out), ref), (n, k, g)


def test_dequant_nvfp4_every_nibble_every_scale(qh):
    # row r holds every nibble twice under block scale codes r and 255 - r
    n, k = 256, 32
    wp = np.tile(np.array([0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE], dtype=np.uint8),
                 (n, 2))
    codes = _finite_e4m3(np.arange(256, dtype=np.uint8))
    bs = np.stack([codes, codes[::-1]], axis=1)
    g = float(np.float32(0.7))
    log("[case] dequant nvfp4 all nibbles x all scales")
    out = qh.dequant_nvfp4_bf16(dev_u8(wp), dev_u8(bs), g)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), oracle.dequant_nvfp4_bf16(wp, bs, g))


def test_dequant_nvfp4_full_head_sampled(qh):
    wp, bs, g, wpd, bsd = nvfp4_head()
    cfg = synth.CONFIGS[synth.NVFP4_Q6K_129280X7168]
    log(f"[case] dequant nvfp4 full head {cfg.vocab}x{cfg.hidden}")
    out = qh.dequant_nvfp4_bf16(wpd, bsd, g)
    torch.cuda.synchronize()
    vidx = sample_vidx(cfg.vocab, 2000, 7)
    got = host_bits(out[torch.from_numpy(vidx).to(DEV)])
    ref = oracle.dequant_nvfp4_bf16(wp[vidx], bs[vidx], g)
    assert np.array_equal(got, ref)
    del out


# -------------------------------------------------- E2M1 + E8M0 -> BF16

@pytest.mark.parametrize("groups,block", [(256, 32), (7, 16), (3, 48), (1, 4096), (1000, 64)])
def test_dequant_e8m0_bit_exact(qh, groups, block):
    total = groups * block
    packed = _rand_bytes(71 + groups, (total // 2,))
    scales = _rand_bytes(81 + block, (groups,))
    if groups >= 256:
        scales[:256] = np.arange(256, dtype=np.uint8)  # every code, e = 0 and 255 included
    log(f"[case] dequant e8m0 groups={groups} block={block}")
    out = qh.dequant_fp4_e8m0_bf16(dev_u8(packed), dev_u8(scales))
    torch.cuda.synchronize()
    ref = oracle.dequant_fp4_e8m0_bf16(packed, scales, total)
    assert np.array_equal(host_bits(out), ref)


def test_dequant_e8m0_rejects_uneven_groups(qh):
    packed = torch.zeros(48, dtype=torch.uint8, device=DEV)
    with pytest.raises(qh.QheadError):
        qh.dequant_fp4_e8m0_bf16(packed, torch.zeros(5, dtype=torch.uint8, device=DEV))
    with pytest.raises(qh.QheadError):  # 96 values in 4 groups of 24
        qh.dequant_fp4_e8m0_bf16(packed, torch.zeros(4, dtype=torch.uint8, device=DEV))


# ------------------------------------------------- weight quantizers

def _weights_with_edges(rows, hidden, seed):
    wf = synth.weight_rows_f32(synth.NVFP4_Q6K_129280X7168, seed, seed + rows, hidden=hidden)
    wf[1] = 0.0
    wf[2, :256] = 1e-9      # Q6_K: d underflows binary16 to 0
    wf[3, :256] *= 1e-3     # Q6_K: d is a binary16 subnormal
    wf[4, 5] = 0.3          # an outlier in one block
    wf[5, :16] = -0.0
    wf[6, 16:32] = np.float32(0.015)  # a constant block: every value is its maximum
    return wf


@pytest.mark.parametrize("rows,hidden", [(1, 256), (300, 7168), (97, 2048)])
def test_quantize_nvfp4_rows_bit_exact(qh, rows, hidden):
    wf = _weights_with_edges(max(rows, 7), hidden, 3 * rows)[:rows]
    amax = float(np.abs(wf).max())
    for g in (oracle.nvfp4_global(amax), float(np.float32(1e-4)), 0.0):
        log(f"[case] quantize nvfp4 rows={rows} hidden={hidden} g={g}")
        wp, bs = qh.quantize_nvfp4_rows(dev_f32(wf), g)
        torch.cuda.synchronize()
        rp, rb = oracle.prep_nvfp4_rows(wf, g)
        assert np.array_equal(wp.cpu().numpy(), rp), g
        assert np.array_equal(bs.cpu().numpy(), rb), g


@pytest.mark.parametrize("rows,hidden", [(1, 256), (300, 7168), (97, 2048)])
def test_quantize_q6k_rows_bit_exact(qh, rows, hidden):
    wf = _weights_with_edges(max(rows, 7), hidden, 5 * rows)[:rows]
    log(f"[case] quantize q6k rows={rows} hidden={hidden}")
    blocks = qh.quantize_q6k_rows(dev_f32(wf))
    torch.cuda.synchronize()
    assert np.array_equal(blocks.cpu().numpy(), oracle.prep_q6k_rows(wf))


def test_quantize_full_heads_bit_exact(qh):
    """The 129280 x 7168 heads quantized on the GPU in one launch each match
    the oracle's chunked preparation byte for byte."""
    cfg = synth.CONFIGS[synth.NVFP4_Q6K_129280X7168]
    wp, bs, g, _, _ = nvfp4_head()
    blocks, _ = q6k_head()
    log(f"[case] quantize full heads {cfg.vocab}x{cfg.hidden}")
    wf = torch.empty((cfg.vocab, cfg.hidden), dtype=torch.float32, device=DEV)
    for lo, hi, chunk in synth.iter_weight_chunks(synth.NVFP4_Q6K_129280X7168):
        wf[lo:hi].copy_(torch.from_numpy(chunk))
    gwp, gbs = qh.quantize_nvfp4_rows(wf, g)
    gbl = qh.quantize_q6k_rows(wf)
    torch.cuda.synchronize()
    del wf
    assert np.array_equal(gwp.cpu().numpy(), wp)
    assert np.array_equal(gbs.cpu().numpy(), bs)
    assert np.array_equal(gbl.cpu().numpy(), blocks)
