"""Heads larger than 2 GiB: the rows past byte offset 2^31 (where 32-bit
offset arithmetic would wrap) decode correctly. Weights are drawn on the
device; sampled rows are copied back and checked against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import DEV, assert_within_bound, dev_bf16, host_bits, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qh():
    import quantized_weight_decode_amd as m

    assert torch.cuda.is_available()
    return m


def _sample_rows(V, first_high):
    rows = list(range(0, 8)) + list(range(first_high - 8, first_high + 8)) + list(range(V - 8, V))
    g = np.random.Generator(np.random.PCG64(5))
    rows += list(g.integers(first_high, V, size=24))
    return np.unique(np.array(rows, dtype=np.int64))


def test_fp8_head_beyond_2gib(qh):
    V, H, R = 266240, 8192, 3                 # 2.18 GB of E4M3 weights
    first_high = (1 << 31) // H               # first row that starts at or past 2^31
    log(f"[case] fp8 {V}x{H} ({V * H / 2**30:.2f} GiB) rows={R}")
    gen = torch.Generator(device=DEV).manual_seed(123)
    w = torch.randint(0, 256, (V, H), dtype=torch.uint8, device=DEV, generator=gen)
    for lo in range(0, V, 1 << 15):           # no NaN codes (elementwise, in row blocks)
        blk = w[lo:lo + (1 << 15)]
        blk ^= ((blk & 0x7F) == 0x7F).to(torch.uint8)
    s = torch.rand(V, dtype=torch.float32, device=DEV, generator=gen) * 1e-3 + 1e-4
    x = synth.activations_bf16(synth.FP8_155136X8192, 40, max_rows=40)
    out = qh.fp8_rowscale(w, s, dev_bf16(x[:R]))
    out8 = qh.w8a8(w, s, dev_bf16(x[:R]))      # the W8A8 variant of the same kernel
    # W8A8 on its MFMA kernel: 16 rows (weights through LDS) and 40 rows
    # (direct weight loads, activations from the staged image)
    out8_16 = qh.w8a8(w, s, dev_bf16(x[:16]))
    out8_40 = qh.w8a8(w, s, dev_bf16(x))
    torch.cuda.synchronize()
    rows = _sample_rows(V, first_high)
    idx = torch.from_numpy(rows).to(DEV)
    w_h, s_h = w[idx].cpu().numpy(), s[idx].cpu().numpy()
    got, got8 = host_bits(out[:, idx]), host_bits(out8[:, idx])
    got8_16, got8_40 = host_bits(out8_16[:, idx]), host_bits(out8_40[:, idx])
    del w
    ref, ad = oracle.fp8_rowscale_ref(w_h, s_h, x[:R])
    assert_within_bound(got, ref, ad, "fp8 beyond 2 GiB")
    xq, sa = oracle.quant_act_e4m3(x)
    ref8, ad8 = oracle.w8a8_ref(w_h, s_h, xq, sa)
    assert_within_bound(got8, ref8[:R], ad8[:R], "w8a8 beyond 2 GiB")
    assert_within_bound(got8_40, ref8, ad8, "w8a8 40 rows beyond 2 GiB")
    assert np.array_equal(got8_16, got8_40[:16]), "w8a8 beyond 2 GiB: 16-row call differs"
    assert np.array_equal(got8, got8_40[:R]), "w8a8 beyond 2 GiB: 3-row call differs"


def test_q6k_head_beyond_2gib(qh):
    V, H, R = 368640, 7168, 2                 # 2.17 GB of Q6_K super-blocks
    rowbytes = H // 256 * 210
    first_high = (1 << 31) // rowbytes
    log(f"[case] q6k {V}x{H} ({V * rowbytes / 2**30:.2f} GiB) rows={R}")
    gen = torch.Generator(device=DEV).manual_seed(321)
    blocks = torch.randint(0, 256, (V, rowbytes), dtype=torch.uint8, device=DEV, generator=gen)
    d = blocks.view(V, H // 256, 210)
    # fp16 d in [2^-12, 2^-8): exponent field 3..6, any mantissa, positive
    d[:, :, 209] = (d[:, :, 209] & 0x03) | 0x0C
    x = synth.activations_bf16(synth.NVFP4_Q6K_129280X7168, R, max_rows=R)
    out = qh.q6k(blocks, dev_bf16(x))
    torch.cuda.synchronize()
    rows = _sample_rows(V, first_high)
    idx = torch.from_numpy(rows).to(DEV)
    b_h = blocks[idx].cpu().numpy()
    got = host_bits(out[:, idx])
    del blocks, d
    ref, ad = oracle.q6k_ref(b_h, oracle.quant_q8_1(x), H)
    assert_within_bound(got, ref, ad, "q6k beyond 2 GiB")


def test_nvfp4_head_and_dequant_beyond_2gib(qh):
    V, H, R = 600064, 7168, 2                 # 2.15 GB of packed nibbles (+0.27 GB scales)
    first_high = (1 << 31) // (H // 2)
    log(f"[case] nvfp4 {V}x{H} ({V * H / 2 / 2**30:.2f} GiB packed) rows={R}")
    gen = torch.Generator(device=DEV).manual_seed(77)
    wp = torch.randint(0, 256, (V, H // 2), dtype=torch.uint8, device=DEV, generator=gen)
    # block scales: finite E4M3 codes 0x28..0x47 (2^-2 .. 2^1.9)
    bs = torch.randint(0x28, 0x48, (V, H // 16), dtype=torch.uint8, device=DEV, generator=gen)
    g = 0.01
    x = synth.activations_bf16(synth.NVFP4_Q6K_129280X7168, R, max_rows=R)
    out = qh.nvfp4(wp, bs, dev_bf16(x), g)
    torch.cuda.synchronize()
    rows = _sample_rows(V, first_high)
    idx = torch.from_numpy(rows).to(DEV)
    wp_h, bs_h = wp[idx].cpu().numpy(), bs[idx].cpu().numpy()
    ref, ad = oracle.nvfp4_ref(wp_h, bs_h, g, x)
    assert_within_bound(host_bits(out[:, idx]), ref, ad, "nvfp4 beyond 2 GiB")
    # load-time dequant of the same head: flat element indices pass 2^32
    deq = qh.dequant_nvfp4_bf16(wp, bs, g)
    torch.cuda.synchronize()
    got = host_bits(deq[idx])
    del deq, wp, bs
    assert np.array_equal(got, oracle.dequant_nvfp4_bf16(wp_h, bs_h, g))
