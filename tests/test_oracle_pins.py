"""Pins for the CPU oracle: each check ties an oracle function to something
other than itself -- values printed on the pages or worked by hand (fixtures
under tests/golden/), library casts (torch float8/bfloat16, numpy float16),
exact rational arithmetic on tiny inputs, a second computation of the same
dot product through numpy's float64 matmul, and invariants of the formats.

CPU only; these run with ``-m "not gpu"``.
"""

from fractions import Fraction
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line.split())
    return out


def _torch_e4m3_decode_all():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_e4m3_encode(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def _bits_f32(u):
    return np.array([u], dtype=np.uint32).view(np.float32)[0]


# ------------------------------------------------------------------ E4M3

def test_e4m3_hand_values():
    for code, val in _rows("e4m3_hand.txt"):
        got = oracle.e4m3_value(int(code, 16))
        assert got == float(val), code
        assert np.signbit(got) == val.startswith("-"), code


def test_e4m3_decode_all_codes_match_torch():
    ref = _torch_e4m3_decode_all()
    mine = oracle.e4m3_table()
    for c in range(256):
        if c in (0x7F, 0xFF):
            assert np.isnan(mine[c]) and np.isnan(ref[c])
        else:
            assert mine[c] == ref[c] and np.signbit(mine[c]) == np.signbit(ref[c]), hex(c)


def test_e4m3_encode_matches_torch_in_range():
    g = np.random.Generator(np.random.PCG64(7))
    vals = np.concatenate([
        g.standard_normal(20000).astype(np.float32) * np.float32(50),
        g.standard_normal(5000).astype(np.float32) * np.float32(0.01),
        (g.random(5000).astype(np.float32) * np.float32(463.9)),
    ])
    # every midpoint between adjacent grid values (the ties) and every grid value
    grid = np.array(sorted(set(oracle.e4m3_table()[:0x7F].tolist())), dtype=np.float64)
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (grid[1:] + grid[:-1]) / 2)  # ties exact in f32
    vals = np.concatenate([vals, mids, -mids, grid.astype(np.float32), -grid.astype(np.float32)])
    vals = vals[np.abs(vals) < 464]
    mine = oracle.enc_e4m3_array(vals)
    assert np.array_equal(mine, _torch_e4m3_encode(vals))


def test_e4m3_encode_brute_force_nearest_even():
    # nearest grid point by exhaustive search with exact rationals; ties -> even code
    grid = [(c, Fraction(oracle.e4m3_value(c))) for c in range(0x7F)]
    g = np.random.Generator(np.random.PCG64(8))
    samples = list(g.random(300).astype(np.float32) * np.float32(460)) + \
        list(g.random(100).astype(np.float32) * np.float32(0.02))
    for t in samples:
        a = Fraction(float(t))
        best = min(grid, key=lambda cv: (abs(cv[1] - a), cv[0] & 1))
        if a >= 448:
            best = (0x7E, None)
        assert oracle.enc_e4m3(float(t)) == best[0], float(t)
        assert oracle.enc_e4m3(-float(t)) == best[0] | 0x80


def test_e4m3_encode_saturation_and_signed_zero():
    assert oracle.enc_e4m3(448.0) == 0x7E
    assert oracle.enc_e4m3(1e30) == 0x7E
    assert oracle.enc_e4m3(-500.0) == 0xFE
    assert oracle.enc_e4m3(-1e-9) == 0x80
    assert oracle.enc_e4m3(-0.0) == 0x80
    assert oracle.enc_e4m3(0.0) == 0x00
    # subnormal ties: 0.5 * 2^-9 -> 0 (even), 1.5 * 2^-9 -> 2 * 2^-9
    assert oracle.enc_e4m3(2.0 ** -10) == 0x00
    assert oracle.enc_e4m3(1.5 * 2.0 ** -9) == 0x02
    # binade edge: 15.5 * 2^-10 rounds up into the first normal binade
    assert oracle.enc_e4m3(7.5 * 2.0 ** -9) == 0x08


# ------------------------------------------------------------------ E2M1

def test_e2m1_table_as_printed():
    for nib, val in _rows("e2m1_table.txt"):
        got = oracle.e2m1_value(int(nib))
        assert got == float(val)
        assert np.signbit(got) == val.startswith("-")


def test_e2m1_encode_ties_and_saturation():
    cases = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6, 7.0: 7, 100.0: 7,
             0.2: 0, 0.3: 1, 2.9: 5, -0.75: 10, -0.1: 8}
    for t, code in cases.items():
        assert oracle.enc_e2m1(t) == code, t


def test_nvfp4_hand_values():
    for byte, bs, g, v_even, v_odd in _rows("nvfp4_nibbles.txt"):
        b, s, gg = int(byte, 16), int(bs, 16), float(g)
        x = np.zeros((2, 2), dtype=np.uint16)
        x[0, 0] = 0x3F80  # one-hot k = 0
        x[1, 1] = 0x3F80  # one-hot k = 1
        # hidden must be a multiple of 16 for the block layout: pad the row
        wp = np.zeros((1, 8), dtype=np.uint8)
        wp[0, 0] = b
        bsr = np.array([[s]], dtype=np.uint8)
        xx = np.zeros((2, 16), dtype=np.uint16)
        xx[:, :2] = x
        ref, _ = oracle.nvfp4_ref(wp, bsr, gg, xx)
        assert ref[0, 0] == float(v_even)
        assert ref[1, 0] == float(v_odd)


# ------------------------------------------------------------ BF16 / FP16

def test_bf16_decode_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    f = oracle.lib().orc_bf16
    mine = np.array([f(int(b)) for b in bits], dtype=np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))


def test_bf16_rne_hand_ties():
    for val, bits in _rows("bf16_ties.txt"):
        assert oracle.bf16_rne(float(val)) == int(bits, 16), val


def test_bf16_rne_matches_torch_on_f32_inputs():
    g = np.random.Generator(np.random.PCG64(9))
    v = np.concatenate([g.standard_normal(20000) * 100, g.standard_normal(2000) * 1e-38,
                        g.standard_normal(2000) * 1e30]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_rne_array(v.astype(np.float64)), ref)


def test_fp16_decode_all_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    f = oracle.lib().orc_fp16
    mine = np.array([f(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))


def test_fp16_rne_matches_numpy():
    g = np.random.Generator(np.random.PCG64(10))
    v = np.concatenate([g.standard_normal(20000) * 10, g.standard_normal(5000) * 1e-5,
                        g.standard_normal(5000) * 1e-7, g.standard_normal(2000) * 7e4,
                        ]).astype(np.float32)
    # exact ties between fp16 neighbours, normal and subnormal
    ties = np.array([1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, 2 ** -24 * 0.5, 2 ** -24 * 1.5,
                     65520.0, 65519.0], dtype=np.float32)
    v = np.concatenate([v, ties, -ties])
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    f = oracle.lib().orc_fp16_rne
    mine = np.array([f(float(a)) for a in v], dtype=np.uint16)
    assert np.array_equal(mine, ref)


# ---------------------------------------------------- activation quantizers

def test_quant_act_e4m3_worked_row():
    rows = _rows("act_quant_row.txt")
    x = np.array([[int(b, 16) for b, _ in rows]], dtype=np.uint16)
    xq, sa = oracle.quant_act_e4m3(x)
    assert [int(c) for c in xq[0]] == [int(c, 16) for _, c in rows]
    assert sa.view(np.uint32)[0] == 0x3BDB6DB7


def test_quant_act_e4m3_properties():
    xf = synth.activations_f32(synth.FP8_32000X4096, 16, max_rows=16)
    x = synth.to_bf16_bits(xf)
    xq, sa = oracle.quant_act_e4m3(x)
    xv = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float().numpy()
    amax = np.abs(xv).max(axis=1)
    # scale is the binary32 quotient amax / 448 (numpy float32 division is IEEE)
    assert np.array_equal(sa, (amax / np.float32(448)).astype(np.float32))
    # the codes are torch's float8 rounding of the binary32 quotients
    t = (xv / sa[:, None]).astype(np.float32)
    assert np.array_equal(xq, _torch_e4m3_encode(t).reshape(xq.shape))
    # each row's largest magnitude lands on +-448
    for r in range(x.shape[0]):
        k = np.argmax(np.abs(xv[r]))
        assert xq[r, k] in (0x7E, 0xFE)
    # scaling x by 2 keeps the codes and doubles the scale exactly
    x2 = synth.to_bf16_bits(xf * 2)
    xq2, sa2 = oracle.quant_act_e4m3(x2)
    assert np.array_equal(xq2, xq)
    assert np.array_equal(sa2, sa * 2)


def test_quant_act_e4m3_zero_and_signed_zero_rows():
    x = np.zeros((3, 32), dtype=np.uint16)
    x[1, :] = 0x8000  # all negative zero
    x[2, 5] = 0xBF80  # -1 and zeros / negative zeros
    x[2, 6] = 0x8000
    xq, sa = oracle.quant_act_e4m3(x)
    assert sa[0] == 0 and sa[1] == 0 and not xq[:2].any()
    assert xq[2, 5] == 0xFE and xq[2, 6] == 0x80 and xq[2, 0] == 0x00


def test_quant_q8_1_worked_ties():
    rows = _rows("q8_1_ties.txt")
    x = np.zeros((1, 32), dtype=np.uint16)
    xs = np.zeros(32, dtype=np.float32)
    for i, (val, _) in enumerate(rows):
        xs[i] = float(val)
    x[0] = synth.to_bf16_bits(xs[None, :])[0]
    q8 = oracle.quant_q8_1(x)[0]
    assert int(q8[0]) | (int(q8[1]) << 8) == 0x3C00
    assert int(q8[2]) | (int(q8[3]) << 8) == 0x5400
    q = q8[4:].view(np.int8)
    for i, (_, qv) in enumerate(rows):
        assert q[i] == int(qv), i
    assert not q[len(rows):].any()


def test_quant_q8_1_properties():
    x = synth.activations_bf16(synth.NVFP4_Q6K_129280X7168, 3, hidden=256, max_rows=3)
    q8 = oracle.quant_q8_1(x).reshape(3, 8, 36)
    xv = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double().numpy().reshape(3, 8, 32)
    for r in range(3):
        for j in range(8):
            blk = q8[r, j]
            d16 = int(blk[0]) | (int(blk[1]) << 8)
            q = blk[4:].view(np.int8).astype(np.int64)
            amax = np.abs(xv[r, j]).max()
            d = np.float32(amax) / np.float32(127)
            assert d16 == np.array([d], dtype=np.float32).astype(np.float16).view(np.uint16)[0]
            # every code is within half a step of x / d, and the largest hits +-127
            assert np.all(np.abs(q * float(d) - xv[r, j]) <= float(d) * 0.5 * (1 + 1e-6))
            assert np.abs(q).max() == 127
            s16 = int(blk[2]) | (int(blk[3]) << 8)
            assert s16 == np.array([d * np.float32(q.sum())], dtype=np.float32).astype(
                np.float16).view(np.uint16)[0]


# ------------------------------------------------------------- Q6_K layout

def test_q6k_layout_hand_positions():
    for i, qb, nib, hb, sh, sc in _rows("q6k_hand.txt"):
        i, qb, hb, sh, sc = int(i), int(qb), int(hb), int(sh), int(sc)
        for q in (0, 1, 17, 31, 32, 40, 63):
            blk = np.zeros(210, dtype=np.uint8)
            blk[208], blk[209] = 0x00, 0x3C  # d = 1.0
            blk[192 + sc] = 3
            blk[qb] = (q & 15) if nib == "lo" else ((q & 15) << 4)
            blk[hb] = ((q >> 4) & 3) << sh
            w = oracle.q6k_decode_block(blk)
            expect = np.zeros(256)
            # every element reads low bits 0 / high bits 0 (q = 0) except i
            for e in range(256):
                expect[e] = 0.0 if (e // 16) != sc else 3.0 * (0 - 32)
            expect[i] = 3.0 * (q - 32)
            assert np.array_equal(w, expect), (i, q)


def test_q6k_worked_value_and_offset():
    blk = np.zeros(210, dtype=np.uint8)
    blk[208], blk[209] = 0x00, 0x3C
    blk[192] = 2
    blk[0] = 40 & 15
    blk[128] = (40 >> 4) & 3
    assert oracle.q6k_decode_block(blk)[0] == 16.0
    # q = 32 everywhere (ql 0x00, qh 0xAA sets high bits 2 for all quarters) is all zeros
    blk = np.zeros(210, dtype=np.uint8)
    blk[128:192] = 0xAA
    blk[192:208] = 77
    blk[208], blk[209] = 0x00, 0x3C
    assert not oracle.q6k_decode_block(blk).any()
    # negative int8 scale and fp16 subnormal d
    blk[192] = 0xFF  # -1
    blk[0] = 0x0F  # element 0: q = 47 -> 15
    blk[208], blk[209] = 0x01, 0x00  # d = 2^-24
    w = oracle.q6k_decode_block(blk)
    assert w[0] == -15 * 2.0 ** -24


# ------------------------------------------------------------- references

def _dequant_fp8_np(w, s):
    return _torch_e4m3_decode_all()[w] * s.astype(np.float64)[:, None]


def _close(a, b, rtol, abs_scale):
    assert np.all(np.abs(a - b) <= rtol * np.abs(b) + abs_scale), np.max(np.abs(a - b))


def _bf16_np(x):
    return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double().numpy()


def test_fp8_ref_matches_numpy_matmul():
    wf = synth.weight_rows_f32(synth.FP8_8192X1024, 0, 512)
    w, s = oracle.prep_fp8_rows(wf)
    x = synth.activations_bf16(synth.FP8_8192X1024, 3, max_rows=3)
    ref, ad = oracle.fp8_rowscale_ref(w, s, x)
    W = _dequant_fp8_np(w, s)
    X = _bf16_np(x)
    _close(ref, X @ W.T, 1e-12, 1e-12 * (np.abs(X) @ np.abs(W).T))
    np.testing.assert_allclose(ad, np.abs(X) @ np.abs(W).T, rtol=1e-12)
    # sampled vocab rows give the same values as the full matrix
    idx = np.array([5, 511, 0, 77])
    r2, _ = oracle.fp8_rowscale_ref(w, s, x, idx)
    assert np.array_equal(r2, ref[:, idx])


def test_fp8_ref_exact_rationals_tiny():
    g = np.random.Generator(np.random.PCG64(11))
    V, H, R = 5, 16, 3
    w = g.integers(0, 256, size=(V, H), dtype=np.uint8)
    w[(w & 0x7F) == 0x7F] = 0x3F  # no NaN codes
    s = np.array([0.5, 3.0, 2.0 ** -20, 1.75, 448.0], dtype=np.float32)
    x = synth.to_bf16_bits(g.standard_normal((R, H)).astype(np.float32))
    ref, _ = oracle.fp8_rowscale_ref(w, s, x)
    for r in range(R):
        for v in range(V):
            exact = sum(Fraction(oracle.bf16_value(x[r, k])) * Fraction(oracle.e4m3_value(w[v, k]))
                        for k in range(H)) * Fraction(float(s[v]))
            assert abs(Fraction(ref[r, v]) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + \
                Fraction(1, 2 ** 200)


def test_w8a8_ref_is_exact():
    g = np.random.Generator(np.random.PCG64(12))
    V, H, R = 4, 32, 3
    w = g.integers(0, 256, size=(V, H), dtype=np.uint8)
    w[(w & 0x7F) == 0x7F] = 0x7E
    xq = g.integers(0, 256, size=(R, H), dtype=np.uint8)
    xq[(xq & 0x7F) == 0x7F] = 0x01
    sw = np.array([1.0, 2.0 ** -9, 0.75, 4.0], dtype=np.float32)
    sa = np.array([2.0 ** -3, 1.0, 0.5], dtype=np.float32)
    ref, ad = oracle.w8a8_ref(w, sw, xq, sa)
    for r in range(R):
        for v in range(V):
            exact = sum(Fraction(oracle.e4m3_value(xq[r, k])) * Fraction(oracle.e4m3_value(w[v, k]))
                        for k in range(H))
            exact *= Fraction(float(sa[r])) * Fraction(float(sw[v]))
            assert Fraction(ref[r, v]) == exact


def test_w8a8_ref_matches_numpy_on_quantized_rows():
    wf = synth.weight_rows_f32(synth.W8A8_129280X7168, 0, 256, hidden=512)
    w, sw = oracle.prep_fp8_rows(wf)
    x = synth.activations_bf16(synth.W8A8_129280X7168, 5, hidden=512, max_rows=5)
    xq, sa = oracle.quant_act_e4m3(x)
    ref, _ = oracle.w8a8_ref(w, sw, xq, sa)
    T = _torch_e4m3_decode_all()
    A = T[xq] * sa.astype(np.float64)[:, None]
    W = T[w] * sw.astype(np.float64)[:, None]
    np.testing.assert_allclose(ref, A @ W.T, rtol=1e-12, atol=1e-13)


def test_nvfp4_ref_matches_numpy_matmul():
    V, H = 300, 512
    wf = synth.weight_rows_f32(synth.NVFP4_Q6K_129280X7168, 0, V, hidden=H)
    g = oracle.nvfp4_global(float(np.abs(wf).max()))
    wp, bs = oracle.prep_nvfp4_rows(wf, g)
    x = synth.activations_bf16(synth.NVFP4_Q6K_129280X7168, 4, hidden=H, max_rows=4)
    ref, ad = oracle.nvfp4_ref(wp, bs, g, x)
    table = np.array([float(v) for _, v in _rows("e2m1_table.txt")])
    nib = np.empty((V, H), dtype=np.uint8)
    nib[:, 0::2] = wp & 15
    nib[:, 1::2] = wp >> 4
    W = table[nib] * np.repeat(_torch_e4m3_decode_all()[bs], 16, axis=1) * g
    X = _bf16_np(x)
    _close(ref, X @ W.T, 1e-12, 1e-12 * (np.abs(X) @ np.abs(W).T))
    # the quantized weights stay close to the f32 draws (a sanity check of the prep recipe)
    assert np.abs(W - wf).max() <= np.abs(wf).max() / 6 * 1.1


def test_q6k_ref_matches_numpy_matmul():
    V, H = 64, 512
    wf = synth.weight_rows_f32(synth.NVFP4_Q6K_129280X7168, 0, V, hidden=H)
    blocks = oracle.prep_q6k_rows(wf)
    x = synth.activations_bf16(synth.NVFP4_Q6K_129280X7168, 3, hidden=H, max_rows=3)
    q8 = oracle.quant_q8_1(x)
    ref, _ = oracle.q6k_ref(blocks, q8, H)
    W = np.stack([np.concatenate([oracle.q6k_decode_block(blocks[v, b * 210:(b + 1) * 210])
                                  for b in range(H // 256)]) for v in range(V)])
    qb = q8.reshape(3, H // 32, 36)
    d = qb[:, :, 0:2].copy().view(np.float16).astype(np.float64).reshape(3, H // 32)
    q = qb[:, :, 4:].view(np.int8).astype(np.float64)
    A = (q * d[:, :, None]).reshape(3, H)
    np.testing.assert_allclose(ref, A @ W.T, rtol=1e-12, atol=1e-14)
    # the decoded Q6_K weights track the f32 draws
    assert np.abs(W - wf).max() < 0.25 * np.abs(wf).max()


def test_prep_fp8_rows_properties():
    wf = synth.weight_rows_f32(synth.FP8_155136X8192, 0, 64, hidden=1024)
    wf[3] = 0
    codes, s = oracle.prep_fp8_rows(wf)
    assert s[3] == 0 and not codes[3].any()
    T = _torch_e4m3_decode_all()
    for v in (0, 1, 63):
        amax = np.abs(wf[v]).max()
        assert s[v] == np.float32(amax) / np.float32(448)
        assert np.array_equal(codes[v], _torch_e4m3_encode(wf[v] / s[v]))
        assert np.abs(T[codes[v]]).max() == 448.0


def test_oracle_rows_independent_of_row_count():
    # a row's reference does not depend on which other rows are present
    wf = synth.weight_rows_f32(synth.FP8_8192X1024, 0, 128)
    w, s = oracle.prep_fp8_rows(wf)
    x = synth.activations_bf16(synth.FP8_8192X1024, 5, max_rows=5)
    full, _ = oracle.fp8_rowscale_ref(w, s, x)
    for r in range(5):
        one, _ = oracle.fp8_rowscale_ref(w, s, x[r:r + 1])
        assert np.array_equal(one[0], full[r])


def test_synth_row_ranges_are_stable():
    a = synth.weight_rows_f32(synth.FP8_32000X4096, 1000, 1100)
    b = synth.weight_rows_f32(synth.FP8_32000X4096, 0, 2048)[1000:1100]
    assert np.array_equal(a, b)
    x4 = synth.activations_f32(synth.FP8_32000X4096, 4)
    x40 = synth.activations_f32(synth.FP8_32000X4096, 40)
    assert np.array_equal(x4, x40[:4])
    cols = synth.outlier_columns(synth.FP8_32000X4096, 4096, 41)
    assert len(cols) == 41


# ------------------------------------------------ load-time FP4 -> BF16

def _g_value(tok):
    if tok.startswith("0x"):
        return float(_bits_f32(int(tok, 16)))
    return float(tok)


def test_e8m0_table_as_printed():
    for code, val in _rows("e8m0_table.txt"):
        assert oracle.e8m0_value(int(code)) == float(val), code


def test_e8m0_matches_exponent_field_construction():
    # 2^(e-127) is the binary32 whose exponent field is e and mantissa 0
    for e in range(1, 255):
        assert oracle.e8m0_value(e) == float(_bits_f32(e << 23)), e
    assert oracle.e8m0_value(0) == 0.0 and oracle.e8m0_value(255) == 0.0


def test_dequant_hand_values():
    for kind, byte, sc, g, even, odd in _rows("dequant_hand.txt"):
        b, s = int(byte, 16), int(sc, 0)
        if kind == "nvfp4":
            wp = np.zeros((1, 16), dtype=np.uint8)
            wp[0, 0] = b
            bs = np.array([[s, s]], dtype=np.uint8)
            out = oracle.dequant_nvfp4_bf16(wp, bs, _g_value(g))[0]
        else:
            packed = np.zeros(8, dtype=np.uint8)
            packed[0] = b
            out = oracle.dequant_fp4_e8m0_bf16(packed, np.array([s], dtype=np.uint8), 16)
        assert int(out[0]) == int(even, 16), (kind, byte, sc, g)
        assert int(out[1]) == int(odd, 16), (kind, byte, sc, g)
        assert not out[2:].any()


def _torch_e2m1_all():
    vals = [float(v) for _, v in _rows("e2m1_table.txt")]
    return torch.tensor(vals, dtype=torch.float32)


def _nibbles(packed: np.ndarray) -> np.ndarray:
    p = packed.reshape(-1)
    out = np.empty(p.size * 2, dtype=np.int64)
    out[0::2] = p & 15
    out[1::2] = p >> 4
    return out


def test_dequant_nvfp4_matches_torch_casts():
    # the same value built from library casts: E2M1 table values times the
    # torch float8_e4m3fn decode of the block scale, binary32 products, and
    # torch's BF16 cast (nearest even)
    rng = np.random.default_rng(11)
    n, k = 7, 96
    wp = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    bs = rng.integers(0, 256, size=(n, k // 16), dtype=np.uint8)
    bs[bs == 0x7F] = 0x41
    bs[bs == 0xFF] = 0xC1
    for g in (1.0, float(np.float32(0.37)), float(np.float32(3.1e-3)), 0.0):
        got = oracle.dequant_nvfp4_bf16(wp, bs, g)
        e2 = _torch_e2m1_all()[torch.from_numpy(_nibbles(wp))].reshape(n, k)
        s = torch.from_numpy(bs).view(torch.float8_e4m3fn).to(torch.float32)
        s = s.repeat_interleave(16, dim=1)
        y = (e2 * s) * torch.tensor(g, dtype=torch.float32)
        ref = y.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, ref), g


def test_dequant_e8m0_matches_torch_casts():
    rng = np.random.default_rng(12)
    groups, block = 256, 32
    total = groups * block
    packed = rng.integers(0, 256, size=total // 2, dtype=np.uint8)
    scales = np.arange(256, dtype=np.uint8)  # every code once
    got = oracle.dequant_fp4_e8m0_bf16(packed, scales, total)
    sc = torch.from_numpy((scales.astype(np.uint32) << 23).view(np.float32).copy())
    sc[0] = 0.0
    sc[255] = 0.0
    e2 = _torch_e2m1_all()[torch.from_numpy(_nibbles(packed))]
    y = e2 * sc.repeat_interleave(block)
    ref = y.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_dequant_e8m0_group_boundaries():
    # groups of 48 values: the scale changes exactly at flat index 48 and 96
    packed = np.full(72, 0x22, dtype=np.uint8)  # every nibble = 1.0
    out = oracle.dequant_fp4_e8m0_bf16(packed, np.array([127, 128, 126], dtype=np.uint8), 144)
    assert (out[:48] == 0x3F80).all() and (out[48:96] == 0x4000).all()
    assert (out[96:] == 0x3F00).all()


# ------------------------------------------- NVFP4 / Q6_K weight preparation

def test_prep_nvfp4_rows_nearest_codes():
    wf = synth.weight_rows_f32(synth.NVFP4_Q6K_129280X7168, 0, 24, hidden=512)
    wf[5] = 0
    g = oracle.nvfp4_global(float(np.abs(wf).max()))
    assert g == np.float32(np.abs(wf).max()) / np.float32(2688)
    packed, bs = oracle.prep_nvfp4_rows(wf, g)
    assert not packed[5].any() and not bs[5].any()
    T = _torch_e4m3_decode_all()
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    nib = _nibbles(packed).reshape(wf.shape)
    for v in (0, 1, 23):
        amax = np.abs(wf[v].reshape(-1, 16)).max(axis=1)
        code = _torch_e4m3_encode(amax / (np.float32(6) * np.float32(g)))
        assert np.array_equal(bs[v], code)
        step = (T[bs[v]].astype(np.float32) * np.float32(g)).repeat(16)
        t = np.abs((wf[v] / step).astype(np.float64))
        # brute force: the code's magnitude is a nearest E2M1 magnitude
        dist = np.abs(t[:, None] - mags[None, :])
        best = dist.min(axis=1)
        mine = dist[np.arange(t.size), nib[v] & 7]
        assert np.array_equal(mine, best)
        nz = (nib[v] & 7) != 0
        assert np.array_equal((nib[v][nz] >> 3) == 1, wf[v][nz] < 0)


def test_prep_q6k_rows_nearest_levels():
    wf = synth.weight_rows_f32(synth.NVFP4_Q6K_129280X7168, 0, 6, hidden=512)
    wf[2, :256] = 0
    blocks = oracle.prep_q6k_rows(wf)
    sb = blocks.reshape(6, 2, 210)
    zero = oracle.q6k_decode_block(sb[2, 0])
    assert not zero.any() and sb[2, 0, 208:].view(np.uint16)[0] == 0
    for v in (0, 3, 5):
        for b in range(2):
            w = wf[v, 256 * b:256 * (b + 1)]
            st = np.abs(w.reshape(16, 16)).max(axis=1) / np.float32(31)
            d16 = np.float16(st.max() / np.float32(127))
            assert sb[v, b, 208:].view(np.float16)[0] == d16
            d = np.float32(d16)
            sc = np.clip(np.rint(st / d), 0, 127).astype(np.int64)
            assert np.array_equal(sb[v, b, 192:208].astype(np.int64), sc)
            step = (d * sc.astype(np.float32)).repeat(16)
            dec = oracle.q6k_decode_block(sb[v, b])
            # decoded weights are the clamped nearest levels of the step grid
            q = np.clip(np.rint(w / step), -32, 31)
            assert np.array_equal(dec, q * step.astype(np.float64))


# ------------------------------------------- SiLU product act-quant (FFN down)

def test_silu_quant_worked_row():
    rows = _rows("silu_quant_row.txt")
    g = np.array([[int(r[0], 16) for r in rows]], dtype=np.uint16)
    u = np.array([[int(r[1], 16) for r in rows]], dtype=np.uint16)
    for r in rows:
        assert oracle.silu_mul_bf16(int(r[0], 16), int(r[1], 16)) == int(r[2], 16), r
    xq, sa, amb = oracle.quant_act_silu_e4m3(g, u)
    assert amb == 0
    assert sa[0] == np.float32(50) / np.float32(448)
    assert [int(c) for c in xq[0]] == [int(r[3], 16) for r in rows]


def _bf16_bits_of(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def test_silu_mul_matches_torch_silu():
    # torch's float64 silu times u, rounded by the (separately pinned) BF16 rounding
    rng = np.random.default_rng(21)
    g = _bf16_bits_of(np.concatenate([rng.normal(0, 2, 3000), rng.normal(0, 30, 500),
                                      [0.0, -0.0, 1e-30, -1e-30, 88.0, -88.0, 700.0]]))
    u = _bf16_bits_of(rng.normal(0, 1.5, g.size))
    gt = torch.from_numpy(bf16_bits_to_f64_local(g))
    ut = torch.from_numpy(bf16_bits_to_f64_local(u))
    ref = (torch.nn.functional.silu(gt) * ut).numpy()
    for i in range(g.size):
        want = oracle.bf16_rne(float(ref[i]))
        got = oracle.silu_mul_bf16(int(g[i]), int(u[i]))
        if oracle.silu_mul_ambiguous(int(g[i]), int(u[i])):
            continue
        assert got == want, (hex(int(g[i])), hex(int(u[i])), hex(got), hex(want))


def bf16_bits_to_f64_local(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def test_silu_mul_exact_midpoint_is_flagged():
    # silu(48) = 48 exactly in binary64 (1 + e^-48 rounds to 1); 48 * (1 + 2^-7)
    # = 48.375 is the midpoint of 48.25 and 48.5, and ties go to the even 48.5
    assert oracle.silu_mul_bf16(0x4240, 0x3F81) == 0x4242
    assert oracle.silu_mul_ambiguous(0x4240, 0x3F81)
    assert not oracle.silu_mul_ambiguous(0x3F80, 0x3F80)


def test_quant_act_silu_strided_rows_and_zero_row():
    rng = np.random.default_rng(22)
    rows, hidden, ld = 5, 96, 112
    g = _bf16_bits_of(rng.normal(0, 2, (rows, ld)))
    u = _bf16_bits_of(rng.normal(0, 1, (rows, ld)))
    u[3] = 0  # a row whose products are all zero (some -0)
    xq, sa, amb = oracle.quant_act_silu_e4m3(g, u, hidden)
    assert amb == 0 and xq.shape == (rows, hidden)
    assert sa[3] == 0 and not xq[3].any()
    p = np.array([[oracle.silu_mul_bf16(int(g[r, k]), int(u[r, k])) for k in range(hidden)]
                  for r in range(rows)], dtype=np.uint16)
    xq2, sa2 = oracle.quant_act_e4m3(p)
    assert np.array_equal(xq, xq2) and np.array_equal(sa, sa2)
    # columns past `hidden` do not matter
    g2 = g.copy()
    g2[:, hidden:] = 0x7F80
    xq3, sa3, _ = oracle.quant_act_silu_e4m3(g2, u, hidden)
    assert np.array_equal(xq, xq3) and np.array_equal(sa, sa3)
