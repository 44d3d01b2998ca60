"""GPU parity of the SiLU down-projection path against the CPU oracle,
through the C ABI (Python binding): the quantized activation bytes of
bf16(silu(gate) * up) bit-exact, the W8A8 logits within
|gpu - ref| <= 2^-7 |ref| + 1e-4 sum|x w|, and row-invariant bits.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import (DEV, assert_within_bound, dev_bf16, dev_f32, dev_u8, fp8_head,
                         host_bits, log, sample_vidx)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qh():
    import quantized_weight_decode_amd as m

    assert torch.cuda.is_available()
    return m


def _bits(v):
    return synth.to_bf16_bits(np.asarray(v, dtype=np.float32))


def _gate_up(rows, hidden, ld, seed):
    """Seeded gate/up [rows, ld] with edge rows planted in the first rows."""
    g, u = synth.gate_up_bf16(synth.SILU_DOWN_7168X18432, rows, hidden=ld, max_rows=rows)
    g, u = g.copy(), u.copy()
    rng = np.random.Generator(np.random.PCG64(seed))
    if rows > 1:
        u[1] = 0  # all-zero products
    if rows > 2:  # an exact BF16 midpoint (48 * (1 + 2^-7)) as the row maximum
        g[2, 0], u[2, 0] = 0x4240, 0x3F81
    if rows > 3:  # large |g|: silu(g) = g or ~0
        idx = rng.choice(hidden, size=min(hidden, 8), replace=False)
        g[3, idx] = _bits([60, -60, 100, -100, 30, -30, 12, -12][:idx.size])
    if rows > 4:  # subnormal BF16 products everywhere in the row
        g[4, :] = _bits(np.full(ld, 1e-30))
        u[4, :] = _bits(rng.uniform(-1e-9, 1e-9, ld))
    if rows > 5:  # tiny gate: silu(g) ~ g / 2
        g[5, :hidden // 2] = _bits(rng.uniform(-1e-6, 1e-6, hidden // 2))
    return g, u


def _check_products(got, ref, amb, what):
    """Bit-exact, except that an element the oracle flags as sitting on a BF16
    rounding boundary may take either neighbouring rounding."""
    bad = np.nonzero((got != ref) & ~amb)[0]
    assert bad.size == 0, f"{what}: {bad.size} products differ, first {bad[:5].tolist()}"
    loose = np.nonzero((got != ref) & amb)[0]
    for i in loose[:100]:
        assert abs(int(got[i]) - int(ref[i])) == 1, (what, i)


def test_silu_mul_every_gate_pattern(qh):
    """Every finite BF16 gate value times a spread of up values: the binary32
    fast path and its binary64 fallback against the binary64 oracle."""
    g_all = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    g_all = g_all[(g_all & 0x7F80) != 0x7F80]  # finite gates
    for ub in (0x3F80, 0xBF40, 0x4060, 0x3A83, 0x4348, 0x0001, 0xC2F7, 0x5F00):
        u = np.full(g_all.size, ub, dtype=np.uint16)
        log(f"[case] silu_mul all gates, up=0x{ub:04X}")
        out = host_bits(qh.silu_mul_bf16(dev_bf16(g_all), dev_bf16(u)))
        ref, amb = oracle.silu_mul_bf16_array(g_all, u)
        _check_products(out, ref, amb, f"up=0x{ub:04X}")


def test_silu_mul_random(qh):
    rng = np.random.Generator(np.random.PCG64(77))
    n = 1 << 22
    g = _bits(np.concatenate([rng.normal(0, 1.5, n // 2), rng.normal(0, 12, n // 2)]))
    u = _bits(rng.normal(0, 1, n) * np.exp(rng.uniform(-20, 20, n)))
    log("[case] silu_mul random 4M")
    out = host_bits(qh.silu_mul_bf16(dev_bf16(g), dev_bf16(u)))
    ref, amb = oracle.silu_mul_bf16_array(g, u)
    _check_products(out, ref, amb, "random")


@pytest.mark.parametrize("rows,hidden,ld", [(1, 16, 16), (7, 1040, 1048), (128, 18432, 18432),
                                            (300, 4096, 4104)])
def test_quant_act_silu_bit_exact(qh, rows, hidden, ld):
    g, u = _gate_up(rows, hidden, ld, 7 + rows)
    log(f"[case] quant_act_silu rows={rows} hidden={hidden} ld={ld}")
    xq, sa = qh.quant_act_silu_e4m3(dev_bf16(g), dev_bf16(u), hidden)
    torch.cuda.synchronize()
    rq, rs, amb = oracle.quant_act_silu_e4m3(g, u, hidden)
    got_q, got_s = xq.cpu().numpy(), sa.cpu().numpy()
    bad = np.argwhere(got_q != rq)
    assert np.array_equal(got_s.view(np.uint32), rs.view(np.uint32)), \
        f"scales differ in rows {np.nonzero(got_s != rs)[0][:5]} (ambiguous: {amb})"
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:5].tolist()} (ambiguous: {amb})"


def test_quant_act_silu_row_max_edges(qh):
    """Rows that stress how the quantizer finds the row maximum (a cheap
    screen of every product, then exact products only for the candidates):
    the maximum held by one element with a very negative gate and a huge up
    (silu(g) below 2^-100, so it is never screened), by an element with
    silu(g) ~ 5e-25, by the only product above 2^-100 in a row of products
    below it, products all within 2^-6 of each other (every one a candidate),
    a row of zeros with one tiny product, and a row of zeros with one
    negative zero. Scales and codes bit-exact."""
    H = 4096
    rng = np.random.Generator(np.random.PCG64(404))
    rows = 8
    g = _bits(rng.normal(0.0, 1.0, (rows, H)))
    u = _bits(rng.normal(0.0, 1e-6, (rows, H)))
    g[0, 777], u[0, 777] = _bits([-90.0])[0], _bits([1e38])[0]
    g[1, 5], u[1, 5] = _bits([-60.0])[0], _bits([1e20])[0]
    g[2, :] = _bits(np.full(H, 1e-20))
    u[2, :] = _bits(rng.uniform(-1e-12, 1e-12, H))
    g[2, 4000], u[2, 4000] = _bits([1e-15])[0], _bits([1e-15])[0]
    g[3, :] = _bits(np.full(H, 2.0))
    u[3, :] = _bits(1.0 - rng.integers(0, 4, H) * 2.0 ** -8)
    g[4, :] = 0
    u[4, :] = _bits(rng.normal(0.0, 1.0, H))
    g[4, 123], u[4, 123] = _bits([1e-25])[0], _bits([-1e-20])[0]
    g[5, :] = 0
    g[5, 9], u[5, 9] = 0x8000, 0x3F80
    g[6, ::2] = _bits(np.full(H // 2, -100.0))   # silu(g) ~ -4e-42
    u[6, ::2] = _bits(np.full(H // 2, 3e38))
    g[7, :] = _bits(rng.normal(0.0, 1.0, H))
    u[7, :] = _bits(np.full(H, 1.0))
    xq, sa = qh.quant_act_silu_e4m3(dev_bf16(g), dev_bf16(u), H)
    torch.cuda.synchronize()
    rq, rs, amb = oracle.quant_act_silu_e4m3(g, u, H)
    got_q, got_s = xq.cpu().numpy(), sa.cpu().numpy()
    assert np.array_equal(got_s.view(np.uint32), rs.view(np.uint32)), \
        f"scales differ in rows {np.nonzero(got_s.view(np.uint32) != rs.view(np.uint32))[0]}"
    bad = np.argwhere(got_q != rq)
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:5].tolist()} (ambiguous: {amb})"


def _fp8_weights(V, H, seed):
    wf = synth.weight_rows_f32(synth.SILU_DOWN_7168X18432, 0, V, vocab=V, hidden=H)
    return oracle.prep_fp8_rows(wf)


def test_w8a8_silu_logits_and_row_invariance(qh):
    V, H, ld = 1000, 2064, 2080
    w, s = _fp8_weights(V, H, 0)
    wd, sd = dev_u8(w), dev_f32(s)
    g, u = _gate_up(130, H, ld, 99)
    xq, sa, amb = oracle.quant_act_silu_e4m3(g, u, H)
    ref, ad = oracle.w8a8_ref(w, s, xq, sa)
    ws = qh.w8a8_workspace(H, DEV)
    outs = {}
    for R in (1, 5, 16, 40, 130):
        log(f"[case] w8a8_silu V={V} H={H} ld={ld} R={R}")
        out = qh.w8a8_silu(wd, sd, dev_bf16(g[:R]), dev_bf16(u[:R]), workspace=ws)
        torch.cuda.synchronize()
        outs[R] = host_bits(out)
        assert_within_bound(outs[R], ref[:R], ad[:R], f"w8a8_silu R={R}")
    for R in outs:
        assert np.array_equal(outs[R], outs[130][:R]), f"row invariance R={R}"
    # the fused call equals quantize-then-GEMV through the separate entry points
    dq, ds = qh.quant_act_silu_e4m3(dev_bf16(g), dev_bf16(u), H)
    two = host_bits(qh.w8a8_gemv(wd, sd, dq, ds))
    assert np.array_equal(two, outs[130])


def test_w8a8_silu_long_rows(qh):
    """An FFN width past the two-launch quantizer's 64 slices of 512 columns
    (33024 > 32768): the call quantizes in one launch instead; logits within
    the bound and equal to quantize-then-GEMV through the separate entry
    points."""
    V, H = 300, 33024
    w, s = _fp8_weights(V, H, 0)
    wd, sd = dev_u8(w), dev_f32(s)
    g, u = _gate_up(3, H, H, 5)
    xq, sa, _ = oracle.quant_act_silu_e4m3(g, u, H)
    ref, ad = oracle.w8a8_ref(w, s, xq, sa)
    log(f"[case] w8a8_silu V={V} H={H} R=3")
    out = host_bits(qh.w8a8_silu(wd, sd, dev_bf16(g), dev_bf16(u)))
    torch.cuda.synchronize()
    assert_within_bound(out, ref, ad, "w8a8_silu long rows")
    dq, ds = qh.quant_act_silu_e4m3(dev_bf16(g), dev_bf16(u), H)
    assert np.array_equal(dq.cpu().numpy(), xq)
    assert np.array_equal(host_bits(qh.w8a8_gemv(wd, sd, dq, ds)), out)


def test_w8a8_silu_full_size(qh):
    """The 7168 x 18432 down projection at rows 1, 16, 128 and 130 (a 128-row
    chunk plus 2); sampled outputs within the bound, row-invariant bits."""
    w, s, wd, sd = fp8_head(synth.SILU_DOWN_7168X18432)
    cfg = synth.CONFIGS[synth.SILU_DOWN_7168X18432]
    g, u = synth.gate_up_bf16(synth.SILU_DOWN_7168X18432, 130)
    xq, sa, amb = oracle.quant_act_silu_e4m3(g, u)
    assert amb == 0
    vidx = sample_vidx(cfg.vocab, 700, 5)
    ref, ad = oracle.w8a8_ref(w, s, xq, sa, vidx)
    ws = qh.w8a8_workspace(cfg.hidden, DEV)
    outs = {}
    for R in cfg.rows:
        log(f"[case] w8a8_silu 7168x18432 R={R}")
        out = qh.w8a8_silu(wd, sd, dev_bf16(g[:R]), dev_bf16(u[:R]), workspace=ws)
        torch.cuda.synchronize()
        outs[R] = host_bits(out)
        assert_within_bound(outs[R][:, vidx], ref[:R], ad[:R], f"7168x18432 R={R}")
    for R in cfg.rows:
        assert np.array_equal(outs[R], outs[130][:R]), f"row invariance R={R}"


def test_w8a8_silu_rejects_bad_shapes(qh):
    w = torch.zeros((64, 32), dtype=torch.uint8, device=DEV)
    s = torch.zeros((64,), dtype=torch.float32, device=DEV)
    g = torch.zeros((2, 40), dtype=torch.bfloat16, device=DEV)  # ld 40 % 8 == 0 but hidden 32 ok
    out = qh.w8a8_silu(w, s, g, g)
    assert out.shape == (2, 64)
    with pytest.raises(ValueError):  # ld < hidden: the binding's shape check
        qh.w8a8_silu(torch.zeros((64, 48), dtype=torch.uint8, device=DEV), s, g, g)
    with pytest.raises(qh.QheadError):  # ld % 8 != 0
        g2 = torch.zeros((2, 36), dtype=torch.bfloat16, device=DEV)
        qh.w8a8_silu(w, s, g2, g2)
