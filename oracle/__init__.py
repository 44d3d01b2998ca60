"""CPU oracle for the quantized few-row LM-head GEMV.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library. It shares no code with the
HIP path; its arithmetic lives in ``qhead_oracle.c`` (plain C, binary64
accumulation, sequential k) and this module only marshals numpy arrays.

What each function computes, and which page passage it follows, is stated in
the C source next to the function. In short:

  fp8_rowscale_ref   ref = s[v] * sum_k bf16(x) e4m3(W)         ("lm_head_fp8_rows.rs")
  quant_act_e4m3     per-row E4M3 activations, sa = amax/448    ("w8a8_layer.rs")
  w8a8_ref           ref = sa[r] sw[v] sum_k e4m3(xq) e4m3(W)   (exact sum)
  nvfp4_ref          ref = g sum_k bf16(x) e2m1 e4m3(bs)        ("fp8_lut.rs")
  quant_q8_1         block_q8_1 of 32 values                    ("lm_head_q6k.rs")
  q6k_ref            ref = sum_k (d sc (q-32)) (d16 q8)         ("lm_head_q6k.rs")

Parity pins (tests/test_oracle_pins.py) tie every function to hand-worked
values, library casts, exact rational arithmetic or a second, independent
computation. The Q6_K byte placement inside a super-block follows the public
GGUF layout; no GGUF file is available, so compatibility with real files is
parity unpinned (the GPU and the oracle read the same documented layout).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qhead_oracle.c")
_LIB_DIR = os.path.join(_HERE, "_build")
_LIB = os.path.join(_LIB_DIR, "liboracle.so")

Q8_BLOCK_BYTES = 36
Q6K_BLOCK_BYTES = 210

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE floating point, no contraction)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    os.makedirs(_LIB_DIR, exist_ok=True)
    tmp = _LIB + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _P(t):
    return ctypes.POINTER(t)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        u8p, u16p, f32p, f64p, i64p = _P(ctypes.c_uint8), _P(ctypes.c_uint16), _P(ctypes.c_float), \
            _P(ctypes.c_double), _P(ctypes.c_int64)
        i32, i64 = ctypes.c_int, ctypes.c_int64
        sig = {
            "orc_num_threads": (ctypes.c_int, []),
            "orc_e4m3": (ctypes.c_double, [ctypes.c_uint8]),
            "orc_e2m1": (ctypes.c_double, [ctypes.c_uint8]),
            "orc_bf16": (ctypes.c_double, [ctypes.c_uint16]),
            "orc_fp16": (ctypes.c_double, [ctypes.c_uint16]),
            "orc_enc_e4m3": (ctypes.c_uint8, [ctypes.c_float]),
            "orc_enc_e2m1": (ctypes.c_uint8, [ctypes.c_float]),
            "orc_fp16_rne": (ctypes.c_uint16, [ctypes.c_float]),
            "orc_bf16_rne": (ctypes.c_uint16, [ctypes.c_double]),
            "orc_quant_act_e4m3": (None, [u16p, i32, i32, u8p, f32p]),
            "orc_quant_q8_1": (None, [u16p, i32, i32, u8p]),
            "orc_q6k_decode_block": (None, [u8p, f64p]),
            "orc_fp8_rowscale": (None, [u8p, f32p, u16p, i32, i32, i32, i64p, i32, f64p, f64p]),
            "orc_w8a8": (None, [u8p, f32p, u8p, f32p, i32, i32, i32, i64p, i32, f64p, f64p]),
            "orc_nvfp4": (None, [u8p, u8p, ctypes.c_float, u16p, i32, i32, i32, i64p, i32, f64p,
                                 f64p]),
            "orc_q6k": (None, [u8p, u8p, i32, i32, i32, i64p, i32, f64p, f64p]),
            "orc_prep_fp8_rows": (None, [_P(ctypes.c_float), i64, i32, u8p, f32p]),
            "orc_prep_nvfp4_global": (ctypes.c_float, [ctypes.c_float]),
            "orc_prep_nvfp4_rows": (None, [f32p, i64, i32, ctypes.c_float, u8p, u8p]),
            "orc_prep_q6k_rows": (None, [f32p, i64, i32, u8p]),
            "orc_dequant_nvfp4_bf16": (None, [u8p, u8p, ctypes.c_float, i64, i32, u16p]),
            "orc_e8m0": (ctypes.c_double, [ctypes.c_uint8]),
            "orc_dequant_fp4_e8m0_bf16": (None, [u8p, u8p, i64, i64, u16p]),
            "orc_silu_mul_bf16": (ctypes.c_uint16, [ctypes.c_uint16, ctypes.c_uint16]),
            "orc_silu_mul_ambiguous": (ctypes.c_int, [ctypes.c_uint16, ctypes.c_uint16]),
            "orc_quant_act_silu_e4m3": (i64, [u16p, u16p, i32, i32, i32, u8p, f32p]),
            "orc_silu_mul_bf16_array": (None, [u16p, u16p, i64, u16p, u8p]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(a: np.ndarray, ctype):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(_P(ctype))


# ---------------------------------------------------------------- scalars

def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().orc_num_threads())


def e4m3_value(code: int) -> float:
    return lib().orc_e4m3(int(code) & 0xFF)


def e2m1_value(nibble: int) -> float:
    return lib().orc_e2m1(int(nibble) & 0xF)


def bf16_value(bits: int) -> float:
    return lib().orc_bf16(int(bits) & 0xFFFF)


def fp16_value(bits: int) -> float:
    return lib().orc_fp16(int(bits) & 0xFFFF)


def enc_e4m3(t: float) -> int:
    return int(lib().orc_enc_e4m3(float(t)))


def enc_e2m1(t: float) -> int:
    return int(lib().orc_enc_e2m1(float(t)))


def fp16_rne(f: float) -> int:
    return int(lib().orc_fp16_rne(float(f)))


def bf16_rne(v: float) -> int:
    return int(lib().orc_bf16_rne(float(v)))


def e4m3_table() -> np.ndarray:
    """All 256 E4M3 decodes as float64 (NaN for 0x7F and 0xFF)."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def enc_e4m3_array(t: np.ndarray) -> np.ndarray:
    t = np.ascontiguousarray(t, dtype=np.float32).ravel()
    f = lib().orc_enc_e4m3
    return np.array([f(float(v)) for v in t], dtype=np.uint8)


def bf16_rne_array(v: np.ndarray) -> np.ndarray:
    f = lib().orc_bf16_rne
    flat = np.ascontiguousarray(v, dtype=np.float64).ravel()
    return np.array([f(float(a)) for a in flat], dtype=np.uint16).reshape(np.shape(v))


# ------------------------------------------------------------ quantizers

def quant_act_e4m3(x_bf16: np.ndarray):
    """Per-row E4M3 activation quantization: returns (xq uint8 [R,H], sa float32 [R])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, hidden = x.shape
    xq = np.empty((rows, hidden), dtype=np.uint8)
    sa = np.empty(rows, dtype=np.float32)
    lib().orc_quant_act_e4m3(_ptr(x, ctypes.c_uint16), rows, hidden, _ptr(xq, ctypes.c_uint8),
                             _ptr(sa, ctypes.c_float))
    return xq, sa


def silu_mul_bf16(g_bits: int, u_bits: int) -> int:
    """bf16(silu(g) * u) from BF16 bit patterns, silu and product in binary64."""
    return int(lib().orc_silu_mul_bf16(int(g_bits) & 0xFFFF, int(u_bits) & 0xFFFF))


def silu_mul_ambiguous(g_bits: int, u_bits: int) -> bool:
    return bool(lib().orc_silu_mul_ambiguous(int(g_bits) & 0xFFFF, int(u_bits) & 0xFFFF))


def silu_mul_bf16_array(g_bits: np.ndarray, u_bits: np.ndarray):
    """Elementwise bf16(silu(g) * u) bits and ambiguity flags (same shape)."""
    g = np.ascontiguousarray(g_bits, dtype=np.uint16)
    u = np.ascontiguousarray(u_bits, dtype=np.uint16)
    assert g.shape == u.shape
    out = np.empty(g.shape, dtype=np.uint16)
    amb = np.empty(g.shape, dtype=np.uint8)
    lib().orc_silu_mul_bf16_array(_ptr(g, ctypes.c_uint16), _ptr(u, ctypes.c_uint16), g.size,
                                  _ptr(out, ctypes.c_uint16), _ptr(amb, ctypes.c_uint8))
    return out, amb.astype(bool)


def quant_act_silu_e4m3(gate_bf16: np.ndarray, up_bf16: np.ndarray, hidden: int | None = None):
    """Per-row E4M3 quantization of bf16(silu(gate) * up) over the first
    `hidden` columns of gate/up ([R, ld] BF16 bits). Returns (xq uint8 [R, hidden],
    sa float32 [R], number of ambiguous elements)."""
    g = np.ascontiguousarray(gate_bf16, dtype=np.uint16)
    u = np.ascontiguousarray(up_bf16, dtype=np.uint16)
    assert g.shape == u.shape
    rows, ld = g.shape
    hidden = ld if hidden is None else hidden
    xq = np.empty((rows, hidden), dtype=np.uint8)
    sa = np.empty(rows, dtype=np.float32)
    amb = lib().orc_quant_act_silu_e4m3(_ptr(g, ctypes.c_uint16), _ptr(u, ctypes.c_uint16), ld,
                                        rows, hidden, _ptr(xq, ctypes.c_uint8),
                                        _ptr(sa, ctypes.c_float))
    return xq, sa, int(amb)


def quant_q8_1(x_bf16: np.ndarray) -> np.ndarray:
    """block_q8_1 quantization: uint8 [R, (H/32)*36]."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, hidden = x.shape
    if hidden % 32:
        raise ValueError("hidden must be a multiple of 32")
    q8 = np.empty((rows, hidden // 32 * Q8_BLOCK_BYTES), dtype=np.uint8)
    lib().orc_quant_q8_1(_ptr(x, ctypes.c_uint16), rows, hidden, _ptr(q8, ctypes.c_uint8))
    return q8


def q6k_decode_block(block: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(block, dtype=np.uint8)
    assert b.size == Q6K_BLOCK_BYTES
    out = np.empty(256, dtype=np.float64)
    lib().orc_q6k_decode_block(_ptr(b, ctypes.c_uint8), _ptr(out, ctypes.c_double))
    return out


# ------------------------------------------------------------ references

def _vidx(vocab: int, vidx):
    if vidx is None:
        return np.arange(vocab, dtype=np.int64)
    v = np.ascontiguousarray(vidx, dtype=np.int64)
    if v.size and (v.min() < 0 or v.max() >= vocab):
        raise IndexError("vocab index out of range")
    return v


def fp8_rowscale_ref(w: np.ndarray, s: np.ndarray, x_bf16: np.ndarray, vidx=None):
    """(ref, absdot), each float64 [R, len(vidx)]."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.float32)
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    vocab, hidden = w.shape
    rows = x.shape[0]
    v = _vidx(vocab, vidx)
    ref = np.empty((rows, v.size), dtype=np.float64)
    ad = np.empty_like(ref)
    lib().orc_fp8_rowscale(_ptr(w, ctypes.c_uint8), _ptr(s, ctypes.c_float),
                           _ptr(x, ctypes.c_uint16), rows, hidden, vocab,
                           _ptr(v, ctypes.c_int64), v.size, _ptr(ref, ctypes.c_double),
                           _ptr(ad, ctypes.c_double))
    return ref, ad


def w8a8_ref(w: np.ndarray, sw: np.ndarray, xq: np.ndarray, sa: np.ndarray, vidx=None):
    w = np.ascontiguousarray(w, dtype=np.uint8)
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    xq = np.ascontiguousarray(xq, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    vocab, hidden = w.shape
    rows = xq.shape[0]
    v = _vidx(vocab, vidx)
    ref = np.empty((rows, v.size), dtype=np.float64)
    ad = np.empty_like(ref)
    lib().orc_w8a8(_ptr(w, ctypes.c_uint8), _ptr(sw, ctypes.c_float), _ptr(xq, ctypes.c_uint8),
                   _ptr(sa, ctypes.c_float), rows, hidden, vocab, _ptr(v, ctypes.c_int64), v.size,
                   _ptr(ref, ctypes.c_double), _ptr(ad, ctypes.c_double))
    return ref, ad


def nvfp4_ref(wp: np.ndarray, bs: np.ndarray, g: float, x_bf16: np.ndarray, vidx=None):
    wp = np.ascontiguousarray(wp, dtype=np.uint8)
    bs = np.ascontiguousarray(bs, dtype=np.uint8)
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    vocab = wp.shape[0]
    hidden = wp.shape[1] * 2
    assert bs.shape == (vocab, hidden // 16)
    rows = x.shape[0]
    v = _vidx(vocab, vidx)
    ref = np.empty((rows, v.size), dtype=np.float64)
    ad = np.empty_like(ref)
    lib().orc_nvfp4(_ptr(wp, ctypes.c_uint8), _ptr(bs, ctypes.c_uint8), float(g),
                    _ptr(x, ctypes.c_uint16), rows, hidden, vocab, _ptr(v, ctypes.c_int64),
                    v.size, _ptr(ref, ctypes.c_double), _ptr(ad, ctypes.c_double))
    return ref, ad


def q6k_ref(blocks: np.ndarray, q8: np.ndarray, hidden: int, vidx=None):
    """blocks uint8 [V, hidden/256*210]; q8 uint8 [R, hidden/32*36]."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8)
    q = np.ascontiguousarray(q8, dtype=np.uint8)
    vocab = b.shape[0]
    assert b.shape[1] == hidden // 256 * Q6K_BLOCK_BYTES
    rows = q.shape[0]
    v = _vidx(vocab, vidx)
    ref = np.empty((rows, v.size), dtype=np.float64)
    ad = np.empty_like(ref)
    lib().orc_q6k(_ptr(b, ctypes.c_uint8), _ptr(q, ctypes.c_uint8), rows, hidden, vocab,
                  _ptr(v, ctypes.c_int64), v.size, _ptr(ref, ctypes.c_double),
                  _ptr(ad, ctypes.c_double))
    return ref, ad


# ------------------------------------------------------- data preparation

def prep_fp8_rows(wf: np.ndarray):
    """float32 [V,H] -> (E4M3 codes uint8 [V,H], row scales float32 [V])."""
    wf = np.ascontiguousarray(wf, dtype=np.float32)
    n, hidden = wf.shape
    codes = np.empty((n, hidden), dtype=np.uint8)
    scales = np.empty(n, dtype=np.float32)
    lib().orc_prep_fp8_rows(_ptr(wf, ctypes.c_float), n, hidden, _ptr(codes, ctypes.c_uint8),
                            _ptr(scales, ctypes.c_float))
    return codes, scales


def nvfp4_global(amax_all: float) -> float:
    return float(lib().orc_prep_nvfp4_global(float(amax_all)))


def prep_nvfp4_rows(wf: np.ndarray, g: float):
    """float32 [V,H] with global g -> (packed uint8 [V,H/2], block scales uint8 [V,H/16])."""
    wf = np.ascontiguousarray(wf, dtype=np.float32)
    n, hidden = wf.shape
    packed = np.empty((n, hidden // 2), dtype=np.uint8)
    bs = np.empty((n, hidden // 16), dtype=np.uint8)
    lib().orc_prep_nvfp4_rows(_ptr(wf, ctypes.c_float), n, hidden, float(g),
                              _ptr(packed, ctypes.c_uint8), _ptr(bs, ctypes.c_uint8))
    return packed, bs


def prep_q6k_rows(wf: np.ndarray) -> np.ndarray:
    """float32 [V,H] -> Q6_K super-blocks uint8 [V, H/256*210]."""
    wf = np.ascontiguousarray(wf, dtype=np.float32)
    n, hidden = wf.shape
    if hidden % 256:
        raise ValueError("hidden must be a multiple of 256")
    blocks = np.empty((n, hidden // 256 * Q6K_BLOCK_BYTES), dtype=np.uint8)
    lib().orc_prep_q6k_rows(_ptr(wf, ctypes.c_float), n, hidden, _ptr(blocks, ctypes.c_uint8))
    return blocks


def prep_config_weights(cfg_index: int, fmt: str, *, vocab=None, hidden=None, std=None):
    """Quantize a whole synthetic head, chunk by chunk, with the oracle's
    data-preparation quantizers. fmt: "fp8" -> (codes, scales);
    "nvfp4" -> (packed, bs, g); "q6k" -> blocks."""
    import synth

    cfg = synth.CONFIGS[cfg_index]
    vocab = vocab if vocab is not None else cfg.vocab
    hidden = hidden if hidden is not None else cfg.hidden
    if fmt == "fp8":
        codes = np.empty((vocab, hidden), dtype=np.uint8)
        scales = np.empty(vocab, dtype=np.float32)
        for lo, hi, wf in synth.iter_weight_chunks(cfg_index, vocab=vocab, hidden=hidden, std=std):
            c, s = prep_fp8_rows(wf)
            codes[lo:hi] = c
            scales[lo:hi] = s
        return codes, scales
    if fmt == "nvfp4":
        amax = np.float32(0.0)
        for _, _, wf in synth.iter_weight_chunks(cfg_index, vocab=vocab, hidden=hidden, std=std):
            amax = max(amax, np.float32(np.abs(wf).max()))
        g = nvfp4_global(float(amax))
        packed = np.empty((vocab, hidden // 2), dtype=np.uint8)
        bs = np.empty((vocab, hidden // 16), dtype=np.uint8)
        for lo, hi, wf in synth.iter_weight_chunks(cfg_index, vocab=vocab, hidden=hidden, std=std):
            p, b = prep_nvfp4_rows(wf, g)
            packed[lo:hi] = p
            bs[lo:hi] = b
        return packed, bs, g
    if fmt == "q6k":
        blocks = np.empty((vocab, hidden // 256 * Q6K_BLOCK_BYTES), dtype=np.uint8)
        for lo, hi, wf in synth.iter_weight_chunks(cfg_index, vocab=vocab, hidden=hidden, std=std):
            blocks[lo:hi] = prep_q6k_rows(wf)
        return blocks
    raise ValueError(fmt)


# ------------------------------------------------------ load-time dequant

def e8m0_value(code: int) -> float:
    return float(lib().orc_e8m0(int(code) & 0xFF))


def dequant_nvfp4_bf16(wp: np.ndarray, bs: np.ndarray, g: float) -> np.ndarray:
    """NVFP4 [n][k] -> BF16 bits [n][k]: bf16(fl32((e2m1 * e4m3(bs)) * g))."""
    wp = np.ascontiguousarray(wp, dtype=np.uint8)
    bs = np.ascontiguousarray(bs, dtype=np.uint8)
    n, k = wp.shape[0], wp.shape[1] * 2
    assert bs.shape == (n, k // 16)
    out = np.empty((n, k), dtype=np.uint16)
    lib().orc_dequant_nvfp4_bf16(_ptr(wp, ctypes.c_uint8), _ptr(bs, ctypes.c_uint8), float(g), n, k,
                                 _ptr(out, ctypes.c_uint16))
    return out


def dequant_fp4_e8m0_bf16(packed: np.ndarray, scales: np.ndarray, total: int) -> np.ndarray:
    """Flat E2M1 with E8M0 group scales -> BF16 bits [total]."""
    p = np.ascontiguousarray(packed, dtype=np.uint8).ravel()
    s = np.ascontiguousarray(scales, dtype=np.uint8).ravel()
    assert p.size * 2 == total and total % s.size == 0
    out = np.empty(total, dtype=np.uint16)
    lib().orc_dequant_fp4_e8m0_bf16(_ptr(p, ctypes.c_uint8), _ptr(s, ctypes.c_uint8), total, s.size,
                                    _ptr(out, ctypes.c_uint16))
    return out
