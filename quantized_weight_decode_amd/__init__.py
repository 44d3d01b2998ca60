"""Python binding of libqhead.so: few-row quantized-weight LM-head GEMV on MI355X.

Thin ctypes marshalling over the C ABI declared in ``include/qhead.h``: every
function takes torch tensors that live in device memory, passes their data
pointers and torch's current HIP stream, and raises ``QheadError`` on a
negative status. All arithmetic runs in the HIP kernels of the library; there
is no CPU path. Importing this module fails loudly when the library has not
been built (``python quantized_weight_decode_amd/build.py`` or
``__graft_entry__.build()``).

Tensors: BF16 activations and logits may be ``torch.bfloat16`` or 16-bit
integer tensors holding BF16 bits; E4M3 / packed FP4 / Q6_K / q8_1 bytes are
``torch.uint8``; scales are ``torch.float32``.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqhead.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "qhead.h")

FMT_FP8, FMT_W8A8, FMT_NVFP4, FMT_Q6K = 0, 1, 2, 3
Q8_BLOCK_BYTES = 36
Q6K_BLOCK_BYTES = 210

_STATUS_NAMES = {0: "QHEAD_OK", -1: "QHEAD_ERR_NULL", -2: "QHEAD_ERR_SHAPE",
                 -3: "QHEAD_ERR_ALIGN", -4: "QHEAD_ERR_WORKSPACE", -5: "QHEAD_ERR_ARG",
                 -6: "QHEAD_ERR_DEVICE", -7: "QHEAD_ERR_HIP",
                 -8: "QHEAD_ERR_SCRATCH"}


class QheadError(RuntimeError):
    def __init__(self, status: int, func: str):
        self.status = status
        super().__init__(f"{func}: {_STATUS_NAMES.get(status, status)} ({status_string(status)})")


if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libqhead.so not found at {LIB_PATH}; build it first with "
        "`python quantized_weight_decode_amd/build.py` (hipcc, gfx950)")

_vp, _i32, _sz, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
_SIGS = {
    "qhead_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "qhead_max_rows_per_launch": (ctypes.c_int, [_i32]),
    "qhead_plan_chunks": (ctypes.c_int, [_i32, _i32, ctypes.POINTER(_i32), _i32]),
    "qhead_fp8_rowscale": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp]),
    "qhead_quant_act_e4m3": (ctypes.c_int, [_vp, _i32, _i32, _vp, _vp, _vp]),
    "qhead_w8a8_workspace_bytes": (_sz, [_i32]),
    "qhead_w8a8_gemv": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp]),
    "qhead_w8a8": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _sz, _vp]),
    "qhead_nvfp4": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _vp, _f32, _vp]),
    "qhead_quant_q8_1": (ctypes.c_int, [_vp, _i32, _i32, _vp, _vp]),
    "qhead_q6k_workspace_bytes": (_sz, [_i32]),
    "qhead_q6k_gemv": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _vp, _vp]),
    "qhead_q6k": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _sz, _vp]),
    "qhead_q6k_static_scratch": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp]),
    "qhead_quantize_fp8_rows": (ctypes.c_int, [_vp, _i32, _i32, _vp, _vp, _vp]),
    "qhead_silu_mul_bf16": (ctypes.c_int, [_vp, _vp, ctypes.c_int64, _vp, _vp]),
    "qhead_quant_act_silu_e4m3": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp]),
    "qhead_w8a8_silu": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp,
                                       ctypes.c_size_t, _vp]),
    "qhead_quantize_nvfp4_rows": (ctypes.c_int, [_vp, _i32, _i32, _f32, _vp, _vp, _vp]),
    "qhead_quantize_q6k_rows": (ctypes.c_int, [_vp, _i32, _i32, _vp, _vp]),
    "qhead_dequant_nvfp4_bf16": (ctypes.c_int, [_vp, _vp, _i32, _i32, _f32, _vp, _vp]),
    "qhead_dequant_fp4_e8m0_bf16": (ctypes.c_int, [_vp, _vp, ctypes.c_int64, ctypes.c_int64, _vp,
                                                   _vp]),
    "qhead_stream_read": (ctypes.c_int, [_vp, ctypes.c_int64, _vp, _vp]),
}

_lib = ctypes.CDLL(LIB_PATH)
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


def lib() -> ctypes.CDLL:
    """The loaded C library, with argtypes set (raw pointer calls)."""
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/qhead.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qhead_[a-z0-9_]+)\s*\(", text)))


def status_string(status: int) -> str:
    return _lib.qhead_status_string(int(status)).decode()


def _check(status: int, func: str) -> None:
    if status != 0:
        raise QheadError(status, func)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(t: torch.Tensor, name: str, dtypes) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be in device memory")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return t.data_ptr()


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
# words of qhead_stream_read's output (QHEAD_STREAM_READ_WORDS in qhead.h)
STREAM_READ_WORDS = 4096
_U8 = (torch.uint8,)
_F32 = (torch.float32,)


def max_rows_per_launch(fmt: int) -> int:
    r = _lib.qhead_max_rows_per_launch(fmt)
    _check(min(r, 0), "qhead_max_rows_per_launch")
    return r


def plan_chunks(fmt: int, rows: int) -> list[int]:
    n = _lib.qhead_plan_chunks(fmt, rows, None, 0)
    _check(min(n, 0), "qhead_plan_chunks")
    buf = (_i32 * max(n, 1))()
    n2 = _lib.qhead_plan_chunks(fmt, rows, buf, n)
    _check(min(n2, 0), "qhead_plan_chunks")
    return [buf[i] for i in range(n2)]


def _shape(t, name: str, shape) -> None:
    """ValueError unless `t` is a tensor of exactly `shape` (None: any extent).
    The library reads and writes by the sizes it is given, so a tensor of
    another shape would be read or written out of bounds."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    got = tuple(t.shape)
    if len(got) != len(shape) or any(e is not None and a != e for a, e in zip(got, shape)):
        want = tuple("*" if e is None else e for e in shape)
        raise ValueError(f"{name} has shape {got}, expected {want}")


def _min_numel(t, name: str, n: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.numel() < n:
        raise ValueError(f"{name} has {t.numel()} elements, needs at least {n}")


def _out(out, rows, vocab, device):
    if out is None:
        return torch.empty((rows, vocab), dtype=torch.bfloat16, device=device)
    _shape(out, "out", (rows, vocab))
    return out


def fp8_rowscale(w: torch.Tensor, row_scale: torch.Tensor, x: torch.Tensor, out=None,
                 stream=None) -> torch.Tensor:
    """logits[rows, vocab] (BF16) from FP8 E4M3 weights [vocab, hidden] with F32 row scales."""
    _shape(w, "w", (None, None))
    vocab, hidden = w.shape
    _shape(row_scale, "row_scale", (vocab,))
    _shape(x, "x", (None, hidden))
    rows = x.shape[0]
    out = _out(out, rows, vocab, w.device)
    st = _lib.qhead_fp8_rowscale(_dev(w, "w", _U8), _dev(row_scale, "row_scale", _F32),
                                 _dev(x, "x", _BF16), rows, hidden, vocab,
                                 _dev(out, "out", _BF16), _stream(stream))
    _check(st, "qhead_fp8_rowscale")
    return out


def quant_act_e4m3(x: torch.Tensor, xq=None, xscale=None, stream=None):
    """Per-row E4M3 activations: returns (xq uint8 [rows, hidden], xscale f32 [rows])."""
    _shape(x, "x", (None, None))
    rows, hidden = x.shape
    if xq is None:
        xq = torch.empty((rows, hidden), dtype=torch.uint8, device=x.device)
    if xscale is None:
        xscale = torch.empty((rows,), dtype=torch.float32, device=x.device)
    _shape(xq, "xq", (rows, hidden))
    _shape(xscale, "xscale", (rows,))
    st = _lib.qhead_quant_act_e4m3(_dev(x, "x", _BF16), rows, hidden, _dev(xq, "xq", _U8),
                                   _dev(xscale, "xscale", _F32), _stream(stream))
    _check(st, "qhead_quant_act_e4m3")
    return xq, xscale


def w8a8_workspace_bytes(hidden: int) -> int:
    return int(_lib.qhead_w8a8_workspace_bytes(hidden))


def w8a8_workspace(hidden: int, device) -> torch.Tensor:
    return torch.empty((w8a8_workspace_bytes(hidden),), dtype=torch.uint8, device=device)


def w8a8_gemv(w, row_scale, xq, xscale, out=None, stream=None) -> torch.Tensor:
    _shape(w, "w", (None, None))
    vocab, hidden = w.shape
    _shape(row_scale, "row_scale", (vocab,))
    _shape(xq, "xq", (None, hidden))
    rows = xq.shape[0]
    _shape(xscale, "xscale", (rows,))
    out = _out(out, rows, vocab, w.device)
    st = _lib.qhead_w8a8_gemv(_dev(w, "w", _U8), _dev(row_scale, "row_scale", _F32),
                              _dev(xq, "xq", _U8), _dev(xscale, "xscale", _F32), rows, hidden,
                              vocab, _dev(out, "out", _BF16), _stream(stream))
    _check(st, "qhead_w8a8_gemv")
    return out


def w8a8(w, row_scale, x, out=None, workspace=None, stream=None) -> torch.Tensor:
    """W8A8 logits: per-row E4M3 activations, then FP8 x FP8 over the same weight bytes."""
    _shape(w, "w", (None, None))
    vocab, hidden = w.shape
    _shape(row_scale, "row_scale", (vocab,))
    _shape(x, "x", (None, hidden))
    rows = x.shape[0]
    out = _out(out, rows, vocab, w.device)
    if workspace is None:
        workspace = w8a8_workspace(hidden, w.device)
    _min_numel(workspace, "workspace", w8a8_workspace_bytes(hidden))
    st = _lib.qhead_w8a8(_dev(w, "w", _U8), _dev(row_scale, "row_scale", _F32),
                         _dev(x, "x", _BF16), rows, hidden, vocab, _dev(out, "out", _BF16),
                         _dev(workspace, "workspace", _U8), workspace.numel(), _stream(stream))
    _check(st, "qhead_w8a8")
    return out


def _silu_shapes(gate, up, hidden):
    _shape(gate, "gate", (None, None))
    if gate.shape != up.shape:
        raise ValueError("gate and up must be [rows, ld] tensors of one shape")
    rows, ld = gate.shape
    hidden = ld if hidden is None else int(hidden)
    if hidden > ld:
        raise ValueError(f"hidden {hidden} exceeds the row length {ld} of gate and up")
    return rows, ld, hidden


def silu_mul_bf16(gate, up, out=None, stream=None) -> torch.Tensor:
    """bf16(silu(gate) * up) elementwise (silu and product in binary64)."""
    if gate.shape != up.shape:
        raise ValueError("gate and up must have one shape")
    if out is None:
        out = torch.empty(gate.shape, dtype=torch.bfloat16, device=gate.device)
    _shape(out, "out", tuple(gate.shape))
    st = _lib.qhead_silu_mul_bf16(_dev(gate, "gate", _BF16), _dev(up, "up", _BF16), gate.numel(),
                                  _dev(out, "out", _BF16), _stream(stream))
    _check(st, "qhead_silu_mul_bf16")
    return out


def quant_act_silu_e4m3(gate, up, hidden=None, xq=None, xscale=None, stream=None):
    """Per-row E4M3 quantization of bf16(silu(gate) * up) over the first
    `hidden` columns: (xq uint8 [rows, hidden], xscale f32 [rows])."""
    rows, ld, hidden = _silu_shapes(gate, up, hidden)
    if xq is None:
        xq = torch.empty((rows, hidden), dtype=torch.uint8, device=gate.device)
    if xscale is None:
        xscale = torch.empty((rows,), dtype=torch.float32, device=gate.device)
    _shape(xq, "xq", (rows, hidden))
    _shape(xscale, "xscale", (rows,))
    st = _lib.qhead_quant_act_silu_e4m3(_dev(gate, "gate", _BF16), _dev(up, "up", _BF16), ld,
                                        rows, hidden, _dev(xq, "xq", _U8),
                                        _dev(xscale, "xscale", _F32), _stream(stream))
    _check(st, "qhead_quant_act_silu_e4m3")
    return xq, xscale


def w8a8_silu(w, row_scale, gate, up, out=None, workspace=None, stream=None) -> torch.Tensor:
    """W8A8 down projection of bf16(silu(gate) * up): w [n_out, k] E4M3 with
    per-row scales, gate/up [rows, ld] BF16 (ld >= k); out [rows, n_out]."""
    _shape(w, "w", (None, None))
    vocab, hidden = w.shape
    _shape(row_scale, "row_scale", (vocab,))
    rows, ld, _ = _silu_shapes(gate, up, hidden)
    out = _out(out, rows, vocab, w.device)
    if workspace is None:
        workspace = w8a8_workspace(hidden, w.device)
    _min_numel(workspace, "workspace", w8a8_workspace_bytes(hidden))
    st = _lib.qhead_w8a8_silu(_dev(w, "w", _U8), _dev(row_scale, "row_scale", _F32),
                              _dev(gate, "gate", _BF16), _dev(up, "up", _BF16), ld, rows, hidden,
                              vocab, _dev(out, "out", _BF16), _dev(workspace, "workspace", _U8),
                              workspace.numel(), _stream(stream))
    _check(st, "qhead_w8a8_silu")
    return out


def nvfp4(w_packed, block_scale, x, global_scale: float, out=None, stream=None) -> torch.Tensor:
    """NVFP4 W4A16 logits; w_packed [vocab, hidden/2], block_scale [vocab, hidden/16]."""
    _shape(w_packed, "w_packed", (None, None))
    vocab = w_packed.shape[0]
    hidden = w_packed.shape[1] * 2
    _shape(block_scale, "block_scale", (vocab, hidden // 16))
    _shape(x, "x", (None, hidden))
    rows = x.shape[0]
    out = _out(out, rows, vocab, w_packed.device)
    st = _lib.qhead_nvfp4(_dev(w_packed, "w_packed", _U8), _dev(block_scale, "block_scale", _U8),
                          _dev(x, "x", _BF16), rows, hidden, vocab, _dev(out, "out", _BF16),
                          float(global_scale), _stream(stream))
    _check(st, "qhead_nvfp4")
    return out


def quant_q8_1(x, q8=None, stream=None) -> torch.Tensor:
    """block_q8_1 activations: uint8 [rows, hidden/32*36]."""
    _shape(x, "x", (None, None))
    rows, hidden = x.shape
    if q8 is None:
        q8 = torch.empty((rows, hidden // 32 * Q8_BLOCK_BYTES), dtype=torch.uint8, device=x.device)
    _min_numel(q8, "q8", rows * (hidden // 32) * Q8_BLOCK_BYTES)
    st = _lib.qhead_quant_q8_1(_dev(x, "x", _BF16), rows, hidden, _dev(q8, "q8", _U8),
                               _stream(stream))
    _check(st, "qhead_quant_q8_1")
    return q8


def q6k_workspace_bytes(hidden: int) -> int:
    return int(_lib.qhead_q6k_workspace_bytes(hidden))


def q6k_gemv(blocks, q8, hidden: int, out=None, stream=None) -> torch.Tensor:
    _shape(blocks, "blocks", (None, hidden // 256 * Q6K_BLOCK_BYTES))
    vocab = blocks.shape[0]
    _shape(q8, "q8", (None, hidden // 32 * Q8_BLOCK_BYTES))
    rows = q8.shape[0]
    out = _out(out, rows, vocab, blocks.device)
    st = _lib.qhead_q6k_gemv(_dev(blocks, "blocks", _U8), _dev(q8, "q8", _U8), rows, hidden, vocab,
                             _dev(out, "out", _BF16), _stream(stream))
    _check(st, "qhead_q6k_gemv")
    return out


def q6k(blocks, x, out=None, workspace=None, stream=None) -> torch.Tensor:
    """Q6_K logits: x quantized to q8_1 per <= 8-row chunk, then the Q6_K GEMV."""
    _shape(x, "x", (None, None))
    rows, hidden = x.shape
    _shape(blocks, "blocks", (None, hidden // 256 * Q6K_BLOCK_BYTES))
    vocab = blocks.shape[0]
    out = _out(out, rows, vocab, blocks.device)
    if workspace is None:
        workspace = torch.empty((q6k_workspace_bytes(hidden),), dtype=torch.uint8,
                                device=blocks.device)
    st = _lib.qhead_q6k(_dev(blocks, "blocks", _U8), None, _dev(x, "x", _BF16), rows, hidden,
                        vocab, _dev(out, "out", _BF16), _dev(workspace, "workspace", _U8),
                        workspace.numel(), _stream(stream))
    _check(st, "qhead_q6k")
    return out


# hidden limit of qhead_q6k_static_scratch (QHEAD_Q6K_STATIC_MAX_HIDDEN in qhead.h)
Q6K_STATIC_MAX_HIDDEN = 65536


def q6k_static_scratch(blocks, x, out=None, stream=None) -> torch.Tensor:
    """Q6_K logits as q6k(), with the q8_1 activations in the library's fixed
    per-GPU device array instead of a workspace (nothing is allocated by the
    call except `out` when it is not given). Calls that may overlap on one GPU
    race on that array."""
    _shape(x, "x", (None, None))
    rows, hidden = x.shape
    _shape(blocks, "blocks", (None, hidden // 256 * Q6K_BLOCK_BYTES))
    vocab = blocks.shape[0]
    out = _out(out, rows, vocab, blocks.device)
    st = _lib.qhead_q6k_static_scratch(_dev(blocks, "blocks", _U8), None, _dev(x, "x", _BF16),
                                       rows, hidden, vocab, _dev(out, "out", _BF16),
                                       _stream(stream))
    _check(st, "qhead_q6k_static_scratch")
    return out


def quantize_fp8_rows(w_f32: torch.Tensor, codes=None, scales=None, stream=None):
    """Load-time per-row E4M3 quantization of F32 weights: (codes uint8, row scales f32)."""
    _shape(w_f32, "w_f32", (None, None))
    vocab, hidden = w_f32.shape
    if codes is None:
        codes = torch.empty((vocab, hidden), dtype=torch.uint8, device=w_f32.device)
    if scales is None:
        scales = torch.empty((vocab,), dtype=torch.float32, device=w_f32.device)
    _shape(codes, "codes", (vocab, hidden))
    _shape(scales, "scales", (vocab,))
    st = _lib.qhead_quantize_fp8_rows(_dev(w_f32, "w_f32", _F32), vocab, hidden,
                                      _dev(codes, "codes", _U8), _dev(scales, "scales", _F32),
                                      _stream(stream))
    _check(st, "qhead_quantize_fp8_rows")
    return codes, scales


def quantize_nvfp4_rows(w_f32: torch.Tensor, global_scale: float, w_packed=None,
                        block_scale=None, stream=None):
    """Load-time NVFP4 quantization of F32 weights with global multiplier g:
    (w_packed uint8 [vocab, hidden/2], block_scale uint8 [vocab, hidden/16])."""
    _shape(w_f32, "w_f32", (None, None))
    vocab, hidden = w_f32.shape
    if w_packed is None:
        w_packed = torch.empty((vocab, hidden // 2), dtype=torch.uint8, device=w_f32.device)
    if block_scale is None:
        block_scale = torch.empty((vocab, hidden // 16), dtype=torch.uint8, device=w_f32.device)
    _shape(w_packed, "w_packed", (vocab, hidden // 2))
    _shape(block_scale, "block_scale", (vocab, hidden // 16))
    st = _lib.qhead_quantize_nvfp4_rows(_dev(w_f32, "w_f32", _F32), vocab, hidden,
                                        float(global_scale), _dev(w_packed, "w_packed", _U8),
                                        _dev(block_scale, "block_scale", _U8), _stream(stream))
    _check(st, "qhead_quantize_nvfp4_rows")
    return w_packed, block_scale


def quantize_q6k_rows(w_f32: torch.Tensor, blocks=None, stream=None) -> torch.Tensor:
    """Load-time Q6_K quantization of F32 weights: uint8 [vocab, hidden/256*210]."""
    _shape(w_f32, "w_f32", (None, None))
    vocab, hidden = w_f32.shape
    if blocks is None:
        blocks = torch.empty((vocab, hidden // 256 * Q6K_BLOCK_BYTES), dtype=torch.uint8,
                             device=w_f32.device)
    _shape(blocks, "blocks", (vocab, hidden // 256 * Q6K_BLOCK_BYTES))
    st = _lib.qhead_quantize_q6k_rows(_dev(w_f32, "w_f32", _F32), vocab, hidden,
                                      _dev(blocks, "blocks", _U8), _stream(stream))
    _check(st, "qhead_quantize_q6k_rows")
    return blocks


def dequant_nvfp4_bf16(w_packed, block_scale, global_scale: float, out=None,
                       stream=None) -> torch.Tensor:
    """Load-time NVFP4 -> BF16: bf16 [rows, cols] from w_packed [rows, cols/2]."""
    _shape(w_packed, "w_packed", (None, None))
    rows = w_packed.shape[0]
    cols = w_packed.shape[1] * 2
    _shape(block_scale, "block_scale", (rows, cols // 16))
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.bfloat16, device=w_packed.device)
    _shape(out, "out", (rows, cols))
    st = _lib.qhead_dequant_nvfp4_bf16(_dev(w_packed, "w_packed", _U8),
                                       _dev(block_scale, "block_scale", _U8), rows, cols,
                                       float(global_scale), _dev(out, "out", _BF16),
                                       _stream(stream))
    _check(st, "qhead_dequant_nvfp4_bf16")
    return out


def dequant_fp4_e8m0_bf16(w_packed, scale_e8m0, out=None, stream=None) -> torch.Tensor:
    """Load-time E2M1 + E8M0 group scales -> BF16 over the flat tensor
    (total = 2 * w_packed.numel() values in scale_e8m0.numel() equal groups)."""
    total = w_packed.numel() * 2
    if out is None:
        out = torch.empty((total,), dtype=torch.bfloat16, device=w_packed.device)
    if out.numel() != total:
        raise ValueError(f"out has {out.numel()} elements, expected {total}")
    st = _lib.qhead_dequant_fp4_e8m0_bf16(_dev(w_packed, "w_packed", _U8),
                                          _dev(scale_e8m0, "scale_e8m0", _U8), total,
                                          scale_e8m0.numel(), _dev(out, "out", _BF16),
                                          _stream(stream))
    _check(st, "qhead_dequant_fp4_e8m0_bf16")
    return out


def stream_read(buf: torch.Tensor, xor_out=None, stream=None) -> torch.Tensor:
    """Read the whole of `buf` once (the streaming-read yardstick of the GEMV
    launches). Returns the int32 device tensor of per-workgroup XORs
    (STREAM_READ_WORDS words, cleared here first); the XOR of its words is the
    XOR of all 32-bit words of the buffer."""
    if xor_out is None:
        xor_out = torch.zeros((STREAM_READ_WORDS,), dtype=torch.int32, device=buf.device)
    else:
        if xor_out.numel() < STREAM_READ_WORDS:
            raise ValueError(f"xor_out needs {STREAM_READ_WORDS} words")
        xor_out.zero_()
    nbytes = buf.numel() * buf.element_size()
    st = _lib.qhead_stream_read(_dev(buf, "buf", (buf.dtype,)), nbytes,
                                _dev(xor_out, "xor_out", (torch.int32,)), _stream(stream))
    _check(st, "qhead_stream_read")
    return xor_out
