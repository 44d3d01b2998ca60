"""Seeded synthetic inputs for the quantized LM-head GEMV.

This module is shared by the oracle, the tests and the benchmark, so it holds
no arithmetic of the method: it only draws float32 numbers from numpy's PCG64
generator and rounds the activations to BF16 through torch's CPU cast.
Quantizing the drawn weights (to E4M3 rows, NVFP4 blocks or Q6_K super-blocks)
is the job of whoever consumes them.

Workload shapes follow the head configurations this library is measured on
(the FP8 head of "lm_head_fp8_rows.rs", the W8A8 head of "w8a8_layer.rs",
the NVFP4 head of "w4a16_gemv_tiers.rs" and the Q6_K head of "lm_head_q6k.rs",
and the SiLU FFN down projection of "w8a8_layer.rs"); each has a seed id:

  FP8_8192X1024          id 0  FP8 W8A16, vocab 8192 x hidden 1024,
                               W ~ N(0, 0.02)
  FP8_32000X4096         id 1  FP8 W8A16, vocab 32000 x hidden 4096,
                               W ~ N(0, 0.02), x with 41 outlier channels
                               scaled x20
  FP8_155136X8192        id 2  FP8 W8A16, vocab 155136 x hidden 8192,
                               W ~ N(0, 0.015) (the 1.27 GB head)
  W8A8_129280X7168       id 3  W8A8, vocab 129280 x hidden 7168, W ~ N(0, 0.02)
  NVFP4_Q6K_129280X7168  id 4  NVFP4 / Q6_K, vocab 129280 x hidden 7168,
                               W ~ N(0, 0.02)
  SILU_DOWN_7168X18432   id 5  W8A8 SiLU down projection: output 7168 x FFN
                               width 18432, W ~ N(0, 0.02); gate
                               ~ N(0, 1.5^2), up ~ N(0, 1) (the FFN's
                               activation is bf16(silu(gate) * up))

Weights are drawn in independent 1024-row chunks, chunk c of the
configuration with id i seeded with SeedSequence([100 + i, c]), so any vocab
row range can be regenerated on its own. Activations for id i use seed
200 + i and are drawn once for the configuration's largest row count; a
smaller row count takes the leading rows. The outlier channels use seed
300 + i; the SiLU gate and up rows seeds 400 + i and 500 + i.
"""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import os

import numpy as np

CHUNK_ROWS = 1024


@dataclass(frozen=True)
class HeadConfig:
    index: int
    fmt: str  # "fp8", "w8a8", "nvfp4q6k"
    vocab: int
    hidden: int
    w_std: float
    rows: tuple
    outlier_channels: int = 0
    label: str = field(default="")


FP8_8192X1024 = 0
FP8_32000X4096 = 1
FP8_155136X8192 = 2
W8A8_129280X7168 = 3
NVFP4_Q6K_129280X7168 = 4
SILU_DOWN_7168X18432 = 5

CONFIGS = {
    FP8_8192X1024: HeadConfig(FP8_8192X1024, "fp8", 8192, 1024, 0.02, (1,), 0,
                              "fp8 head 8192x1024"),
    FP8_32000X4096: HeadConfig(FP8_32000X4096, "fp8", 32000, 4096, 0.02,
                               (1, 2, 3, 4, 8, 16, 40), 41,
                               "fp8 head 32000x4096, outlier channels"),
    FP8_155136X8192: HeadConfig(FP8_155136X8192, "fp8", 155136, 8192, 0.015,
                                (1, 2, 4, 8, 16, 64), 0, "fp8 head 155136x8192 (1.27 GB)"),
    W8A8_129280X7168: HeadConfig(W8A8_129280X7168, "w8a8", 129280, 7168, 0.02,
                                 (1, 16, 128, 300), 0, "w8a8 head 129280x7168"),
    NVFP4_Q6K_129280X7168: HeadConfig(NVFP4_Q6K_129280X7168, "nvfp4q6k", 129280, 7168, 0.02,
                                      (1, 2, 3, 4, 5, 6, 7, 8), 0,
                                      "nvfp4 / q6_k head 129280x7168"),
    SILU_DOWN_7168X18432: HeadConfig(SILU_DOWN_7168X18432, "w8a8silu", 7168, 18432, 0.02,
                                     (1, 16, 128, 130), 0,
                                     "w8a8 silu down projection 7168x18432"),
}


def _chunk_generator(seed_base: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed_base, chunk])))


def weight_rows_f32(cfg_index: int, start: int, stop: int, *, vocab: int | None = None,
                    hidden: int | None = None, std: float | None = None,
                    threads: int | None = None) -> np.ndarray:
    """Float32 weights for vocab rows [start, stop) of a config, shape [stop-start, hidden].

    Row v always gets the same values, whatever range it is drawn in. `vocab`,
    `hidden` and `std` override the config's (for small test shapes drawn with
    the same seeding scheme).
    """
    cfg = CONFIGS.get(cfg_index)
    vocab = vocab if vocab is not None else cfg.vocab
    hidden = hidden if hidden is not None else cfg.hidden
    std = std if std is not None else cfg.w_std
    if not (0 <= start <= stop <= vocab):
        raise ValueError(f"row range [{start}, {stop}) outside vocab {vocab}")
    out = np.empty((stop - start, hidden), dtype=np.float32)
    first, last = start // CHUNK_ROWS, (stop - 1) // CHUNK_ROWS if stop > start else -1

    def fill(c: int) -> None:
        lo = c * CHUNK_ROWS
        n = min(CHUNK_ROWS, vocab - lo)
        block = _chunk_generator(100 + cfg_index, c).standard_normal((n, hidden), dtype=np.float32)
        block *= np.float32(std)
        a, b = max(start, lo), min(stop, lo + n)
        out[a - start:b - start] = block[a - lo:b - lo]

    chunks = range(first, last + 1)
    nthreads = threads or min(16, os.cpu_count() or 1)
    if nthreads > 1 and len(chunks) > 1:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(fill, chunks))
    else:
        for c in chunks:
            fill(c)
    return out


def iter_weight_chunks(cfg_index: int, *, vocab: int | None = None, hidden: int | None = None,
                       std: float | None = None, rows_per_chunk: int = 16 * CHUNK_ROWS):
    """Yield (start, stop, f32 rows) over the whole vocab in large row blocks."""
    cfg = CONFIGS.get(cfg_index)
    vocab = vocab if vocab is not None else cfg.vocab
    for lo in range(0, vocab, rows_per_chunk):
        hi = min(vocab, lo + rows_per_chunk)
        yield lo, hi, weight_rows_f32(cfg_index, lo, hi, vocab=vocab, hidden=hidden, std=std)


def activations_f32(cfg_index: int, rows: int, *, hidden: int | None = None,
                    max_rows: int | None = None, outlier_channels: int | None = None) -> np.ndarray:
    """Float32 activations [rows, hidden]: the leading rows of one seeded draw."""
    cfg = CONFIGS.get(cfg_index)
    hidden = hidden if hidden is not None else cfg.hidden
    max_rows = max(max_rows if max_rows is not None else max(cfg.rows), rows)
    outliers = outlier_channels if outlier_channels is not None else cfg.outlier_channels
    g = np.random.Generator(np.random.PCG64(200 + cfg_index))
    x = g.standard_normal((max_rows, hidden), dtype=np.float32)
    if outliers:
        go = np.random.Generator(np.random.PCG64(300 + cfg_index))
        cols = go.choice(hidden, size=outliers, replace=False)
        x[:, cols] *= np.float32(20.0)
    return np.ascontiguousarray(x[:rows])


def outlier_columns(cfg_index: int, hidden: int, count: int) -> np.ndarray:
    """The channel indices activations_f32 scales for a config (for reporting)."""
    go = np.random.Generator(np.random.PCG64(300 + cfg_index))
    return np.sort(go.choice(hidden, size=count, replace=False))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to BF16 (torch's CPU cast, round to nearest even); uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def activations_bf16(cfg_index: int, rows: int, **kw) -> np.ndarray:
    return to_bf16_bits(activations_f32(cfg_index, rows, **kw))


def gate_up_bf16(cfg_index: int, rows: int, *, hidden: int | None = None,
                 max_rows: int | None = None):
    """BF16 bits of the SiLU FFN's gate [rows, hidden] ~ N(0, 1.5^2) and up
    [rows, hidden] ~ N(0, 1): the leading rows of one seeded draw each."""
    cfg = CONFIGS.get(cfg_index)
    hidden = hidden if hidden is not None else cfg.hidden
    max_rows = max(max_rows if max_rows is not None else max(cfg.rows), rows)
    gg = np.random.Generator(np.random.PCG64(400 + cfg_index))
    gu = np.random.Generator(np.random.PCG64(500 + cfg_index))
    gate = gg.standard_normal((max_rows, hidden), dtype=np.float32) * np.float32(1.5)
    up = gu.standard_normal((max_rows, hidden), dtype=np.float32)
    return to_bf16_bits(gate[:rows]), to_bf16_bits(up[:rows])


def random_bytes(seed: int, n: int) -> np.ndarray:
    """Uniform random bytes (for format-agnostic edge-case inputs)."""
    g = np.random.Generator(np.random.PCG64(seed))
    return g.integers(0, 256, size=n, dtype=np.uint8)
