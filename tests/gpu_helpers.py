"""Shared helpers for the GPU parity tests: device transfer, the acceptance
bound, sampled vocab indices and cached full-size heads (quantized on the
host by the oracle's data-preparation quantizers, then uploaded)."""

from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import oracle
import synth

DEV = torch.device("cuda:0")


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def dev_f32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).to(DEV).view(torch.bfloat16)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


# Half the spacing of BF16's subnormals (2^-133): no BF16 value lies closer
# than this to every real number in BF16's subnormal range, where 2^-7 |ref|
# is smaller than the output format can resolve.
BF16_SUBNORMAL_HALF_SPACING = 2.0 ** -134


def assert_within_bound(got_bits: np.ndarray, ref: np.ndarray, absdot: np.ndarray, what: str):
    """|gpu - ref| <= 2^-7 |ref| + 1e-4 sum|x w| for every logit, read with a
    floor of 2^-134 for logits in BF16's subnormal range."""
    got = bf16_bits_to_f64(got_bits)
    err = np.abs(got - ref)
    bound = 2.0 ** -7 * np.abs(ref) + 1e-4 * absdot + BF16_SUBNORMAL_HALF_SPACING
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = [(tuple(int(v) for v in i), float(got[tuple(i)]), float(ref[tuple(i)]),
                   float(bound[tuple(i)])) for i in idx]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} logits outside the bound; "
                             f"first (index, gpu, ref, bound): {detail}")
    return float(np.max(err / np.maximum(bound, 1e-300)))


def sample_vidx(vocab: int, n: int, seed: int = 0) -> np.ndarray:
    """Sorted sample of vocab rows: the first and last rows plus random ones."""
    if n >= vocab:
        return np.arange(vocab, dtype=np.int64)
    g = np.random.Generator(np.random.PCG64(1000 + seed))
    pick = g.choice(vocab, size=n, replace=False)
    pick[:4] = [0, 1, vocab - 2, vocab - 1]
    return np.unique(pick).astype(np.int64)


@functools.lru_cache(maxsize=2)
def fp8_head(cfg_index: int):
    """Host (codes, scales) and device copies of a config's full FP8 head."""
    log(f"[prep] fp8 head cfg{cfg_index}")
    codes, scales = oracle.prep_config_weights(cfg_index, "fp8")
    return codes, scales, dev_u8(codes), dev_f32(scales)


@functools.lru_cache(maxsize=1)
def nvfp4_head():
    """Host (packed, block scales, g) and device copies of the full NVFP4 head
    of the 129280 x 7168 config."""
    log("[prep] nvfp4 head 129280x7168")
    wp, bs, g = oracle.prep_config_weights(synth.NVFP4_Q6K_129280X7168, "nvfp4")
    return wp, bs, g, dev_u8(wp), dev_u8(bs)


@functools.lru_cache(maxsize=1)
def q6k_head():
    """Host and device copies of the full Q6_K head of the 129280 x 7168 config."""
    log("[prep] q6k head 129280x7168")
    blocks = oracle.prep_config_weights(synth.NVFP4_Q6K_129280X7168, "q6k")
    return blocks, dev_u8(blocks)


def x_rows(cfg_index: int, rows: int, **kw) -> np.ndarray:
    return synth.activations_bf16(cfg_index, rows, **kw)
