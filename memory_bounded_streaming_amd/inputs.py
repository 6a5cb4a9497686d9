"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds no attention arithmetic: it only draws numbers and stores
them.  Q, K and V are i.i.d. standard normal, token-major [N, H, d], batch 1,
matching the Gaussian long-context workloads the method is measured on.

Stream definition (fixed, independent of thread count):
    tensor i in {0: Q, 1: K, 2: V}, block b of BLOCK_TOKENS tokens:
        numpy Generator(PCG64(SeedSequence(seed, spawn_key=(i, b))))
        .standard_normal(rows_in_block * H * d, dtype=float32)
bfloat16 inputs are those float32 draws rounded to nearest-even, stored as the
uint16 bit patterns.

Sampled query rows for large-N checks:
    Generator(PCG64(seed + 1000)).choice(N, R, replace=False), plus the first
    and last token of every unit, sorted and unique.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = ["BLOCK_TOKENS", "gen_tensor", "gen_qkv", "round_to_bf16_bits",
           "bf16_bits_to_f32", "sample_rows", "worker_count"]

BLOCK_TOKENS = 65536


def worker_count() -> int:
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return max(1, min(16, cores))


def round_to_bf16_bits(x: np.ndarray, out: np.ndarray | None = None) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    if out is None:
        return rounded.astype(np.uint16)
    out[...] = rounded.reshape(out.shape)
    return out


def bf16_bits_to_f32(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32, exact."""
    return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _fill_block(seed, tensor_index, block, n, h, d, dtype, out):
    t0 = block * BLOCK_TOKENS
    t1 = min(n, t0 + BLOCK_TOKENS)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tensor_index, block))))
    draws = rng.standard_normal((t1 - t0) * h * d, dtype=np.float32).reshape(t1 - t0, h, d)
    if dtype == "bf16":
        round_to_bf16_bits(draws, out=out[t0:t1])
    else:
        out[t0:t1] = draws


def gen_tensor(seed: int, tensor_index: int, n: int, h: int, d: int, dtype: str = "bf16",
               out: np.ndarray | None = None) -> np.ndarray:
    """One of Q (0), K (1), V (2) or an upstream gradient dO (3) as [n, h, d]; float32,
    or uint16 bf16 bits.

    ``out`` may be a preallocated array (e.g. a view of pinned host memory).
    """
    np_dtype = np.uint16 if dtype == "bf16" else np.float32
    if dtype not in ("bf16", "f32"):
        raise ValueError(dtype)
    if out is None:
        out = np.empty((n, h, d), dtype=np_dtype)
    if out.shape != (n, h, d) or out.dtype != np_dtype:
        raise ValueError("out has the wrong shape or dtype")
    blocks = (n + BLOCK_TOKENS - 1) // BLOCK_TOKENS
    if blocks <= 1:
        for b in range(blocks):
            _fill_block(seed, tensor_index, b, n, h, d, dtype, out)
        return out
    with ThreadPoolExecutor(max_workers=worker_count()) as pool:
        list(pool.map(lambda b: _fill_block(seed, tensor_index, b, n, h, d, dtype, out), range(blocks)))
    return out


def gen_qkv(seed: int, n: int, h: int, d: int, dtype: str = "bf16", outs=None):
    """(Q, K, V) for one seed; see the module docstring for the stream definition."""
    if outs is None:
        outs = (None, None, None)
    return tuple(gen_tensor(seed, i, n, h, d, dtype, out=outs[i]) for i in range(3))


def sample_rows(n: int, count: int, seed: int, unit_tokens: int | None = None) -> np.ndarray:
    """Seeded sample of query rows (sorted, unique), plus every unit's first and last token."""
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    rows = rng.choice(n, size=min(count, n), replace=False).astype(np.int64)
    extra = []
    if unit_tokens:
        starts = np.arange(0, n, unit_tokens, dtype=np.int64)
        extra = [starts, np.minimum(starts + unit_tokens - 1, n - 1)]
    return np.unique(np.concatenate([rows] + extra))
