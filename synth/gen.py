"""Seeded synthetic inputs for the Ulysses attention share.

This module only draws random numbers and lays them out; it contains none of
the arithmetic of the method (no relayout, no attention, no loss).  Both the
CPU oracle tests and the GPU path's tests/benchmark take their inputs from
here, so the two sides see the same bit patterns.

Random streams
--------------
Every tensor is identified by a key tuple, e.g. ``(cfg, stream)``.  A tensor
of ``n`` elements is drawn in chunks of ``CHUNK`` elements; chunk ``c`` comes
from ``numpy.random.default_rng([*key, c])`` (PCG64 seeded through
SeedSequence).  Chunking makes the large workloads cheap to draw in parallel
and lets a test regenerate only the rows it samples.

bf16 values are float32 standard normals rounded to the nearest bf16 with
ties to even (an integer bit trick on the float32 pattern); normals are finite,
so no NaN/Inf pattern can appear.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22


def _threads() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


def _chunked(key, n, fill, out):
    """Run ``fill(rng, lo, hi)`` for every chunk of ``[0, n)`` on a thread pool."""
    nchunks = (n + CHUNK - 1) // CHUNK

    def one(c):
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        fill(np.random.default_rng([*key, c]), lo, hi)

    if nchunks <= 1:
        for c in range(nchunks):
            one(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(nchunks)))
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def normal_bf16(key, shape) -> np.ndarray:
    """bf16 ~ N(0,1) bit patterns (uint16) of the given shape."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.uint16)

    def fill(rng, lo, hi):
        out[lo:hi] = f32_to_bf16_bits(rng.standard_normal(hi - lo, dtype=np.float32))

    return _chunked(tuple(key), n, fill, out).reshape(shape)


def normal_bf16_scaled(key, shape, scale: float) -> np.ndarray:
    """bf16 ~ N(0, scale^2) bit patterns: float32 standard normal times scale,
    rounded to nearest-even bf16."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.uint16)
    sc = np.float32(scale)

    def fill(rng, lo, hi):
        out[lo:hi] = f32_to_bf16_bits(rng.standard_normal(hi - lo, dtype=np.float32) * sc)

    return _chunked(tuple(key), n, fill, out).reshape(shape)


def raw_bits_u16(key, shape) -> np.ndarray:
    """Uniformly random 16-bit patterns: every bf16 class appears (NaN payloads, +-0, subnormals, +-Inf)."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.uint16)

    def fill(rng, lo, hi):
        out[lo:hi] = rng.integers(0, 1 << 16, hi - lo, dtype=np.uint16)

    return _chunked(tuple(key), n, fill, out).reshape(shape)


def uniform_f32(key, shape, lo: float, hi: float) -> np.ndarray:
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.float32)

    def fill(rng, a, b):
        out[a:b] = rng.uniform(lo, hi, b - a).astype(np.float32)

    return _chunked(tuple(key), n, fill, out).reshape(shape)


def integers_i64(key, shape, lo: int, hi: int) -> np.ndarray:
    """Integers uniform in [lo, hi)."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.int64)

    def fill(rng, a, b):
        out[a:b] = rng.integers(lo, hi, b - a, dtype=np.int64)

    return _chunked(tuple(key), n, fill, out).reshape(shape)


def sample_lengths(key, n_tokens: int, lo: int, hi: int) -> list[int]:
    """Packed-sample lengths: integers uniform in [lo, hi] (inclusive), drawn from
    ``default_rng(key)`` until they cover ``n_tokens``; the last one is cut to fit."""
    rng = np.random.default_rng(list(key))
    out: list[int] = []
    total = 0
    while total < n_tokens:
        L = int(rng.integers(lo, hi, endpoint=True))
        L = min(L, n_tokens - total)
        out.append(L)
        total += L
    return out


def position_ids_from_lengths(lengths) -> np.ndarray:
    """position_ids of packed samples: 0..L-1 for each sample, concatenated (int64)."""
    parts = [np.arange(int(L), dtype=np.int64) for L in lengths]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)
