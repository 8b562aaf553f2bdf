"""Seeded synthetic inputs, shared by the tests and the benchmark.

This module holds none of the reduction's arithmetic: it only draws random
binary32 values with numpy and keeps their upper 16 bits (truncation toward
zero), which turns a binary32 value into a bf16 bit pattern without any
rounding step.  The result is returned as numpy ``uint16`` bf16 bit patterns.

Rank r of seed s draws from ``numpy.random.default_rng(s * 1000 + r)``.
"""
from __future__ import annotations

import numpy as np


def rank_seed(seed: int, rank: int) -> int:
    return seed * 1000 + rank


def _upper_half(f32: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def uniform_bf16(n: int, seed: int, rank: int) -> np.ndarray:
    """bf16 values uniform in [-1, 1).

    numpy draws binary32 values k * 2**-24 in [0, 1); 2v - 1 is then exact on
    the 2**-23 grid in [-1, 1), and its upper half is a bf16 in [-1, 1) (the
    largest is 0x3F7F, 1 - 2**-8).
    """
    rng = np.random.default_rng(rank_seed(seed, rank))
    v = rng.random(n, dtype=np.float32) * np.float32(2) - np.float32(1)
    return _upper_half(v)


def normal_clipped_bf16(n: int, seed: int, rank: int, limit: float = 4.0) -> np.ndarray:
    """bf16 values from N(0, 1) clipped to [-limit, limit]."""
    rng = np.random.default_rng(rank_seed(seed, rank))
    v = rng.standard_normal(n, dtype=np.float32)
    np.clip(v, np.float32(-limit), np.float32(limit), out=v)
    return _upper_half(v)


def position_fill_bf16(n: int, rank: int) -> np.ndarray:
    """x_r[i] = ((131 i + 17 r) mod 251 - 125) / 128.

    Every value is k/128 with |k| <= 125, exact in bf16, and any sum of up to
    eight of them is exact in binary32; a swapped index, rank or block offset
    changes the values, so a permutation cannot pass a comparison.
    """
    i = np.arange(n, dtype=np.int64)
    k = (i * 131 + rank * 17) % 251 - 125
    return _upper_half(k.astype(np.float32) / np.float32(128))


def make_inputs(kind: str, P: int, n: int, seed: int = 0) -> list:
    if kind == "uniform":
        return [uniform_bf16(n, seed, r) for r in range(P)]
    if kind == "normal":
        return [normal_clipped_bf16(n, seed, r) for r in range(P)]
    if kind == "position":
        return [position_fill_bf16(n, r) for r in range(P)]
    raise ValueError(f"unknown input kind {kind!r}")
