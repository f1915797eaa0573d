"""The CPU oracle over many threads (test infrastructure, not a test module).

Blocks are independent, so a tensor's lines are split into contiguous ranges
and each range goes through the oracle's own line-range call, which keeps the
whole tensor's block numbering (the stochastic-rounding stream is keyed by it).
The oracle's C calls release the GIL, so Python threads run them in parallel.
The results are the single-call results byte for byte.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np


def threads() -> int:
    """Host threads for the oracle: at most 16 (one GPU's share of a host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def split(n: int, parts: int) -> list[tuple[int, int]]:
    parts = max(1, min(parts, n))
    step = (n + parts - 1) // parts
    return [(s, min(step, n - s)) for s in range(0, n, step)] if n else []


def quantize(orc, x, axis: int, p, fmt: int):
    """orc.quantize(x, axis, p, fmt) computed over line ranges in parallel."""
    rows, cols = x.shape
    lines = rows if axis == orc.AXIS_ROW else cols
    ranges = split(lines, threads() * 2)
    if len(ranges) <= 1:
        return orc.quantize(x, axis, p, fmt)
    with ThreadPoolExecutor(threads()) as ex:
        parts = list(ex.map(lambda r: orc.quantize_lines(x, axis, p, r[0], r[1], fmt), ranges))
    return (np.concatenate([c for c, _ in parts]), np.concatenate([s for _, s in parts]))


def dequantize(orc, codes, scales, grid: int, fmt: int) -> np.ndarray:
    ranges = split(scales.shape[0], threads() * 2)
    if len(ranges) <= 1:
        return orc.dequantize(codes, scales, grid, fmt)
    with ThreadPoolExecutor(threads()) as ex:
        parts = list(ex.map(lambda r: orc.dequantize(codes[r[0]:r[0] + r[1]],
                                                     scales[r[0]:r[0] + r[1]], grid, fmt), ranges))
    return np.concatenate(parts)


def gemm_abt_f64(orc, a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """C = A B^T in fp64 by the oracle, row bands of A in parallel."""
    ranges = split(a.shape[0], threads() * 2)
    if len(ranges) <= 1:
        return orc.gemm_abt_f64(a, b)
    b = np.ascontiguousarray(b, dtype=np.float64)
    with ThreadPoolExecutor(threads()) as ex:
        parts = list(ex.map(lambda r: orc.gemm_abt_f64(a[r[0]:r[0] + r[1]], b), ranges))
    return np.concatenate(parts)
