"""Seeded synthetic inputs shaped like the Llama-3.1-8B linear-layer operands.

The pages train Llama-3.1-8B on C4 (gist.science summary "Pre-treinamento de
Modelos de Linguagem Grandes com MXFP4", section "Metodologia"); neither the
data nor the weights are available, so only their shapes are used and the
values are drawn from numpy's PCG64 with fixed seeds.  This module holds no
quantization arithmetic: it makes bf16 bit patterns (uint16 arrays) and the
random +-1 sign masks of the randomized Hadamard transform, which both the
GPU library and the CPU oracle take as inputs.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

GRID_E2M1, GRID_E1M2, GRID_E2M1_MAX4, GRID_E2M1_MAX3 = 0, 1, 2, 3
RTNE, SR = 0, 1
FMT_FP4, FMT_E2M3 = 0, 1
LAYOUT_ROWS, LAYOUT_MFMA = 0, 1


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("synthetic inputs must be finite")
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def sign_mask(seed: int, n: int) -> int:
    """n random sign bits (bit i set: negate block position i) for the RHT."""
    if n == 0:
        return 0
    return int(rng(seed).integers(0, 1 << n, dtype=np.uint64))


def normal(rows: int, cols: int, seed: int, std: float = 1.0) -> np.ndarray:
    g = rng(seed)
    x = g.standard_normal((rows, cols), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


def normal_outlier_channels(rows: int, cols: int, seed: int, ch_seed: int,
                            frac: float = 0.005, factor: float = 50.0) -> np.ndarray:
    """N(0,1) activations with floor(frac*cols) whole channels (columns) scaled."""
    g = rng(seed)
    x = g.standard_normal((rows, cols), dtype=np.float32)
    nch = int(np.floor(frac * cols))
    ch = rng(ch_seed).permutation(cols)[:nch]
    x[:, ch] *= np.float32(factor)
    return f32_to_bf16_bits(x)


def laplace_outlier_entries(rows: int, cols: int, seed: int, out_seed: int,
                            scale: float = 1e-3, frac: float = 0.001,
                            factor: float = 100.0) -> np.ndarray:
    """Laplace(0, scale) gradients with round(frac*numel) random entries scaled."""
    g = rng(seed)
    x = g.laplace(0.0, scale, size=(rows, cols)).astype(np.float32)
    n = rows * cols
    k = int(round(frac * n))
    idx = rng(out_seed).choice(n, size=k, replace=False)
    x.reshape(-1)[idx] *= np.float32(factor)
    return f32_to_bf16_bits(x)


@dataclass
class QuantCase:
    """One quantize call: a tensor recipe plus the knobs."""
    name: str
    rows: int
    cols: int
    make: object                      # () -> uint16 [rows, cols]
    grid: int = GRID_E2M1
    round: int = RTNE
    hadamard_n: int = 0
    sign_mask: int = 0
    row_out: bool = True
    col_out: bool = False
    fmt: int = FMT_FP4
    sr_seed: int = 0
    sr_stream: int = 0
    sr_bits: int = 16
    sign_mode: int = 0                # 0: one mask for every block; 1: drawn per block
    sign_seed: int = 0
    layout: int = LAYOUT_ROWS         # of every output: row layout or the matrix-core layout
    extra: dict = field(default_factory=dict)

    def knobs(self) -> dict:
        return dict(grid=self.grid, round=self.round, hadamard_n=self.hadamard_n,
                    sign_mask=self.sign_mask, sr_seed=self.sr_seed, sr_stream=self.sr_stream,
                    sr_bits=self.sr_bits, sign_mode=self.sign_mode, sign_seed=self.sign_seed)


# --- the five workloads ------------------------------------------------------

def x_1024() -> np.ndarray:
    """1024 x 1024 activation, N(0,1), seed 0."""
    return normal(1024, 1024, seed=0)


def x_8192x4096(seed: int = 1, ch_seed: int = 11) -> np.ndarray:
    """8192 tokens x 4096 hidden, N(0,1) with 20 outlier channels x50."""
    return normal_outlier_channels(8192, 4096, seed, ch_seed)


def w_14336x4096() -> np.ndarray:
    """MLP up-projection weight 14336 x 4096, N(0, 0.02), seed 2."""
    return normal(14336, 4096, seed=2, std=0.02)


def dy_16384x4096() -> np.ndarray:
    """Upstream gradient 16384 tokens x 4096, Laplace(0,1e-3), 0.1% entries x100."""
    return laplace_outlier_entries(16384, 4096, seed=3, out_seed=13)


def dy_8192x4096() -> np.ndarray:
    """Weight-gradient step upstream gradient (same recipe as the 16384-token one)."""
    return laplace_outlier_entries(8192, 4096, seed=5, out_seed=15)


def x_wgrad_8192x4096() -> np.ndarray:
    """Weight-gradient step activation (same recipe as the 8192 x 4096 activation)."""
    return x_8192x4096(seed=6, ch_seed=16)


def dy_8192x14336() -> np.ndarray:
    """Upstream gradient of the 14336-wide up-projection output for 8192 tokens
    (the gradient recipe: Laplace(0,1e-3), 0.1% of entries x100), seeds 8 / 18."""
    return laplace_outlier_entries(8192, 14336, seed=8, out_seed=18)


SIGNS_W = 1002      # 32-bit mask for the weight's H32 RHT
SIGNS_DY = 1004     # 16-bit mask for the gradient's H16 RHT
SIGNS_WGRAD = 1005  # 16-bit mask shared by dY and X of the weight-gradient step
SR_SEED_WGRAD = 7


def workload_cases() -> list[QuantCase]:
    """The quantize calls of the five workloads at full size, plus the
    range-restricted E2M1 grid and per-block signs on the same tensors, and
    the layer's Fprop / Dgrad operands in the matrix-core layout."""
    return [
        QuantCase("x1024_e2m1_rtne", 1024, 1024, x_1024),
        QuantCase("x8192_h16_e2m1", 8192, 4096, x_8192x4096, hadamard_n=16),
        QuantCase("x8192_h16_e1m2", 8192, 4096, x_8192x4096, grid=GRID_E1M2, hadamard_n=16),
        QuantCase("w14336_rht32_e2m1_dual", 14336, 4096, w_14336x4096, hadamard_n=32,
                  sign_mask=sign_mask(SIGNS_W, 32), col_out=True),
        QuantCase("w14336_rht32_e1m2_dual", 14336, 4096, w_14336x4096, grid=GRID_E1M2,
                  hadamard_n=32, sign_mask=sign_mask(SIGNS_W, 32), col_out=True),
        # the range-restricted E2M1 grid and per-block random signs on the same tensors
        QuantCase("x8192_h16_e2m1max4", 8192, 4096, x_8192x4096, grid=GRID_E2M1_MAX4,
                  hadamard_n=16),
        QuantCase("w14336_rht32_e2m1_dual_signs_per_block", 14336, 4096, w_14336x4096,
                  hadamard_n=32, col_out=True, sign_mode=1, sign_seed=SIGNS_W),
        QuantCase("dy16384_rht16_e1m2_sr_col", 16384, 4096, dy_16384x4096, grid=GRID_E1M2,
                  round=SR, hadamard_n=16, sign_mask=sign_mask(SIGNS_DY, 16), row_out=False,
                  col_out=True, sr_seed=0),
        QuantCase("wgrad_dy_rht16_e1m2_sr_col_e2m3", 8192, 4096, dy_8192x4096, grid=GRID_E1M2,
                  round=SR, hadamard_n=16, sign_mask=sign_mask(SIGNS_WGRAD, 16), row_out=False,
                  col_out=True, fmt=FMT_E2M3, sr_seed=SR_SEED_WGRAD),
        QuantCase("wgrad_x_rht16_e1m2_col_e2m3", 8192, 4096, x_wgrad_8192x4096, grid=GRID_E1M2,
                  hadamard_n=16, sign_mask=sign_mask(SIGNS_WGRAD, 16), row_out=False,
                  col_out=True, fmt=FMT_E2M3),
        # stochastic rounding with 8-bit draws (half the Philox work per element)
        QuantCase("dy16384_rht16_e1m2_sr8_col", 16384, 4096, dy_16384x4096, grid=GRID_E1M2,
                  round=SR, hadamard_n=16, sign_mask=sign_mask(SIGNS_DY, 16), row_out=False,
                  col_out=True, sr_seed=0, sr_bits=8),
        QuantCase("wgrad_dy_rht16_e1m2_sr8_col_e2m3", 8192, 4096, dy_8192x4096, grid=GRID_E1M2,
                  round=SR, hadamard_n=16, sign_mask=sign_mask(SIGNS_WGRAD, 16), row_out=False,
                  col_out=True, fmt=FMT_E2M3, sr_seed=SR_SEED_WGRAD, sr_bits=8),
        # the operands of the layer's other two products, written straight into
        # the matrix-core layout: Fprop takes X and W row-wise, Dgrad dY row-wise
        # and W column-wise
        QuantCase("fprop_x8192_rht32_e2m1_row_mfma", 8192, 4096, x_8192x4096, hadamard_n=32,
                  sign_mask=sign_mask(SIGNS_W, 32), layout=LAYOUT_MFMA),
        QuantCase("w14336_rht32_e2m1_dual_mfma", 14336, 4096, w_14336x4096, hadamard_n=32,
                  sign_mask=sign_mask(SIGNS_W, 32), col_out=True, layout=LAYOUT_MFMA),
        QuantCase("dgrad_dy8192x14336_rht32_e2m1_sr_row_mfma", 8192, 14336, dy_8192x14336,
                  round=SR, hadamard_n=32, sign_mask=sign_mask(SIGNS_W, 32), sr_seed=11,
                  layout=LAYOUT_MFMA),
    ]
