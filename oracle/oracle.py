"""TEST INFRASTRUCTURE ONLY: numpy/ctypes front end of the CPU oracle.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  It loads oracle/libmxq_oracle.so (built by oracle/build.py) and
shares nothing with the GPU library.  Each function names the step of the
method it defines; the arithmetic itself lives in mxq_oracle.c.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "libmxq_oracle.so")

GRID_E2M1, GRID_E1M2, GRID_E2M1_MAX4, GRID_E2M1_MAX3 = 0, 1, 2, 3
RTNE, SR = 0, 1
FMT_FP4, FMT_E2M3 = 0, 1
AXIS_ROW, AXIS_COL = 0, 1
SIGNS_MASK, SIGNS_PER_BLOCK = 0, 1


class QParams(C.Structure):
    _fields_ = [
        ("grid", C.c_int32),
        ("round", C.c_int32),
        ("hadamard_n", C.c_int32),
        ("sign_mask", C.c_uint32),
        ("sr_seed", C.c_uint64),
        ("sr_stream", C.c_uint32),
        ("sr_bits", C.c_uint32),
        ("sign_mode", C.c_uint32),
        ("pad_", C.c_uint32),
        ("sign_seed", C.c_uint64),
    ]


class Stats(C.Structure):
    _fields_ = [
        ("sum_abs_y", C.c_double),
        ("sum_signed_err", C.c_double),
        ("sum_y2", C.c_double),
        ("sum_err2", C.c_double),
        ("sum_err_norm", C.c_double),
        ("sum_err_norm_sat", C.c_double),
        ("level_err_norm", C.c_double * 8),
        ("n", C.c_uint64),
        ("n_saturated", C.c_uint64),
        ("n_nonfinite_blocks", C.c_uint64),
        ("level_count", C.c_uint64 * 8),
    ]

    def as_dict(self) -> dict:
        d = {k: getattr(self, k) for k, _ in self._fields_}
        d["level_err_norm"] = list(self.level_err_norm)
        d["level_count"] = list(self.level_count)
        return d


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = C.CDLL(_LIB_PATH)
        P = C.c_void_p
        i64 = C.c_int64
        L.orc_philox4x32_10.argtypes = [P, P, P]
        L.orc_grid_level.argtypes = [C.c_int, C.c_int]
        L.orc_grid_level.restype = C.c_double
        L.orc_grid_emax.argtypes = [C.c_int]
        L.orc_grid_top.argtypes = [C.c_int]
        L.orc_fwht_f32.argtypes = [P, C.c_int]
        L.orc_rotate_block.argtypes = [P, C.c_int, C.c_uint32, P]
        L.orc_rotate_block_signs.argtypes = [P, C.c_int, C.c_uint32, P]
        L.orc_block_signs.argtypes = [C.POINTER(QParams), C.c_uint64]
        L.orc_block_signs.restype = C.c_uint32
        L.orc_scale_code.argtypes = [C.c_int, P]
        L.orc_round_rtne.argtypes = [C.c_int, C.c_double]
        L.orc_round_sr.argtypes = [C.c_int, C.c_double, C.c_uint32, C.c_int]
        L.orc_sr_random.argtypes = [C.c_uint64, C.c_uint32, C.c_uint64, C.c_int, C.c_int]
        L.orc_sr_random.restype = C.c_uint32
        L.orc_quantize_block.argtypes = [P, C.POINTER(QParams), C.c_uint64, C.c_uint64, P, P]
        L.orc_e2m3_code.argtypes = [C.c_int, C.c_int]
        L.orc_quantize.argtypes = [P, i64, i64, i64, C.c_int, C.POINTER(QParams), C.c_int, P, P]
        L.orc_quantize_lines.argtypes = [P, i64, i64, i64, C.c_int, C.POINTER(QParams), C.c_int,
                                         i64, P, P]
        L.orc_dequantize.argtypes = [P, P, i64, i64, C.c_int, C.c_int, P]
        L.orc_to_mfma_layout.argtypes = [P, P, i64, i64, C.c_int, P, P]
        L.orc_gemm_abt_f64.argtypes = [P, P, i64, i64, i64, P]
        L.orc_stats.argtypes = [P, i64, i64, i64, C.c_int, C.POINTER(QParams), C.c_int, P, P,
                                C.POINTER(Stats)]
        L.orc_rotate.argtypes = [P, i64, i64, i64, C.c_int, C.POINTER(QParams), P]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


def qparams(grid=GRID_E2M1, round=RTNE, hadamard_n=0, sign_mask=0, sr_seed=0, sr_stream=0,
            sr_bits=16, sign_mode=0, sign_seed=0) -> QParams:
    return QParams(grid, round, hadamard_n, sign_mask & 0xFFFFFFFF, sr_seed, sr_stream, sr_bits,
                   sign_mode, 0, sign_seed)


# ---- scalar pieces --------------------------------------------------------

def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, dtype=np.uint32)
    lib().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def grid_levels(grid: int) -> list[float]:
    return [lib().orc_grid_level(grid, m) for m in range(8)]


def grid_emax(grid: int) -> int:
    return lib().orc_grid_emax(grid)


def grid_top(grid: int) -> int:
    """Largest code m the grid emits (7; 6 and 5 for E2M1 capped at 4 and 3)."""
    return lib().orc_grid_top(grid)


def fwht_f32(u: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(u, dtype=np.float32).copy()
    lib().orc_fwht_f32(_ptr(v), v.size)
    return v


def rotate_block(x: np.ndarray, n: int, sign_mask: int = 0) -> np.ndarray:
    xb = np.ascontiguousarray(x, dtype=np.float32)
    assert xb.size == 32
    y = np.zeros(32, dtype=np.float32)
    lib().orc_rotate_block(_ptr(xb), n, sign_mask & 0xFFFFFFFF, _ptr(y))
    return y


def scale_code(grid: int, y: np.ndarray) -> int:
    yb = np.ascontiguousarray(y, dtype=np.float32)
    assert yb.size == 32
    return lib().orc_scale_code(grid, _ptr(yb))


def round_rtne(grid: int, a: float) -> int:
    return lib().orc_round_rtne(grid, float(a))


def round_sr(grid: int, a: float, r: int, bits: int) -> int:
    return lib().orc_round_sr(grid, float(a), r, bits)


def sr_random(seed: int, stream: int, b: int, j: int, bits: int) -> int:
    return lib().orc_sr_random(seed, stream, b, j, bits)


def rotate_block_signs(x: np.ndarray, n: int, signs: int) -> np.ndarray:
    """Rotation of one 32-block with one sign bit per position (bit i: position i)."""
    xb = np.ascontiguousarray(x, dtype=np.float32)
    assert xb.size == 32
    y = np.zeros(32, dtype=np.float32)
    lib().orc_rotate_block_signs(_ptr(xb), n, signs & 0xFFFFFFFF, _ptr(y))
    return y


def block_signs(p: QParams, j: int) -> int:
    """The 32 sign bits of block j along the quantization axis under p."""
    return lib().orc_block_signs(C.byref(p), j)


def quantize_block(x: np.ndarray, p: QParams, block_index: int = 0, j: int = 0):
    xb = np.ascontiguousarray(x, dtype=np.float32)
    nib = np.zeros(32, dtype=np.uint8)
    sc = np.zeros(1, dtype=np.uint8)
    lib().orc_quantize_block(_ptr(xb), C.byref(p), block_index, j, _ptr(nib), _ptr(sc))
    return nib, int(sc[0])


def e2m3_code(grid: int, nibble: int) -> int:
    return lib().orc_e2m3_code(grid, nibble)


# ---- tensor-level ---------------------------------------------------------

def _bf16_bits(x) -> np.ndarray:
    """Accept a uint16 array of bf16 bit patterns (or a torch bf16 tensor)."""
    if hasattr(x, "view") and hasattr(x, "dtype") and str(x.dtype) == "torch.bfloat16":
        import torch
        x = x.contiguous().view(torch.int16).numpy().view(np.uint16)
    x = np.asarray(x)
    assert x.dtype == np.uint16, "oracle expects bf16 bit patterns as uint16"
    return x


def block_bytes(fmt: int) -> int:
    return 16 if fmt == FMT_FP4 else 24


def quantize(x, axis: int, p: QParams, fmt: int = FMT_FP4, ld: int | None = None):
    """Quantize bf16 x [rows x cols].  Returns (codes [lines, k/32*bb], scales [lines, k/32])."""
    xb = np.ascontiguousarray(_bf16_bits(x))
    rows, cols = xb.shape
    ld = cols if ld is None else ld
    lines, k = (rows, cols) if axis == AXIS_ROW else (cols, rows)
    nblk = k // 32
    codes = np.zeros((lines, nblk * block_bytes(fmt)), dtype=np.uint8)
    scales = np.zeros((lines, nblk), dtype=np.uint8)
    rc = lib().orc_quantize(_ptr(xb), rows, cols, ld, axis, C.byref(p), fmt, _ptr(codes),
                            _ptr(scales))
    if rc != 0:
        raise ValueError(f"oracle quantize rejected shape {xb.shape} axis {axis}")
    return codes, scales


def quantize_lines(x, axis: int, p: QParams, line0: int, nlines: int, fmt: int = FMT_FP4):
    """Quantize lines [line0, line0 + nlines) of the bf16 tensor x only (rows for
    AXIS_ROW, columns for AXIS_COL), with the block indices of the whole tensor."""
    xb = _bf16_bits(x)
    sub = xb[line0:line0 + nlines] if axis == AXIS_ROW else xb[:, line0:line0 + nlines]
    sub = np.ascontiguousarray(sub)
    rows, cols = sub.shape
    k = cols if axis == AXIS_ROW else rows
    nblk = k // 32
    codes = np.zeros((nlines, nblk * block_bytes(fmt)), dtype=np.uint8)
    scales = np.zeros((nlines, nblk), dtype=np.uint8)
    rc = lib().orc_quantize_lines(_ptr(sub), rows, cols, cols, axis, C.byref(p), fmt, line0,
                                  _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError("oracle quantize_lines rejected shape")
    return codes, scales


def mfma_layout_sizes(lines: int, k: int, fmt: int):
    ntiles = (lines + 15) // 16
    nsteps = k // 128
    return nsteps * ntiles * 64 * block_bytes(fmt), ((nsteps + 3) // 4) * ntiles * 256


def to_mfma_layout(codes: np.ndarray, scales: np.ndarray, fmt: int, fill: int = 0):
    """Row-layout (codes, scales) -> flat MFMA-layout byte arrays (prefilled with `fill`)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    lines, nblk = scales.shape
    k = nblk * 32
    cb, sb = mfma_layout_sizes(lines, k, fmt)
    tc = np.full(cb, fill, dtype=np.uint8)
    ts = np.full(sb, fill, dtype=np.uint8)
    rc = lib().orc_to_mfma_layout(_ptr(codes), _ptr(scales), lines, k, fmt, _ptr(tc), _ptr(ts))
    if rc != 0:
        raise ValueError("oracle layout: k must be a multiple of 128")
    return tc, ts


def dequantize(codes: np.ndarray, scales: np.ndarray, grid: int, fmt: int = FMT_FP4) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    lines, nblk = scales.shape
    out = np.zeros((lines, nblk * 32), dtype=np.float64)
    rc = lib().orc_dequantize(_ptr(codes), _ptr(scales), lines, nblk * 32, grid, fmt, _ptr(out))
    if rc != 0:
        raise ValueError("oracle dequantize: bad codes")
    return out


def gemm_abt_f64(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float64)
    b = np.ascontiguousarray(b, dtype=np.float64)
    m, k = a.shape
    n, k2 = b.shape
    assert k == k2
    c = np.zeros((m, n), dtype=np.float64)
    lib().orc_gemm_abt_f64(_ptr(a), _ptr(b), m, n, k, _ptr(c))
    return c


def rotate(x, axis: int, hadamard_n: int, sign_mask: int = 0, sign_mode: int = 0,
           sign_seed: int = 0) -> np.ndarray:
    xb = np.ascontiguousarray(_bf16_bits(x))
    rows, cols = xb.shape
    lines, k = (rows, cols) if axis == AXIS_ROW else (cols, rows)
    y = np.zeros((lines, k), dtype=np.float32)
    p = qparams(hadamard_n=hadamard_n, sign_mask=sign_mask, sign_mode=sign_mode,
                sign_seed=sign_seed)
    rc = lib().orc_rotate(_ptr(xb), rows, cols, cols, axis, C.byref(p), _ptr(y))
    if rc != 0:
        raise ValueError("oracle rotate rejected shape")
    return y


def stats(x, axis: int, p: QParams, codes: np.ndarray, scales: np.ndarray,
          fmt: int = FMT_FP4) -> dict:
    xb = np.ascontiguousarray(_bf16_bits(x))
    rows, cols = xb.shape
    st = Stats()
    rc = lib().orc_stats(_ptr(xb), rows, cols, cols, axis, C.byref(p), fmt,
                         _ptr(np.ascontiguousarray(codes)), _ptr(np.ascontiguousarray(scales)),
                         C.byref(st))
    if rc != 0:
        raise ValueError("oracle stats failed")
    return st.as_dict()
