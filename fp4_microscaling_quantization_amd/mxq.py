"""Thin ctypes binding of libmxq (include/mxq.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libmxq.so.  PyTorch supplies device memory and the current stream.
Loading fails loudly when the library has not been built; there is no
fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmxq.so")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_UNSUPPORTED, ERR_DEVICE, ERR_WORKSPACE = range(7)
GRID_E2M1, GRID_E1M2, GRID_E2M1_MAX4, GRID_E2M1_MAX3 = 0, 1, 2, 3
RTNE, SR = 0, 1
FMT_FP4, FMT_E2M3 = 0, 1
LAYOUT_ROWS, LAYOUT_MFMA = 0, 1
AXIS_ROW, AXIS_COL = 0, 1
OUT_F32, OUT_BF16 = 0, 1
SIGNS_MASK, SIGNS_PER_BLOCK = 0, 1

SYMBOLS = ("mxq_quantize", "mxq_quantize_batch", "mxq_dequantize", "mxq_wgrad_gemm", "mxq_gemm_abt", "mxq_bias_stats",
           "mxq_bias_stats_workspace_size", "mxq_bias_stats_noalloc", "mxq_bucket_ratio", "mxq_round_to_grid", "mxq_rht_sign_mask", "mxq_rotate",
           "mxq_status_string", "mxq_abi_version")


class QConfig(C.Structure):
    _fields_ = [("grid", C.c_int32), ("round", C.c_int32), ("hadamard_n", C.c_int32),
                ("sign_mask", C.c_uint32), ("sr_seed", C.c_uint64), ("sr_stream", C.c_uint32),
                ("sr_bits", C.c_uint32), ("sign_mode", C.c_uint32), ("reserved", C.c_uint32),
                ("sign_seed", C.c_uint64)]


class QTensor(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("fmt", C.c_int32),
                ("grid", C.c_int32), ("layout", C.c_int32)]


class QuantizeJob(C.Structure):
    _fields_ = [("cfg", C.POINTER(QConfig)), ("x", C.c_void_p), ("rows", C.c_int64),
                ("cols", C.c_int64), ("ld_x", C.c_int64), ("row_out", C.POINTER(QTensor)),
                ("col_out", C.POINTER(QTensor))]


class Stats(C.Structure):
    _fields_ = [("sum_abs_y", C.c_double), ("sum_signed_err", C.c_double),
                ("sum_y2", C.c_double), ("sum_err2", C.c_double), ("sum_err_norm", C.c_double),
                ("sum_err_norm_sat", C.c_double), ("level_err_norm", C.c_double * 8),
                ("n", C.c_uint64), ("n_saturated", C.c_uint64),
                ("n_nonfinite_blocks", C.c_uint64), ("level_count", C.c_uint64 * 8)]


class MxqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})")
        self.status = status


_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libmxq.so is not built ({LIB_PATH}); run "
                              "`python -m fp4_microscaling_quantization_amd.build` first")
        L = C.CDLL(LIB_PATH)
        P, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
        L.mxq_quantize.argtypes = [C.POINTER(QConfig), P, i64, i64, i64, C.POINTER(QTensor),
                                   C.POINTER(QTensor), P]
        L.mxq_quantize_batch.argtypes = [C.POINTER(QuantizeJob), i32, P]
        L.mxq_dequantize.argtypes = [C.POINTER(QTensor), i64, i64, i32, P, i64, P]
        L.mxq_wgrad_gemm.argtypes = [C.POINTER(QTensor), C.POINTER(QTensor), i64, i64, i64, P,
                                     i64, P]
        L.mxq_gemm_abt.argtypes = L.mxq_wgrad_gemm.argtypes
        L.mxq_rht_sign_mask.argtypes = [C.c_uint64, C.c_uint32]
        L.mxq_rotate.argtypes = [C.POINTER(QConfig), P, i64, i64, i64, i32, i32, P, i64, P]
        L.mxq_rht_sign_mask.restype = C.c_uint32
        L.mxq_bias_stats.argtypes = [C.POINTER(QConfig), P, i64, i64, i64, i32, C.POINTER(QTensor),
                                     P, P, C.c_size_t, P]
        L.mxq_bias_stats_noalloc.argtypes = [C.POINTER(QConfig), P, i64, i64, i64, i32,
                                             C.POINTER(QTensor), P, P]
        L.mxq_bias_stats_workspace_size.argtypes = [i64, i64, i32]
        L.mxq_bias_stats_workspace_size.restype = C.c_size_t
        L.mxq_round_to_grid.argtypes = [i32, i32, i32, P, P, i64, P, P]
        L.mxq_bucket_ratio.argtypes = [C.POINTER(Stats), i32]
        L.mxq_bucket_ratio.restype = C.c_double
        L.mxq_status_string.argtypes = [i32]
        L.mxq_status_string.restype = C.c_char_p
        L.mxq_abi_version.restype = i32
        for name in ("mxq_quantize", "mxq_quantize_batch", "mxq_dequantize", "mxq_wgrad_gemm", "mxq_gemm_abt",
                     "mxq_bias_stats", "mxq_bias_stats_noalloc", "mxq_round_to_grid", "mxq_rotate"):
            getattr(L, name).restype = i32
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().mxq_status_string(status).decode()


def _check(fn: str, status: int):
    if status != OK:
        raise MxqError(fn, status)


def _ptr(t) -> C.c_void_p | None:
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def qconfig(grid=GRID_E2M1, round=RTNE, hadamard_n=0, sign_mask=0, sr_seed=0, sr_stream=0,
            sr_bits=16, sign_mode=SIGNS_MASK, sign_seed=0) -> QConfig:
    return QConfig(grid, round, hadamard_n, sign_mask & 0xFFFFFFFF, sr_seed, sr_stream, sr_bits,
                   sign_mode, 0, sign_seed)


def block_bytes(fmt: int) -> int:
    return 16 if fmt == FMT_FP4 else 24


def qtensor_sizes(lines: int, k: int, fmt: int, layout: int = LAYOUT_ROWS):
    """(code bytes, scale bytes) of a [lines x k] block-quantized tensor."""
    nb = k // 32
    if layout == LAYOUT_ROWS:
        return lines * nb * block_bytes(fmt), lines * nb
    ntiles = (lines + 15) // 16
    nsteps = k // 128
    return nsteps * ntiles * 64 * block_bytes(fmt), ((nsteps + 3) // 4) * ntiles * 256


def empty_qtensor(lines: int, k: int, fmt: int, device, layout: int = LAYOUT_ROWS, fill=None):
    """Device buffers (codes, scales): 2-D [lines, ...] for the row layout,
    1-D byte arrays for the MFMA layout."""
    import torch
    nb = k // 32
    if layout == LAYOUT_ROWS:
        codes = torch.empty((lines, nb * block_bytes(fmt)), dtype=torch.uint8, device=device)
        scales = torch.empty((lines, nb), dtype=torch.uint8, device=device)
    else:
        cb, sb = qtensor_sizes(lines, k, fmt, layout)
        codes = torch.empty(cb, dtype=torch.uint8, device=device)
        scales = torch.empty(sb, dtype=torch.uint8, device=device)
    if fill is not None:
        codes.fill_(fill)
        scales.fill_(fill)
    return codes, scales


def qtensor(codes, scales, fmt: int, grid: int, layout: int = LAYOUT_ROWS) -> QTensor:
    return QTensor(codes.data_ptr(), scales.data_ptr(), fmt, grid, layout)


# ---- entry points ---------------------------------------------------------

def quantize_into(cfg: QConfig, x, row=None, col=None, rows=None, cols=None, ld=None,
                  stream=None):
    """mxq_quantize on caller-owned buffers.
    row/col: (codes, scales, fmt) or (codes, scales, fmt, layout), or None."""
    rows = x.shape[0] if rows is None else rows
    cols = x.shape[1] if cols is None else cols
    ld = x.stride(0) if ld is None else ld

    def desc(o):
        if not o:
            return None
        lay = o[3] if len(o) > 3 else LAYOUT_ROWS
        return QTensor(o[0].data_ptr(), o[1].data_ptr(), o[2], cfg.grid, lay)
    rt, ct = desc(row), desc(col)
    st = lib().mxq_quantize(C.byref(cfg), _ptr(x), rows, cols, ld,
                            C.byref(rt) if rt else None, C.byref(ct) if ct else None,
                            _stream(stream))
    _check("mxq_quantize", st)


def prepare_quantize(cfg: QConfig, x, row=None, col=None, stream=None):
    """The call quantize_into(cfg, x, row, col) marshalled once: returns a
    function of no arguments that launches it again on the same buffers (for
    timing loops, where per-call argument conversion would leave the GPU
    waiting on the host).  The function holds every tensor it was given, so
    their memory cannot be freed and handed to another tensor while it can
    still launch."""
    rows, cols, ld = x.shape[0], x.shape[1], x.stride(0)

    def desc(o):
        if not o:
            return None
        lay = o[3] if len(o) > 3 else LAYOUT_ROWS
        return QTensor(o[0].data_ptr(), o[1].data_ptr(), o[2], cfg.grid, lay)
    rt, ct = desc(row), desc(col)
    cfg_ = QConfig.from_buffer_copy(cfg)
    args = (C.byref(cfg_), _ptr(x), rows, cols, ld, C.byref(rt) if rt else None,
            C.byref(ct) if ct else None, _stream(stream))
    fn = lib().mxq_quantize
    keep = (cfg_, rt, ct, x, row, col)

    def call():
        _check("mxq_quantize", fn(*args))
    call._keep = keep
    return call


def _addr(t) -> int:
    """Device address of t; an empty view keeps the address of its storage
    (torch reports 0 for tensors without elements)."""
    p = t.data_ptr()
    if p == 0 and t.numel() == 0:
        p = t.untyped_storage().data_ptr() + t.storage_offset() * t.element_size()
    return p


def _batch_args(jobs):
    """ctypes array of QuantizeJob for [(cfg, x, row, col), ...] (row / col as
    in quantize_into) and the objects it points into."""
    arr = (QuantizeJob * len(jobs))()
    keep = [arr]
    for i, (cfg, x, row, col) in enumerate(jobs):
        cfg_ = QConfig.from_buffer_copy(cfg)

        def desc(o):
            if not o:
                return None
            lay = o[3] if len(o) > 3 else LAYOUT_ROWS
            return QTensor(o[0].data_ptr(), o[1].data_ptr(), o[2], cfg_.grid, lay)
        rt, ct = desc(row), desc(col)
        keep += [cfg_, rt, ct, x, row, col]
        arr[i] = QuantizeJob(C.pointer(cfg_), _addr(x), x.shape[0], x.shape[1], x.stride(0),
                             C.pointer(rt) if rt else None, C.pointer(ct) if ct else None)
    return arr, keep


def quantize_batch(jobs, stream=None):
    """mxq_quantize_batch: jobs = [(cfg, x, row, col), ...] with row / col
    (codes, scales, fmt[, layout]) or None, as quantize_into."""
    arr, keep = _batch_args(jobs)
    st = lib().mxq_quantize_batch(arr, len(jobs), _stream(stream))
    del keep
    _check("mxq_quantize_batch", st)


def prepare_quantize_batch(jobs, stream=None):
    """quantize_batch(jobs) marshalled once (see prepare_quantize; the function
    holds every job's tensors)."""
    arr, keep = _batch_args(jobs)
    args = (arr, len(jobs), _stream(stream))
    fn = lib().mxq_quantize_batch

    def call():
        _check("mxq_quantize_batch", fn(*args))
    call._keep = keep
    return call


def quantize(x, grid=GRID_E2M1, round=RTNE, hadamard_n=0, sign_mask=0, sr_seed=0, sr_stream=0,
             sr_bits=16, row=True, col=False, row_fmt=FMT_FP4, col_fmt=FMT_FP4,
             row_layout=LAYOUT_ROWS, col_layout=LAYOUT_ROWS, fill=None, stream=None,
             sign_mode=SIGNS_MASK, sign_seed=0):
    """Quantize a 2-D bf16 CUDA tensor; returns {'row': (codes, scales), 'col': (...)}."""
    cfg = qconfig(grid, round, hadamard_n, sign_mask, sr_seed, sr_stream, sr_bits, sign_mode,
                  sign_seed)
    rows, cols = x.shape
    out = {}
    r = c = None
    if row:
        rc, rs = empty_qtensor(rows, cols, row_fmt, x.device, row_layout, fill)
        r = (rc, rs, row_fmt, row_layout)
        out["row"] = (rc, rs)
    if col:
        cc, cs = empty_qtensor(cols, rows, col_fmt, x.device, col_layout, fill)
        c = (cc, cs, col_fmt, col_layout)
        out["col"] = (cc, cs)
    quantize_into(cfg, x, r, c, stream=stream)
    return out


def dequantize(codes, scales, fmt: int, grid: int, out_dtype=OUT_F32, layout=LAYOUT_ROWS,
               lines=None, k=None, stream=None):
    import torch
    if layout == LAYOUT_ROWS:
        lines = scales.shape[0] if lines is None else lines
        k = scales.shape[1] * 32 if k is None else k
    dt = torch.float32 if out_dtype == OUT_F32 else torch.bfloat16
    out = torch.empty((lines, k), dtype=dt, device=codes.device)
    q = qtensor(codes, scales, fmt, grid, layout)
    _check("mxq_dequantize", lib().mxq_dequantize(C.byref(q), lines, k, out_dtype, _ptr(out), k,
                                                  _stream(stream)))
    return out


def wgrad_gemm(a_codes, a_scales, a_fmt, a_grid, b_codes, b_scales, b_fmt, b_grid, out=None,
               layout=LAYOUT_ROWS, m=None, n=None, k=None, stream=None):
    """C [m x n] fp32 = A [m x k] B [n x k]^T on block-quantized operands (both
    in `layout`; m, n, k are required for the MFMA layout)."""
    import torch
    if layout == LAYOUT_ROWS:
        m = a_scales.shape[0] if m is None else m
        n = b_scales.shape[0] if n is None else n
        k = a_scales.shape[1] * 32 if k is None else k
        assert b_scales.shape[1] * 32 == k
    c = torch.empty((m, n), dtype=torch.float32, device=a_codes.device) if out is None else out
    qa = qtensor(a_codes, a_scales, a_fmt, a_grid, layout)
    qb = qtensor(b_codes, b_scales, b_fmt, b_grid, layout)
    _check("mxq_wgrad_gemm", lib().mxq_wgrad_gemm(C.byref(qa), C.byref(qb), m, n, k, _ptr(c),
                                                  c.stride(0), _stream(stream)))
    return c


def prepare_wgrad_gemm(a_codes, a_scales, a_fmt, a_grid, b_codes, b_scales, b_fmt, b_grid, out,
                       layout, m, n, k, stream=None, entry="mxq_wgrad_gemm"):
    """wgrad_gemm(...) marshalled once into a function of no arguments
    (entry="mxq_gemm_abt" for the same product under its general name) that
    holds every tensor it was given."""
    qa = qtensor(a_codes, a_scales, a_fmt, a_grid, layout)
    qb = qtensor(b_codes, b_scales, b_fmt, b_grid, layout)
    args = (C.byref(qa), C.byref(qb), m, n, k, _ptr(out), out.stride(0), _stream(stream))
    fn = getattr(lib(), entry)

    def call():
        _check(entry, fn(*args))
    call._keep = (qa, qb, a_codes, a_scales, b_codes, b_scales, out)
    return call


def gemm_abt(a_codes, a_scales, a_fmt, a_grid, b_codes, b_scales, b_fmt, b_grid, out=None,
             layout=LAYOUT_ROWS, m=None, n=None, k=None, stream=None):
    """C [m x n] fp32 = A [m x k] B [n x k]^T through mxq_gemm_abt: Fprop
    (X row-wise, W row-wise), Dgrad (dY row-wise, W column-wise) or Wgrad
    (dY column-wise, X column-wise)."""
    import torch
    if layout == LAYOUT_ROWS:
        m = a_scales.shape[0] if m is None else m
        n = b_scales.shape[0] if n is None else n
        k = a_scales.shape[1] * 32 if k is None else k
    c = torch.empty((m, n), dtype=torch.float32, device=a_codes.device) if out is None else out
    qa = qtensor(a_codes, a_scales, a_fmt, a_grid, layout)
    qb = qtensor(b_codes, b_scales, b_fmt, b_grid, layout)
    _check("mxq_gemm_abt", lib().mxq_gemm_abt(C.byref(qa), C.byref(qb), m, n, k, _ptr(c),
                                              c.stride(0), _stream(stream)))
    return c


def rotate(x, axis: int, hadamard_n: int, sign_mask: int = 0, out_dtype=OUT_F32, out=None,
           stream=None, sign_mode=SIGNS_MASK, sign_seed=0):
    """The block rotation alone, in x's orientation (fp32 or bf16 out)."""
    import torch
    dt = torch.float32 if out_dtype == OUT_F32 else torch.bfloat16
    o = torch.empty(x.shape, dtype=dt, device=x.device) if out is None else out
    cfg = qconfig(hadamard_n=hadamard_n, sign_mask=sign_mask, sign_mode=sign_mode,
                  sign_seed=sign_seed)
    _check("mxq_rotate", lib().mxq_rotate(C.byref(cfg), _ptr(x), x.shape[0], x.shape[1],
                                          x.stride(0), axis, out_dtype, _ptr(o), o.stride(0),
                                          _stream(stream)))
    return o


def prepare_rotate(x, axis: int, hadamard_n: int, sign_mask: int, out_dtype, out, stream=None):
    """rotate(...) marshalled once into a function of no arguments that holds
    x and out."""
    cfg = qconfig(hadamard_n=hadamard_n, sign_mask=sign_mask)
    args = (C.byref(cfg), _ptr(x), x.shape[0], x.shape[1], x.stride(0), axis, out_dtype, _ptr(out),
            out.stride(0), _stream(stream))
    fn = lib().mxq_rotate

    def call():
        _check("mxq_rotate", fn(*args))
    call._keep = (cfg, x, out)
    return call


def rht_sign_mask(seed: int, n: int) -> int:
    """Sign mask of the randomized Hadamard rotation drawn from `seed` (host)."""
    return int(lib().mxq_rht_sign_mask(seed, n))


def bias_stats(x, axis: int, codes, scales, fmt: int, grid=GRID_E2M1, round=RTNE, hadamard_n=0,
               sign_mask=0, sr_seed=0, sr_stream=0, sr_bits=16, stream=None,
               sign_mode=SIGNS_MASK, sign_seed=0) -> dict:
    import torch
    cfg = qconfig(grid, round, hadamard_n, sign_mask, sr_seed, sr_stream, sr_bits, sign_mode,
                  sign_seed)
    rows, cols = x.shape
    wsb = lib().mxq_bias_stats_workspace_size(rows, cols, axis)
    ws = torch.empty(max(wsb, 8), dtype=torch.uint8, device=x.device)
    out = torch.zeros(C.sizeof(Stats), dtype=torch.uint8, device=x.device)
    q = qtensor(codes, scales, fmt, grid)
    _check("mxq_bias_stats", lib().mxq_bias_stats(C.byref(cfg), _ptr(x), rows, cols, x.stride(0),
                                                  axis, C.byref(q), _ptr(out), _ptr(ws), wsb,
                                                  _stream(stream)))
    return _stats_dict(out)


def prepare_bias_stats(x, axis: int, codes, scales, fmt: int, out, ws, grid=GRID_E2M1,
                       round=RTNE, hadamard_n=0, sign_mask=0, sr_seed=0, sr_stream=0,
                       sr_bits=16, stream=None, sign_mode=SIGNS_MASK, sign_seed=0):
    """bias_stats(...) marshalled once into a function of no arguments that
    holds every tensor it was given: `out` is a device byte tensor of
    sizeof(mxq_stats), `ws` one of at least mxq_bias_stats_workspace_size
    bytes.  The call leaves the statistics in `out` (no host copy)."""
    cfg = qconfig(grid, round, hadamard_n, sign_mask, sr_seed, sr_stream, sr_bits, sign_mode,
                  sign_seed)
    rows, cols = x.shape
    q = qtensor(codes, scales, fmt, grid)
    args = (C.byref(cfg), _ptr(x), rows, cols, x.stride(0), axis, C.byref(q), _ptr(out),
            _ptr(ws), ws.numel(), _stream(stream))
    fn = lib().mxq_bias_stats

    def call():
        _check("mxq_bias_stats", fn(*args))
    call._keep = (cfg, q, x, codes, scales, out, ws)
    return call


def _stats_dict(out) -> dict:
    """The mxq_stats a call wrote into the device byte tensor `out`."""
    st = Stats.from_buffer_copy(bytes(out.cpu().numpy().tobytes()))
    d = {k: getattr(st, k) for k, _ in Stats._fields_}
    d["level_err_norm"] = list(st.level_err_norm)
    d["level_count"] = list(st.level_count)
    return d


def bias_stats_noalloc(x, axis: int, codes, scales, fmt: int, out=None, grid=GRID_E2M1, round=RTNE,
                       hadamard_n=0, sign_mask=0, sr_seed=0, sr_stream=0, sr_bits=16, stream=None,
                       sign_mode=SIGNS_MASK, sign_seed=0, raw=False):
    """mxq_bias_stats_noalloc into `out` (a device byte tensor of sizeof(mxq_stats),
    allocated here when not given); returns the stats dict, or `out` itself
    when raw=True (no host copy)."""
    import torch
    cfg = qconfig(grid, round, hadamard_n, sign_mask, sr_seed, sr_stream, sr_bits, sign_mode,
                  sign_seed)
    rows, cols = x.shape
    if out is None:
        out = torch.zeros(C.sizeof(Stats), dtype=torch.uint8, device=x.device)
    q = qtensor(codes, scales, fmt, grid)
    _check("mxq_bias_stats_noalloc",
           lib().mxq_bias_stats_noalloc(C.byref(cfg), _ptr(x), rows, cols, x.stride(0), axis,
                                        C.byref(q), _ptr(out), _stream(stream)))
    return out if raw else _stats_dict(out)


def bucket_ratio(level_count, grid: int) -> float:
    """mxq_bucket_ratio on a histogram of magnitude codes (8 counts)."""
    st = Stats()
    for m, c in enumerate(level_count[:8]):
        st.level_count[m] = int(c)
    return float(lib().mxq_bucket_ratio(C.byref(st), grid))


def round_to_grid(a, grid: int, round=RTNE, rand=None, sr_bits=16, out=None, stream=None):
    """Nibble of each fp32 value of `a` (already divided by its block scale)."""
    import torch
    n = a.numel()
    codes = torch.empty(n, dtype=torch.uint8, device=a.device) if out is None else out
    _check("mxq_round_to_grid", lib().mxq_round_to_grid(grid, round, sr_bits, _ptr(a), _ptr(rand),
                                                        n, _ptr(codes), _stream(stream)))
    return codes
