"""CPU checks of the C ABI: the library loads, exports every function that
include/mxq.h declares, and rejects bad arguments with the documented status
before touching the GPU (no compute call is made here)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "mxq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mxq_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for want in ("mxq_quantize", "mxq_quantize_batch", "mxq_dequantize", "mxq_wgrad_gemm", "mxq_bias_stats",
                 "mxq_bias_stats_workspace_size", "mxq_round_to_grid", "mxq_status_string",
                 "mxq_abi_version"):
        assert want in names


def test_library_exports_every_declared_symbol(mxq_lib):
    L = mxq_lib.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name
    assert set(_declared_functions()) == set(mxq_lib.SYMBOLS)


def test_abi_version_and_status_strings(mxq_lib):
    L = mxq_lib.lib()
    import re
    hdr = open(os.path.join(ROOT, "include", "mxq.h")).read()
    assert L.mxq_abi_version() == int(re.search(r"#define MXQ_ABI_VERSION (\d+)", hdr).group(1)) == 5
    for s in range(7):
        assert mxq_lib.status_string(s)
    assert mxq_lib.status_string(0) == "ok"


def _fake(addr=0x10000):
    return C.c_void_p(addr)


def test_quantize_validation(mxq_lib):
    L = mxq_lib.lib()
    M = mxq_lib
    good = M.qconfig()
    out = M.QTensor(0x20000, 0x30000, M.FMT_FP4, M.GRID_E2M1)

    def q(cfg, x=_fake(), rows=64, cols=64, ld=64, row=out, col=None):
        return L.mxq_quantize(C.byref(cfg) if cfg is not None else None, x, rows, cols, ld,
                              C.byref(row) if row is not None else None,
                              C.byref(col) if col is not None else None, None)

    assert q(None) == M.ERR_NULL
    assert q(good, x=None) == M.ERR_NULL
    assert q(good, row=None, col=None) == M.ERR_NULL
    assert q(M.qconfig(grid=4)) == M.ERR_UNSUPPORTED
    assert q(M.qconfig(sign_mode=2)) == M.ERR_UNSUPPORTED
    assert q(M.qconfig(round=5)) == M.ERR_UNSUPPORTED
    assert q(M.qconfig(hadamard_n=8)) == M.ERR_UNSUPPORTED
    assert q(M.qconfig(round=M.SR, sr_bits=12)) == M.ERR_UNSUPPORTED
    assert q(good, cols=48, ld=48) == M.ERR_SHAPE                 # row blocks need cols % 32
    assert q(good, rows=48, row=None, col=out) == M.ERR_SHAPE     # col blocks need rows % 32
    assert q(good, rows=-1) == M.ERR_SHAPE
    assert q(good, ld=32) == M.ERR_SHAPE                          # ld < cols
    assert q(good, x=_fake(0x10001)) == M.ERR_ALIGN               # x not 2-byte aligned
    bad_codes = M.QTensor(0x20002, 0x30000, M.FMT_FP4, M.GRID_E2M1)
    assert q(good, row=bad_codes) == M.ERR_ALIGN
    wrong_grid = M.QTensor(0x20000, 0x30000, M.FMT_FP4, M.GRID_E1M2)
    assert q(good, row=wrong_grid) == M.ERR_UNSUPPORTED
    bad_fmt = M.QTensor(0x20000, 0x30000, 7, M.GRID_E2M1)
    assert q(good, row=bad_fmt) == M.ERR_UNSUPPORTED
    null_codes = M.QTensor(None, 0x30000, M.FMT_FP4, M.GRID_E2M1)
    assert q(good, row=null_codes) == M.ERR_NULL
    # empty inputs are valid and launch nothing
    assert q(good, rows=0) == M.OK
    assert q(good, cols=0, ld=0) == M.OK


def test_quantize_batch_validation(mxq_lib):
    # every job is checked before anything is launched; the first failing
    # job's status comes back, with mxq_quantize's codes
    L = mxq_lib.lib()
    M = mxq_lib
    good, sr = M.qconfig(), M.qconfig(round=M.SR, grid=M.GRID_E1M2)
    out = M.QTensor(0x20000, 0x30000, M.FMT_FP4, M.GRID_E2M1)
    out1 = M.QTensor(0x24000, 0x34000, M.FMT_FP4, M.GRID_E1M2)
    keep = [good, sr, out, out1]

    def job(cfg=good, x=0x10000, rows=64, cols=64, ld=64, row=None, col=out):
        return M.QuantizeJob(C.pointer(cfg) if cfg is not None else None, x, rows, cols, ld,
                             C.pointer(row) if row is not None else None,
                             C.pointer(col) if col is not None else None)

    def b(*jobs, count=None):
        arr = (M.QuantizeJob * max(len(jobs), 1))(*jobs)
        return L.mxq_quantize_batch(arr, len(jobs) if count is None else count, None)

    assert L.mxq_quantize_batch(None, 0, None) == M.OK
    assert L.mxq_quantize_batch(None, 2, None) == M.ERR_NULL
    assert b(job(), count=-1) == M.ERR_SHAPE
    # the bad job is the last one: the good ones before it are not launched
    assert b(job(), job(cfg=sr, col=out1), job(cfg=None)) == M.ERR_NULL
    assert b(job(), job(x=None)) == M.ERR_NULL
    assert b(job(), job(rows=48)) == M.ERR_SHAPE          # column blocks need rows % 32
    assert b(job(), job(col=None, row=None)) == M.ERR_NULL
    assert b(job(), job(cfg=sr, col=out)) == M.ERR_UNSUPPORTED   # output grid != cfg grid
    assert b(job(), job(x=0x10001)) == M.ERR_ALIGN
    assert b(job(), job(cfg=M.qconfig(hadamard_n=8))) == M.ERR_UNSUPPORTED
    # jobs with nothing to do are valid and launch nothing
    assert b(job(rows=0), job(cols=0, ld=0), job(cfg=sr, col=out1, rows=0)) == M.OK
    del keep


def test_gemm_validation(mxq_lib):
    L = mxq_lib.lib()
    M = mxq_lib
    a = M.QTensor(0x20000, 0x30000, M.FMT_FP4, M.GRID_E2M1)
    b6 = M.QTensor(0x40000, 0x50000, M.FMT_E2M3, M.GRID_E1M2)
    c = _fake(0x60000)

    def g(a_, b_, m=64, n=64, k=256, cptr=c, ldc=64):
        return L.mxq_wgrad_gemm(C.byref(a_) if a_ else None, C.byref(b_) if b_ else None, m, n, k,
                                cptr, ldc, None)

    assert g(None, a) == M.ERR_NULL
    assert g(a, a, cptr=None) == M.ERR_NULL
    e1m2_nibbles = M.QTensor(0x20000, 0x30000, M.FMT_FP4, M.GRID_E1M2)
    assert g(e1m2_nibbles, a) == M.ERR_UNSUPPORTED     # no matrix-core type for E1M2 nibbles
    assert g(a, b6, k=96) == M.ERR_SHAPE
    assert g(a, b6, ldc=32) == M.ERR_SHAPE
    assert g(a, b6, m=-3) == M.ERR_SHAPE
    assert g(M.QTensor(0x20008, 0x30000, M.FMT_FP4, M.GRID_E2M1), b6) == M.ERR_ALIGN
    assert g(a, b6, m=0) == M.OK


def test_dequant_stats_round_validation(mxq_lib):
    L = mxq_lib.lib()
    M = mxq_lib
    q = M.QTensor(0x20000, 0x30000, M.FMT_FP4, M.GRID_E2M1)
    assert L.mxq_dequantize(None, 4, 64, 0, _fake(), 64, None) == M.ERR_NULL
    assert L.mxq_dequantize(C.byref(q), 4, 48, 0, _fake(), 64, None) == M.ERR_SHAPE
    assert L.mxq_dequantize(C.byref(q), 4, 64, 9, _fake(), 64, None) == M.ERR_UNSUPPORTED
    assert L.mxq_dequantize(C.byref(q), 4, 64, 0, _fake(0x10004), 64, None) == M.ERR_ALIGN
    cfg = M.qconfig()
    ws = L.mxq_bias_stats_workspace_size(64, 64, 0)
    assert ws > 0
    assert L.mxq_bias_stats(C.byref(cfg), _fake(), 64, 64, 64, 0, C.byref(q), _fake(0x70000),
                            None, 0, None) == M.ERR_WORKSPACE
    assert L.mxq_bias_stats(C.byref(cfg), _fake(), 64, 64, 64, 0, C.byref(q), _fake(0x70000),
                            _fake(0x80000), ws - 8, None) == M.ERR_WORKSPACE
    assert L.mxq_bias_stats(C.byref(cfg), _fake(), 64, 64, 64, 3, C.byref(q), _fake(0x70000),
                            _fake(0x80000), ws, None) == M.ERR_UNSUPPORTED
    assert L.mxq_round_to_grid(4, 0, 16, _fake(), None, 10, _fake(), None) == M.ERR_UNSUPPORTED
    assert L.mxq_round_to_grid(-1, 0, 16, _fake(), None, 10, _fake(), None) == M.ERR_UNSUPPORTED
    assert L.mxq_round_to_grid(0, 1, 16, _fake(), None, 10, _fake(), None) == M.ERR_NULL
    assert L.mxq_round_to_grid(0, 0, 16, _fake(), None, -1, _fake(), None) == M.ERR_SHAPE


def test_product_path_has_no_oracle_dependency():
    # the binding and the sources never reference the oracle
    pkg = os.path.join(ROOT, "fp4_microscaling_quantization_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower() or f == "synth.py", f


def test_binding_is_argument_marshalling_only():
    """The Python binding computes nothing of the method: it imports no math
    or array library, holds no floating-point literal, and uses no true
    division, power or math call; its only arithmetic is integer buffer
    sizing (block and tile counts).  Every diagnostic it exposes calls the
    library (the bucket ratio is mxq_bucket_ratio)."""
    import ast
    src = open(os.path.join(ROOT, "fp4_microscaling_quantization_amd", "mxq.py")).read()
    tree = ast.parse(src)
    for node in ast.walk(tree):
        if isinstance(node, (ast.Import, ast.ImportFrom)):
            mods = [a.name for a in node.names] if isinstance(node, ast.Import) else [node.module]
            for m in mods:
                assert m.split(".")[0] not in ("math", "numpy", "statistics", "cmath", "scipy"), m
        if isinstance(node, ast.Constant) and isinstance(node.value, float):
            raise AssertionError(f"float literal {node.value} at line {node.lineno}")
        if isinstance(node, ast.BinOp):
            assert not isinstance(node.op, (ast.Div, ast.Pow)), node.lineno
        if isinstance(node, ast.Attribute) and isinstance(node.value, ast.Name):
            assert node.value.id not in ("math", "np", "numpy"), node.lineno


def test_bucket_ratio_is_the_library_call(mxq_lib):
    # the binding's bucket_ratio is marshalling around mxq_bucket_ratio
    import ctypes as C
    L = mxq_lib.lib()
    st = mxq_lib.Stats()
    for m, c in enumerate([3, 1, 0, 4, 0, 0, 0, 2]):
        st.level_count[m] = c
    assert L.mxq_bucket_ratio(C.byref(st), mxq_lib.GRID_E1M2) == \
        mxq_lib.bucket_ratio([3, 1, 0, 4, 0, 0, 0, 2], mxq_lib.GRID_E1M2)
    import math
    assert math.isnan(L.mxq_bucket_ratio(None, 0))
    assert math.isnan(L.mxq_bucket_ratio(C.byref(st), 9))


def test_rht_sign_mask_is_philox_word0(mxq_lib, orc):
    """mxq_rht_sign_mask (host code of the library) against the oracle's own
    Philox4x32-10, itself pinned to rocRAND: word 0 of the draw at counter
    (0, ~0, ~0, ~0) under key (lo, hi) of the seed, low n bits."""
    for seed in (0, 1, 1002, 1005, 0xDEADBEEFCAFEF00D, (1 << 64) - 1):
        w = int(orc.philox4x32_10([0, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF],
                                  [seed & 0xFFFFFFFF, seed >> 32])[0])
        assert mxq_lib.rht_sign_mask(seed, 32) == w
        assert mxq_lib.rht_sign_mask(seed, 16) == w & 0xFFFF
    assert mxq_lib.rht_sign_mask(7, 8) == 0


def test_prepared_calls_hold_their_buffers(mxq_lib):
    """A prepared call launches later on raw device pointers, so it must keep
    every tensor it was given alive: a freed buffer would go back to the
    allocator and could be handed to another tensor (timing loops that
    rotate several buffer sets would then all touch the same memory).  Only
    marshalling runs here; nothing is launched."""
    import gc
    import types
    import weakref

    import torch
    mxq = mxq_lib
    cfg = mxq.qconfig(hadamard_n=16)
    st = types.SimpleNamespace(cuda_stream=0)      # a stream handle; nothing is launched

    def alive_after(make):
        tensors, call = make()
        refs = [weakref.ref(t) for t in tensors]
        del tensors
        gc.collect()
        assert all(r() is not None for r in refs)
        del call
        gc.collect()
        assert all(r() is None for r in refs)

    def quantize():
        x = torch.zeros((32, 64), dtype=torch.bfloat16)
        rc, rs = torch.zeros(32 * 2 * 16, dtype=torch.uint8), torch.zeros(64, dtype=torch.uint8)
        cc, cs = torch.zeros(64 * 16, dtype=torch.uint8), torch.zeros(64, dtype=torch.uint8)
        return [x, rc, rs, cc, cs], mxq.prepare_quantize(cfg, x, row=(rc, rs, mxq.FMT_FP4),
                                                         col=(cc, cs, mxq.FMT_FP4), stream=st)

    def batch():
        x = torch.zeros((32, 64), dtype=torch.bfloat16)
        cc, cs = torch.zeros(64 * 16, dtype=torch.uint8), torch.zeros(64, dtype=torch.uint8)
        return [x, cc, cs], mxq.prepare_quantize_batch([(cfg, x, None, (cc, cs, mxq.FMT_FP4))],
                                                          stream=st)

    def gemm():
        ac, as_ = torch.zeros(16 * 4 * 16, dtype=torch.uint8), torch.zeros(16 * 4, dtype=torch.uint8)
        bc, bs = torch.zeros(16 * 4 * 16, dtype=torch.uint8), torch.zeros(16 * 4, dtype=torch.uint8)
        out = torch.zeros((16, 16), dtype=torch.float32)
        return [ac, as_, bc, bs, out], mxq.prepare_wgrad_gemm(
            ac, as_, mxq.FMT_FP4, mxq.GRID_E2M1, bc, bs, mxq.FMT_FP4, mxq.GRID_E2M1, out,
            mxq.LAYOUT_ROWS, 16, 16, 128, stream=st)

    def rotate():
        x = torch.zeros((32, 64), dtype=torch.bfloat16)
        out = torch.zeros((32, 64), dtype=torch.float32)
        return [x, out], mxq.prepare_rotate(x, mxq.AXIS_ROW, 16, 0, mxq.OUT_F32, out, stream=st)

    for make in (quantize, batch, gemm, rotate):
        alive_after(make)
