"""GPU edge cases: empty inputs (every entry point returns OK and writes
nothing), the empty reduction of the GEMM (C = 0), and the largest number of
rows the column-wise quantizer's launch allows (65535 row tiles of 128),
checked on sampled lines against the oracle."""
import ctypes as C

import numpy as np
import pytest

from fp4_microscaling_quantization_amd import synth
from gpuhelp import dev, host, say, to_dev_bf16

pytestmark = pytest.mark.gpu


def _buf(nbytes, fill):
    import torch
    return torch.full((nbytes,), fill, dtype=torch.uint8, device=dev())


def test_empty_inputs_are_noops():
    import torch
    from fp4_microscaling_quantization_amd import mxq
    L = mxq.lib()
    x = _buf(256, 0x3F)
    codes, scales = _buf(256, 0xA5), _buf(64, 0xA5)
    q = mxq.QTensor(codes.data_ptr(), scales.data_ptr(), mxq.FMT_FP4, mxq.GRID_E2M1, mxq.LAYOUT_ROWS)
    cfg = mxq.qconfig(hadamard_n=16)
    s = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    say("empty quantize")
    assert L.mxq_quantize(C.byref(cfg), C.c_void_p(x.data_ptr()), 0, 64, 64, C.byref(q), None, s) == mxq.OK
    assert L.mxq_quantize(C.byref(cfg), C.c_void_p(x.data_ptr()), 64, 0, 0, None, C.byref(q), s) == mxq.OK
    assert L.mxq_quantize(C.byref(cfg), C.c_void_p(x.data_ptr()), 0, 0, 0, C.byref(q), C.byref(q), s) == mxq.OK
    say("empty dequantize / rotate / round")
    out = _buf(256, 0x77)
    assert L.mxq_dequantize(C.byref(q), 0, 64, mxq.OUT_F32, C.c_void_p(out.data_ptr()), 64, s) == mxq.OK
    assert L.mxq_rotate(C.byref(cfg), C.c_void_p(x.data_ptr()), 0, 64, 64, mxq.AXIS_ROW, mxq.OUT_F32,
                        C.c_void_p(out.data_ptr()), 64, s) == mxq.OK
    assert L.mxq_round_to_grid(0, 0, 16, None, None, 0, None, s) == mxq.OK
    say("empty gemm")
    qa = mxq.QTensor(codes.data_ptr(), scales.data_ptr(), mxq.FMT_FP4, mxq.GRID_E2M1, mxq.LAYOUT_ROWS)
    cf = torch.full((4, 4), float("nan"), device=dev())
    assert L.mxq_wgrad_gemm(C.byref(qa), C.byref(qa), 0, 4, 128, C.c_void_p(cf.data_ptr()), 4, s) == mxq.OK
    assert L.mxq_wgrad_gemm(C.byref(qa), C.byref(qa), 4, 0, 128, C.c_void_p(cf.data_ptr()), 4, s) == mxq.OK
    torch.cuda.synchronize()
    assert bool(torch.isnan(cf).all())                      # untouched
    assert bool((codes == 0xA5).all()) and bool((scales == 0xA5).all()) and bool((out == 0x77).all())


@pytest.mark.parametrize("layout", [0, 1], ids=["rows", "mfma"])
def test_gemm_empty_reduction_writes_zeros(layout):
    import torch
    from fp4_microscaling_quantization_amd import mxq
    codes, scales = _buf(4096, 0x11), _buf(256, 127)
    q = mxq.QTensor(codes.data_ptr(), scales.data_ptr(), mxq.FMT_FP4, mxq.GRID_E2M1, layout)
    s = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    for m, n in ((5, 7), (300, 260)):
        say("gemm k=0", m, n, layout)
        c = torch.full((m, n + 3), float("nan"), device=dev())
        assert mxq.lib().mxq_wgrad_gemm(C.byref(q), C.byref(q), m, n, 0, C.c_void_p(c.data_ptr()),
                                        n + 3, s) == mxq.OK
        got = host(c)
        assert np.all(got[:, :n] == 0.0)
        assert np.all(np.isnan(got[:, n:]))               # the ldc padding is left alone


def test_largest_column_launch(orc):
    # 65535 row tiles of 128 rows: the largest rows the column kernel's 2-D
    # launch covers; one more tile is rejected on the host
    from fp4_microscaling_quantization_amd import mxq
    rows, cols = 65535 * 128, 32
    x = synth.laplace_outlier_entries(rows, cols, seed=41, out_seed=42, frac=1e-4)
    kw = dict(grid=mxq.GRID_E1M2, round=mxq.SR, hadamard_n=16, sign_mask=synth.sign_mask(43, 16),
              sr_seed=44)
    say("largest column launch", rows, cols)
    q = mxq.quantize(to_dev_bf16(x), row=False, col=True, col_fmt=mxq.FMT_E2M3, **kw)["col"]
    gc, gs = host(q[0]), host(q[1])
    p = orc.qparams(**kw)
    for line in (0, 17, 31):
        c, s = orc.quantize_lines(x, orc.AXIS_COL, p, line, 1, orc.FMT_E2M3)
        assert np.array_equal(gs[line], s[0]), line
        assert np.array_equal(gc[line], c[0]), line
    import torch
    too_many = torch.empty((rows + 128, cols), dtype=torch.bfloat16, device=dev())
    with pytest.raises(mxq.MxqError) as e:
        mxq.quantize(too_many, row=False, col=True, **kw)
    assert e.value.status == mxq.ERR_SHAPE


def test_largest_column_launch_in_a_batch(orc):
    # the same largest column job batched with a small one: one 1-D launch of
    # 65535 + 1 tiles, the small job's tiles after the large one's
    import torch
    from fp4_microscaling_quantization_amd import mxq
    rows, cols = 65535 * 128, 32
    x = synth.laplace_outlier_entries(rows, cols, seed=45, out_seed=46, frac=1e-4)
    y = synth.normal(128, 96, seed=47)
    kw = dict(grid=mxq.GRID_E1M2, round=mxq.SR, hadamard_n=16, sign_mask=synth.sign_mask(48, 16),
              sr_seed=49)
    ky = dict(kw, round=mxq.RTNE)
    say("largest column launch, batched", rows, cols)
    xt, yt = to_dev_bf16(x), to_dev_bf16(y)
    qx = mxq.empty_qtensor(cols, rows, mxq.FMT_E2M3, xt.device)
    qy = mxq.empty_qtensor(96, 128, mxq.FMT_E2M3, yt.device)
    mxq.quantize_batch([(mxq.qconfig(**kw), xt, None, (qx[0], qx[1], mxq.FMT_E2M3)),
                        (mxq.qconfig(**ky), yt, None, (qy[0], qy[1], mxq.FMT_E2M3))])
    torch.cuda.synchronize()
    gc, gs = host(qx[0]), host(qx[1])
    p = orc.qparams(**kw)
    for line in (0, 17, 31):
        c, s = orc.quantize_lines(x, orc.AXIS_COL, p, line, 1, orc.FMT_E2M3)
        assert np.array_equal(gs[line], s[0]), line
        assert np.array_equal(gc[line], c[0]), line
    c, s = orc.quantize(y, orc.AXIS_COL, orc.qparams(**ky), orc.FMT_E2M3)
    assert np.array_equal(host(qy[1]), s) and np.array_equal(host(qy[0]), c)
