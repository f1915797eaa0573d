"""The other two GEMMs of a linear layer through mxq_gemm_abt, at the shapes
of an 8B-model MLP up-projection (8192 tokens, K = 4096, N = 14336), with the
operands quantized by the GPU straight into the matrix-core layout:

  Fprop  Y  = X W^T : X row-wise, W row-wise (both rotated along K);
  Dgrad  dX = dY W  : dY row-wise, W column-wise (both rotated along N).

W's two operands come from one dual-output quantize call, which rotates each
direction with the same knobs.  Every operand byte is checked against the
oracle, and three 256-row bands of each output (every column) against the
fp64 product of the oracle's dequantized operands: per element within the
fp32 accumulation bound, and relative Frobenius error <= 1e-6."""
import numpy as np
import pytest

from fp4_microscaling_quantization_amd import synth
from gpuhelp import check_product, say, to_dev_bf16

pytestmark = pytest.mark.gpu

T, K, N = 8192, 4096, 14336
VARIANTS = {"e1m2_e2m3": (1, 1), "e2m1_fp4": (0, 0)}   # (grid, fmt)


BANDS = (0, 4000, T - 256)      # first rows of the checked 256-row output bands


def _band_check(orc, c, a_lines, B, k, what):
    """Rows of C in BANDS against the fp64 product of the oracle's dequantized
    operands: a_lines(r0, n) gives A's dequantized rows r0 .. r0 + n - 1, B
    is the whole dequantized B.  Every output of each band is checked (every
    column of C), with the per-element bound of gpuhelp.check_product."""
    import oracle_par
    absB = np.abs(B)
    for r0 in BANDS:
        A = a_lines(r0, 256)
        ref = oracle_par.gemm_abt_f64(orc, A, B)
        absref = oracle_par.gemm_abt_f64(orc, np.abs(A), absB)
        got = c[r0:r0 + 256].cpu().numpy().astype(np.float64)
        say(what, "band", r0, "rel. Frobenius error", check_product(got, ref, absref, k, (what, r0)))


def _whole_operand(orc, q, x, axis, p, fmt, name):
    """Every byte of a matrix-core-layout operand against the oracle; returns
    the oracle's dequantized operand."""
    import oracle_par
    oc, os_ = oracle_par.quantize(orc, x, axis, p, fmt)
    tc, ts = orc.to_mfma_layout(oc, os_, fmt)
    assert np.array_equal(q[1].cpu().numpy(), ts), (name, "scales")
    assert np.array_equal(q[0].cpu().numpy(), tc), (name, "codes")
    return oracle_par.dequantize(orc, oc, os_, p.grid, fmt)


@pytest.fixture(scope="module")
def weight():
    return synth.w_14336x4096()


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_fprop_full_size(orc, weight, variant):
    import torch
    from fp4_microscaling_quantization_amd import mxq
    grid, fmt = VARIANTS[variant]
    x = synth.x_8192x4096()
    kn = dict(grid=grid, round=0, hadamard_n=32, sign_mask=synth.sign_mask(synth.SIGNS_W, 32))
    say("fprop", variant)
    qx = mxq.quantize(to_dev_bf16(x), row=True, col=False, row_fmt=fmt,
                      row_layout=mxq.LAYOUT_MFMA, **kn)["row"]
    qw = mxq.quantize(to_dev_bf16(weight), row=True, col=True, row_fmt=fmt, col_fmt=fmt,
                      row_layout=mxq.LAYOUT_MFMA, col_layout=mxq.LAYOUT_MFMA, **kn)
    y = mxq.gemm_abt(qx[0], qx[1], fmt, grid, qw["row"][0], qw["row"][1], fmt, grid,
                     layout=mxq.LAYOUT_MFMA, m=T, n=N, k=K)
    torch.cuda.synchronize()
    p = orc.qparams(**kn)
    _whole_operand(orc, qx, x, orc.AXIS_ROW, p, fmt, "X row-wise")
    _whole_operand(orc, qw["col"], weight, orc.AXIS_COL, p, fmt, "W column-wise")
    B = _whole_operand(orc, qw["row"], weight, orc.AXIS_ROW, p, fmt, "W row-wise")
    la = lambda r0, n: orc.dequantize(*orc.quantize_lines(x, orc.AXIS_ROW, p, r0, n, fmt), grid, fmt)
    _band_check(orc, y, la, B, K, "fprop")


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_dgrad_full_size(orc, weight, variant):
    import torch
    from fp4_microscaling_quantization_amd import mxq
    grid, fmt = VARIANTS[variant]
    dy = synth.dy_8192x14336()
    signs = synth.sign_mask(synth.SIGNS_W, 32)
    kw = dict(grid=grid, round=0, hadamard_n=32, sign_mask=signs)
    kd = dict(grid=grid, round=1, hadamard_n=32, sign_mask=signs, sr_seed=11)   # SR on the gradient
    say("dgrad", variant)
    qd = mxq.quantize(to_dev_bf16(dy), row=True, col=False, row_fmt=fmt,
                      row_layout=mxq.LAYOUT_MFMA, **kd)["row"]
    qw = mxq.quantize(to_dev_bf16(weight), row=True, col=True, row_fmt=fmt, col_fmt=fmt,
                      row_layout=mxq.LAYOUT_MFMA, col_layout=mxq.LAYOUT_MFMA, **kw)
    dx = mxq.gemm_abt(qd[0], qd[1], fmt, grid, qw["col"][0], qw["col"][1], fmt, grid,
                      layout=mxq.LAYOUT_MFMA, m=T, n=K, k=N)
    torch.cuda.synchronize()
    pd, pw = orc.qparams(**kd), orc.qparams(**kw)
    _whole_operand(orc, qd, dy, orc.AXIS_ROW, pd, fmt, "dY row-wise")
    B = _whole_operand(orc, qw["col"], weight, orc.AXIS_COL, pw, fmt, "W column-wise")
    la = lambda r0, n: orc.dequantize(*orc.quantize_lines(dy, orc.AXIS_ROW, pd, r0, n, fmt), grid, fmt)
    _band_check(orc, dx, la, B, N, "dgrad")


def test_gemm_abt_is_the_wgrad_product():
    """The general entry point and the weight-gradient one are the same call."""
    import torch
    from fp4_microscaling_quantization_amd import mxq
    x = synth.normal(512, 384, seed=41)
    q = mxq.quantize(to_dev_bf16(x), grid=1, row=False, col=True, col_fmt=1,
                     col_layout=mxq.LAYOUT_MFMA)["col"]
    a = mxq.gemm_abt(q[0], q[1], 1, 1, q[0], q[1], 1, 1, layout=mxq.LAYOUT_MFMA, m=384, n=384, k=512)
    b = mxq.wgrad_gemm(q[0], q[1], 1, 1, q[0], q[1], 1, 1, layout=mxq.LAYOUT_MFMA, m=384, n=384, k=512)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("sign_mode", [0, 1], ids=["mask", "per-block"])
def test_rotation_cancels_in_the_gpu_product(orc, sign_mode):
    # Fprop with both operands rotated along K by the same signs: the GPU
    # product matches the oracle pipeline and approximates the unrotated fp64
    # X W^T to within quantization noise; with W's signs drawn from another
    # seed the rotation no longer cancels and the result is noise
    import torch
    from fp4_microscaling_quantization_amd import mxq
    m, n, k = 512, 768, 1024
    x = synth.normal(m, k, seed=51)
    w = synth.normal(n, k, seed=52, std=0.02)
    kn = dict(grid=1, round=0, hadamard_n=32, sign_mask=synth.sign_mask(53, 32),
              sign_mode=sign_mode, sign_seed=54)
    say("cancel", sign_mode)

    def fprop(kx, kw):
        qx = mxq.quantize(to_dev_bf16(x), row=True, row_fmt=1, row_layout=mxq.LAYOUT_MFMA, **kx)["row"]
        qw = mxq.quantize(to_dev_bf16(w), row=True, row_fmt=1, row_layout=mxq.LAYOUT_MFMA, **kw)["row"]
        y = mxq.gemm_abt(qx[0], qx[1], 1, 1, qw[0], qw[1], 1, 1, layout=mxq.LAYOUT_MFMA, m=m, n=n, k=k)
        torch.cuda.synchronize()
        return y.cpu().numpy().astype(np.float64)

    y = fprop(kn, kn)
    p = orc.qparams(**kn)
    A = orc.dequantize(*orc.quantize(x, orc.AXIS_ROW, p, 1), 1, 1)
    B = orc.dequantize(*orc.quantize(w, orc.AXIS_ROW, p, 1), 1, 1)
    ref = orc.gemm_abt_f64(A, B)
    assert np.linalg.norm(y - ref) <= 1e-6 * np.linalg.norm(ref)
    exact = synth.bf16_bits_to_f32(x).astype(np.float64) @ synth.bf16_bits_to_f32(w).astype(np.float64).T
    sqnr = lambda v: 10 * np.log10(np.sum(exact ** 2) / np.sum((v - exact) ** 2))
    assert sqnr(y) > 12.0, sqnr(y)
    other = dict(kn, sign_mask=synth.sign_mask(55, 32), sign_seed=56)
    assert sqnr(fprop(kn, other)) < 1.0
