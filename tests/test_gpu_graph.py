"""The weight-gradient step under HIP graph capture: the batched column-wise
quantize of dY (stochastic rounding) and X (RTNE) into the matrix-core layout,
then the block-scaled GEMM, captured once into a graph and replayed several
times, each replay after eager work that scrambles every output, must give the
eager result byte for byte (codes, scales and the fp32 product).  The library
issues no memset and allocates nothing on these paths, so the captured graph
holds only its kernels.  Both operand forms are covered: FP6 (E2M3) codes take
the three-slot ring GEMM, FP4 codes with K a multiple of 512 the read-ahead
one.  A second test captures the layer's other operand preparation (the
staged row kernel, the dual kernel) and the Fprop and Dgrad products."""
import numpy as np
import pytest

from fp4_microscaling_quantization_amd import synth
from gpuhelp import dev, host, say, to_dev_bf16

pytestmark = pytest.mark.gpu


def _inputs(t, cols, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return synth.f32_to_bf16_bits(g.standard_normal((t, cols)).astype(np.float32))


@pytest.mark.parametrize("variant", ["e1m2_e2m3", "e2m1_fp4"])
def test_wgrad_step_graph_replays_match_eager(variant):
    import torch
    from fp4_microscaling_quantization_amd import mxq
    t, n_dy, n_x = 2048, 512, 768
    grid, fmt = (mxq.GRID_E1M2, mxq.FMT_E2M3) if variant == "e1m2_e2m3" else (mxq.GRID_E2M1, mxq.FMT_FP4)
    say("graph wgrad step", variant, (t, n_dy, n_x))
    signs = synth.sign_mask(41, 16)
    dy = to_dev_bf16(_inputs(t, n_dy, 1))
    x = to_dev_bf16(_inputs(t, n_x, 2))
    cd = mxq.qconfig(grid=grid, round=mxq.SR, hadamard_n=16, sign_mask=signs, sr_seed=77)
    cx = mxq.qconfig(grid=grid, round=mxq.RTNE, hadamard_n=16, sign_mask=signs)
    qd = mxq.empty_qtensor(n_dy, t, fmt, dev(), mxq.LAYOUT_MFMA)
    qx = mxq.empty_qtensor(n_x, t, fmt, dev(), mxq.LAYOUT_MFMA)
    c = torch.empty((n_dy, n_x), dtype=torch.float32, device=dev())
    jobs = [(cd, dy, None, (*qd, fmt, mxq.LAYOUT_MFMA)), (cx, x, None, (*qx, fmt, mxq.LAYOUT_MFMA))]

    def step():
        mxq.quantize_batch(jobs)
        mxq.wgrad_gemm(qd[0], qd[1], fmt, grid, qx[0], qx[1], fmt, grid, out=c,
                       layout=mxq.LAYOUT_MFMA, m=n_dy, n=n_x, k=t)

    outs = [qd[0], qd[1], qx[0], qx[1], c]
    step()
    ref = [host(o).copy() for o in outs]
    assert np.isfinite(ref[4]).all()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                 # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    junk = torch.randn(512, 512, device=dev())
    for r in range(3):
        for o in outs[:4]:
            o.fill_(0x5A + r)
        c.fill_(float("nan"))
        _ = (junk @ junk).sum().item()         # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for got, want, name in zip(outs, ref, ["dY codes", "dY scales", "X codes", "X scales", "dW"]):
            assert np.array_equal(host(got).view(np.uint8), want.view(np.uint8)), (r, name)


@pytest.mark.parametrize("layout", ["mfma", "rows"])
def test_layer_operands_graph_replays_match_eager(layout):
    """The Fprop / Dgrad operand preparation under capture: X and dY quantized
    row-wise (whole 16-line tiles of 32 blocks: the kernel that stages each
    tile in LDS) and W quantized both ways from one read (the dual kernel, full
    tiles staging their row half in LDS), then, in the matrix-core layout, the
    Fprop and Dgrad products.  Three replays after scrambling every output
    must give the eager bytes."""
    import torch
    from fp4_microscaling_quantization_amd import mxq
    t, k, n = 256, 1024, 2048
    lay = mxq.LAYOUT_MFMA if layout == "mfma" else mxq.LAYOUT_ROWS
    grid, fmt = mxq.GRID_E2M1, mxq.FMT_FP4
    say("graph layer operands", layout, (t, k, n))
    signs = synth.sign_mask(43, 32)
    x = to_dev_bf16(_inputs(t, k, 3))
    w = to_dev_bf16(_inputs(n, k, 4))
    dy = to_dev_bf16(_inputs(t, n, 5))
    cw = mxq.qconfig(grid=grid, round=mxq.RTNE, hadamard_n=32, sign_mask=signs)
    cd = mxq.qconfig(grid=grid, round=mxq.SR, hadamard_n=32, sign_mask=signs, sr_seed=19)
    qx = mxq.empty_qtensor(t, k, fmt, dev(), lay)
    qwr = mxq.empty_qtensor(n, k, fmt, dev(), lay)
    qwc = mxq.empty_qtensor(k, n, fmt, dev(), lay)
    qd = mxq.empty_qtensor(t, n, fmt, dev(), lay)
    y = torch.empty((t, n), dtype=torch.float32, device=dev())
    dx = torch.empty((t, k), dtype=torch.float32, device=dev())

    def step():
        mxq.quantize_into(cw, x, row=(*qx, fmt, lay))
        mxq.quantize_into(cw, w, row=(*qwr, fmt, lay), col=(*qwc, fmt, lay))
        mxq.quantize_into(cd, dy, row=(*qd, fmt, lay))
        if lay == mxq.LAYOUT_MFMA:
            mxq.gemm_abt(qx[0], qx[1], fmt, grid, qwr[0], qwr[1], fmt, grid, out=y,
                         layout=lay, m=t, n=n, k=k)
            mxq.gemm_abt(qd[0], qd[1], fmt, grid, qwc[0], qwc[1], fmt, grid, out=dx,
                         layout=lay, m=t, n=k, k=n)

    qouts = [*qx, *qwr, *qwc, *qd]
    outs = qouts + ([y, dx] if lay == mxq.LAYOUT_MFMA else [])
    step()
    ref = [host(o).copy() for o in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    junk = torch.randn(512, 512, device=dev())
    for r in range(3):
        for o in qouts:
            o.fill_(0x3C + r)
        for o in outs[len(qouts):]:
            o.fill_(float("nan"))
        _ = (junk @ junk).sum().item()
        g.replay()
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip(outs, ref)):
            assert np.array_equal(host(got).view(np.uint8), want.view(np.uint8)), (r, i)
