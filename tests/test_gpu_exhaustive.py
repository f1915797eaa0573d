"""Every bf16 bit pattern through the product quantize kernels, byte for byte
against the oracle.

The rounding the product path runs lives inside the fused kernels (rotation,
scale, the folded normalisation and the conversion to codes), so it is swept
there, in every kernel form mxq_quantize and mxq_quantize_batch launch:
  * row-only       (blocks along the contiguous dimension),
  * column-only    (the transpose of the same tensor: identical blocks and
                    block numbers, written transposed),
  * dual           (both outputs from one read, on the tensor and on its
                    transpose),
  * batched        (two column-only jobs in one launch: the mixed RTNE + SR
                    body, and the single-rounding body),
for the four grids, RTNE and stochastic rounding (16-bit draws with two seeds,
8-bit draws), both code formats, and no rotation, H16 and H32.  The inputs
(tests/sweep_inputs.py) pin each block's scale with an anchor on both sides of
the scale codes where the kernels change arithmetic order.

The method: MX blocks of 32 with one E8M0 exponent (htx.com news on MXFP4
pretraining, "Que es MXFP4?"); RTNE onto E2M1 and onto the uniform grid, SR on
the gradient (gist.science summary "Repensando o Vies de Encolhimento ... em
FP4", "Metodologia 1" and "Metodologia 2"); H16 / H32 (gist.science summary
"Pre-treinamento de Modelos de Linguagem Grandes com MXFP4", "Metodologia").
"""
import functools

import numpy as np
import pytest

import oracle_par
import sweep_inputs
from gpuhelp import host, say, to_dev_bf16

pytestmark = pytest.mark.gpu

GRIDS = {"e2m1": 0, "e1m2": 1, "e2m1max4": 2, "e2m1max3": 3}
EMAX = {0: 2, 1: 1, 2: 1, 3: 1}
ROUNDINGS = {
    "rtne": dict(round=0),
    "sr16a": dict(round=1, sr_bits=16, sr_seed=0x5EED0001, sr_stream=3),
    "sr16b": dict(round=1, sr_bits=16, sr_seed=0x123456789, sr_stream=0),
    "sr8": dict(round=1, sr_bits=8, sr_seed=77, sr_stream=1),
}
LAYOUTS = {"hn0": 0, "hn16": 16, "hn32": 32}
SIGNS = {0: 0, 16: 0xB5C3, 32: 0x6D2B79F5}


@functools.lru_cache(maxsize=4)
def _tensors(layout, emax):
    x = sweep_inputs.tensor(layout, emax)
    return x, np.ascontiguousarray(x.T)


def _knobs(grid, rnd, hn):
    return dict(grid=grid, hadamard_n=hn, sign_mask=SIGNS[hn], **ROUNDINGS[rnd])


def _companion(rnd):
    """The other job of a mixed batch: RTNE beside SR, SR beside RTNE."""
    return "sr16b" if rnd == "rtne" else "rtne"


def _eq(got, want, what):
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        raise AssertionError(f"{what}: {len(bad)} bytes differ, first at {bad[:4].tolist()}")


@pytest.mark.parametrize("layout", list(LAYOUTS))
@pytest.mark.parametrize("fmt", [0, 1], ids=["fp4", "e2m3"])
@pytest.mark.parametrize("rnd", list(ROUNDINGS))
@pytest.mark.parametrize("gname", list(GRIDS))
def test_every_bf16_pattern_every_kernel(orc, mxq_lib, gname, rnd, fmt, layout):
    mxq = mxq_lib
    grid, hn = GRIDS[gname], LAYOUTS[layout]
    x, xt = _tensors(layout, EMAX[grid])
    kn = _knobs(grid, rnd, hn)
    p = orc.qparams(**kn)
    say("sweep", gname, rnd, fmt, layout, x.shape)
    # the oracle: blocks of x along rows (R) and along columns (C); the
    # transpose's row blocks are C and its column blocks are R
    R = oracle_par.quantize(orc, x, orc.AXIS_ROW, p, fmt)
    C = oracle_par.quantize(orc, x, orc.AXIS_COL, p, fmt)
    xd, xtd = to_dev_bf16(x), to_dev_bf16(xt)

    q = mxq.quantize(xd, row=True, col=False, row_fmt=fmt, **kn)["row"]
    _eq(host(q[1]), R[1], "row kernel scales")
    _eq(host(q[0]), R[0], "row kernel codes")

    q = mxq.quantize(xtd, row=False, col=True, col_fmt=fmt, **kn)["col"]
    _eq(host(q[1]), R[1], "column kernel scales")
    _eq(host(q[0]), R[0], "column kernel codes")

    # the row kernel on the same blocks as lines of 32 blocks (whole 16-line
    # tiles: the kernel that stages a tile in LDS), into both layouts
    x2 = x.reshape(x.shape[0] // 2, 2 * x.shape[1])
    x2d = to_dev_bf16(x2)
    R4 = oracle_par.quantize(orc, x2, orc.AXIS_ROW, p, fmt)
    q = mxq.quantize(x2d, row=True, col=False, row_fmt=fmt, **kn)["row"]
    _eq(host(q[1]), R4[1], "row kernel (32-block lines) scales")
    _eq(host(q[0]), R4[0], "row kernel (32-block lines) codes")
    tc, ts = orc.to_mfma_layout(R4[0], R4[1], fmt, fill=0xA5)
    q = mxq.quantize(x2d, row=True, col=False, row_fmt=fmt,
                     row_layout=mxq.LAYOUT_MFMA, fill=0xA5, **kn)["row"]
    _eq(host(q[1]), ts, "row kernel (matrix-core layout) scales")
    _eq(host(q[0]), tc, "row kernel (matrix-core layout) codes")

    for name, t, want_row in (("x", xd, R), ("xT", xtd, C)):
        q = mxq.quantize(t, row=True, col=True, row_fmt=fmt, col_fmt=1 - fmt, **kn)
        _eq(host(q["row"][1]), want_row[1], f"dual({name}) row scales")
        _eq(host(q["row"][0]), want_row[0], f"dual({name}) row codes")
        # the column half in the other code format (the oracle's bytes of it)
        oc = oracle_par.quantize(orc, x if name == "x" else xt, orc.AXIS_COL, p, 1 - fmt)
        _eq(host(q["col"][1]), oc[1], f"dual({name}) column scales")
        _eq(host(q["col"][0]), oc[0], f"dual({name}) column codes")

    # batched: this config beside its companion rounding (mixed body), and
    # beside itself with another seed (single-rounding body)
    other = _companion(rnd)
    kn2 = _knobs(grid, other, hn)
    R2 = oracle_par.quantize(orc, x, orc.AXIS_ROW, orc.qparams(**kn2), fmt)
    kn3 = dict(kn, sr_seed=kn.get("sr_seed", 0) + 1, sr_stream=7)
    R3 = R if rnd == "rtne" else oracle_par.quantize(orc, x, orc.AXIS_ROW, orc.qparams(**kn3), fmt)
    lines, k = xt.shape[1], xt.shape[0]
    for tag, jobs in (("mixed", [(kn, R), (kn2, R2)]), ("single", [(kn, R), (kn3, R3)])):
        outs = [mxq.empty_qtensor(lines, k, fmt, xtd.device) for _ in jobs]
        mxq.quantize_batch([(mxq.qconfig(**kj), xtd, None, (o[0], o[1], fmt))
                            for (kj, _), o in zip(jobs, outs)])
        for i, ((_, want), o) in enumerate(zip(jobs, outs)):
            _eq(host(o[1]), want[1], f"batch {tag} job {i} scales")
            _eq(host(o[0]), want[0], f"batch {tag} job {i} codes")


@pytest.mark.parametrize("bits", [8, 16])
@pytest.mark.parametrize("gname", ["e2m1", "e1m2"])
def test_sr_threshold_equalities(orc, mxq_lib, gname, bits):
    """Stochastic rounding exactly at its threshold: r + 1/2 = p 2^B rounds
    down.  In the bin [0, 0.5) (the only bin where bf16 holds such values) an
    element with draw r is given the magnitude (2r + 1) 2^-(B+2) when that
    has at most 8 significant bits; the block's anchor fixes its scale at
    2^0.  Every kernel form must reproduce the oracle byte for byte."""
    mxq = mxq_lib
    grid = GRIDS[gname]
    emax = EMAX[grid]
    seed, stream = 0xC0FFEE + bits, 5
    nbk, lines = 16, 512
    g = np.random.Generator(np.random.PCG64(bits + 10 * grid))
    x = np.zeros((lines, nbk * 32), np.uint16)
    filler = g.integers(0x3A00, 0x3F00, size=x.shape, dtype=np.uint16)   # magnitudes 2^-11 .. 0.5
    ties = 0
    for line in range(lines):
        for jb in range(nbk):
            b = line * nbk + jb
            for j in range(32):
                if j == 31 - (b % 2) * 31:
                    x[line, jb * 32 + j] = (127 + emax) << 7 | ((b // 2) % 2) << 15   # +-2^emax
                    continue
                r = orc.sr_random(seed, stream, b, j, bits)
                sgn = (j % 2) << 15
                if 2 * r + 1 < 256:
                    v = np.float32((2 * r + 1) * 2.0 ** -(bits + 2))
                    x[line, jb * 32 + j] = (int(v.view(np.uint32)) >> 16) | sgn
                    ties += 1
                else:
                    x[line, jb * 32 + j] = filler[line, jb * 32 + j] | sgn
    assert ties > (200 if bits == 16 else 50000)
    kn = dict(grid=grid, round=1, sr_bits=bits, sr_seed=seed, sr_stream=stream)
    p = orc.qparams(**kn)
    xt = np.ascontiguousarray(x.T)
    say("sr ties", gname, bits, ties)
    for fmt in (0, 1):
        R = oracle_par.quantize(orc, x, orc.AXIS_ROW, p, fmt)
        assert np.all(R[1][R[1] != 0] == 127)          # every block at scale 2^0
        q = mxq.quantize(to_dev_bf16(x), row=True, row_fmt=fmt, **kn)["row"]
        _eq(host(q[0]), R[0], "row codes")
        q = mxq.quantize(to_dev_bf16(xt), row=False, col=True, col_fmt=fmt, **kn)["col"]
        _eq(host(q[0]), R[0], "column codes")
        q = mxq.quantize(to_dev_bf16(xt), row=True, col=True, row_fmt=1 - fmt, col_fmt=fmt, **kn)
        _eq(host(q["col"][0]), R[0], "dual column codes")
        o = mxq.empty_qtensor(lines, nbk * 32, fmt, q["col"][0].device)
        mxq.quantize_batch([(mxq.qconfig(**kn), to_dev_bf16(xt), None, (o[0], o[1], fmt))])
        _eq(host(o[0]), R[0], "batched column codes")
