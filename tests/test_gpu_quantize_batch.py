"""GPU parity of mxq_quantize_batch: every job's codes and scales bit-exact
against the CPU oracle, for batches that share one launch (column-only jobs
with the same grid family, rotation size and code format, each with its own
rounding, seeds, signs, shape and layout), batches split over several
launches (other kernels, more than 8 jobs, empty jobs), and, at the full
size of the weight-gradient step, the dY (SR) + X (RTNE) pair the benchmark
times, which must equal two mxq_quantize calls byte for byte."""
import numpy as np
import pytest

from fp4_microscaling_quantization_amd import synth
from gpuhelp import host, say, to_dev_bf16

pytestmark = pytest.mark.gpu


class Job:
    """One tensor of a batch: bf16 bits x, knobs, and which outputs (fmt,
    layout) it asks for; ld pads x's rows on the device."""

    def __init__(self, x, knobs, row=None, col=None, ld=None):
        self.x, self.knobs, self.row, self.col, self.ld = x, knobs, row, col, ld

    def device_input(self):
        rows, cols = self.x.shape
        if rows == 0:
            # a real (non-NULL) address with no rows
            return to_dev_bf16(np.zeros((1, cols), np.uint16))[:0]
        if self.ld is None:
            return to_dev_bf16(self.x)
        wide = np.zeros((rows, self.ld), np.uint16)
        wide[:, :cols] = self.x
        return to_dev_bf16(wide)[:, :cols]


def _knobs(grid, rnd, n, seed, sign_mode=0):
    return dict(grid=grid, round=rnd, hadamard_n=n,
                sign_mask=synth.sign_mask(200 + seed, n) if n else 0,
                sr_seed=0xBA7C0000 + seed, sr_stream=seed, sr_bits=16, sign_mode=sign_mode,
                sign_seed=0x5151 + seed)


def _run_batch(jobs):
    """Launch the batch; returns, per job, {'row': (codes, scales), 'col': ...}."""
    from fp4_microscaling_quantization_amd import mxq
    import torch
    args, outs, keep = [], [], []
    for j in jobs:
        xt = j.device_input()
        rows, cols = j.x.shape

        def buffers(lines, k, fmt, lay):
            if lines * k == 0:
                # nothing is written; the pointers only have to be valid
                return (torch.empty(16, dtype=torch.uint8, device=xt.device),
                        torch.empty(16, dtype=torch.uint8, device=xt.device))
            return mxq.empty_qtensor(lines, k, fmt, xt.device, lay, fill=0xA5)
        o, r, c = {}, None, None
        if j.row:
            fmt, lay = j.row
            rc, rs = buffers(rows, cols, fmt, lay)
            r, o["row"] = (rc, rs, fmt, lay), (rc, rs)
        if j.col:
            fmt, lay = j.col
            cc, cs = buffers(cols, rows, fmt, lay)
            c, o["col"] = (cc, cs, fmt, lay), (cc, cs)
        args.append((mxq.qconfig(**j.knobs), xt, r, c))
        outs.append(o)
        keep.append(xt)
    mxq.quantize_batch(args)
    return outs


def _check_job(orc, j, out, tag):
    p = orc.qparams(**j.knobs)
    for axis, key, spec in ((orc.AXIS_ROW, "row", j.row), (orc.AXIS_COL, "col", j.col)):
        if not spec:
            continue
        fmt, lay = spec
        c, s = orc.quantize(j.x, axis, p, fmt)
        if lay == 1:
            c, s = orc.to_mfma_layout(c, s, fmt, fill=0xA5)
        gc, gs = host(out[key][0]), host(out[key][1])
        assert np.array_equal(gs, s), (tag, key, "scales")
        assert np.array_equal(gc, c), (tag, key, "codes", np.argwhere(gc != c)[:5])


def _col_jobs(grid_family, n, fmt, count, seed0, rnd=None):
    """`count` column-only jobs of one kernel: ragged shapes, both roundings
    (or only `rnd`), both sign modes, both layouts where the shape allows the
    MFMA one."""
    shapes = [(256, 100), (160, 72), (96, 130), (128, 256), (32, 8), (384, 40), (64, 129),
              (512, 16), (224, 200)]
    grids = [0, 2, 3] if grid_family == 0 else [1]
    jobs = []
    for i in range(count):
        rows, cols = shapes[i % len(shapes)]
        x = synth.laplace_outlier_entries(rows, cols, seed=seed0 + i, out_seed=i, frac=0.01)
        knobs = _knobs(grids[i % len(grids)], i % 2 if rnd is None else rnd, n, seed0 + i,
                       sign_mode=(i // 2) % 2)
        lay = 1 if rows % 128 == 0 and i % 3 != 2 else 0
        jobs.append(Job(x, knobs, col=(fmt, lay)))
    return jobs


@pytest.mark.parametrize("family,n,fmt", [(1, 16, 1), (1, 32, 0), (0, 16, 0), (0, 0, 1),
                                          (0, 32, 1), (1, 0, 0)])
def test_one_launch_batch_parity(orc, family, n, fmt):
    jobs = _col_jobs(family, n, fmt, 5, seed0=10 * n + fmt + family)
    say("batch one launch", family, n, fmt, [j.x.shape for j in jobs])
    outs = _run_batch(jobs)
    for i, (j, o) in enumerate(zip(jobs, outs)):
        _check_job(orc, j, o, f"job {i}")


@pytest.mark.parametrize("rnd", [0, 1], ids=["rtne", "sr"])
@pytest.mark.parametrize("family,n,fmt", [(1, 16, 1), (0, 32, 0)])
def test_one_rounding_batch_parity(orc, family, n, fmt, rnd):
    # every job rounds the same way: the launch takes the one-body kernel
    jobs = _col_jobs(family, n, fmt, 4, seed0=40 + rnd, rnd=rnd)
    say("batch one rounding", family, n, fmt, rnd)
    outs = _run_batch(jobs)
    for i, (j, o) in enumerate(zip(jobs, outs)):
        _check_job(orc, j, o, f"job {i}")


def test_mixed_batch_parity(orc):
    """Column runs of different kernels, row-only, dual, empty and padded jobs,
    and a run of 9 same-kernel jobs (two launches of at most 8)."""
    jobs = _col_jobs(1, 16, 1, 2, seed0=1)
    jobs.append(Job(synth.normal(33, 4128, seed=3), _knobs(1, 0, 32, 3), row=(0, 0)))
    jobs += _col_jobs(0, 16, 0, 2, seed0=5)
    jobs.append(Job(synth.normal(256, 288, seed=4, std=0.02), _knobs(0, 1, 16, 4),
                    row=(1, 0), col=(0, 1)))
    jobs.append(Job(np.zeros((0, 64), np.uint16), _knobs(1, 1, 16, 6), col=(1, 0)))
    jobs.append(Job(synth.normal(64, 96, seed=5), _knobs(0, 0, 16, 7), col=(0, 0), ld=136))
    jobs += _col_jobs(1, 32, 0, 9, seed0=20)
    say("batch mixed", len(jobs))
    outs = _run_batch(jobs)
    for i, (j, o) in enumerate(zip(jobs, outs)):
        if j.x.shape[0] == 0:
            continue
        _check_job(orc, j, o, f"job {i}")


def _mfma_tile(codes, scales, t, lines, k, fmt):
    """Bytes of 16-line tile t of an MFMA-layout tensor [lines x k], as the
    layout of a 16-line tensor: codes [steps][64 lanes][bb], scales [groups][64][4]."""
    bb = 16 if fmt == 0 else 24
    ntiles, steps = (lines + 15) // 16, k // 128
    c = codes.reshape(steps, ntiles, 64 * bb)[:, t, :].reshape(-1)
    s = scales.reshape((steps + 3) // 4, ntiles, 256)[:, t, :].reshape(-1)
    return c, s


def test_wgrad_pair_full_size(orc):
    """The weight-gradient step's two operands in one launch, as the benchmark
    runs them: byte-equal to two mxq_quantize calls, and every byte of both
    outputs equal to the oracle's (in the matrix-core layout, placed by the
    oracle's layout map), in both layouts."""
    import oracle_par
    from fp4_microscaling_quantization_amd import mxq
    import torch
    cases = [c for c in synth.workload_cases() if c.name.startswith("wgrad_") and c.sr_bits == 16]
    assert [c.round for c in cases] == [mxq.SR, mxq.RTNE]
    say("batch wgrad pair", [c.name for c in cases])
    hx = [c.make() for c in cases]
    xs = [to_dev_bf16(h) for h in hx]
    want = [oracle_par.quantize(orc, x, orc.AXIS_COL, orc.qparams(**c.knobs()), c.fmt)
            for c, x in zip(cases, hx)]
    for lay in (mxq.LAYOUT_MFMA, mxq.LAYOUT_ROWS):
        batch, single = [], []
        for c, xt in zip(cases, xs):
            rows, cols = xt.shape
            bc, bs = mxq.empty_qtensor(cols, rows, c.fmt, xt.device, lay, fill=0)
            sc, ss = mxq.empty_qtensor(cols, rows, c.fmt, xt.device, lay, fill=0)
            cfg = mxq.qconfig(**c.knobs())
            batch.append((cfg, xt, None, (bc, bs, c.fmt, lay)))
            single.append((cfg, xt, (sc, ss, c.fmt, lay)))
        mxq.quantize_batch(batch)
        for cfg, xt, out in single:
            mxq.quantize_into(cfg, xt, None, out)
        torch.cuda.synchronize()
        for (_, _, _, b), (_, _, s) in zip(batch, single):
            assert torch.equal(b[0], s[0]) and torch.equal(b[1], s[1]), lay
        for c, (oc, os_), (_, _, _, b) in zip(cases, want, batch):
            if lay == mxq.LAYOUT_MFMA:
                oc, os_ = orc.to_mfma_layout(oc, os_, c.fmt)
            assert np.array_equal(host(b[1]), os_), (c.name, lay, "scales")
            assert np.array_equal(host(b[0]), oc), (c.name, lay, "codes")
