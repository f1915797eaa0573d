"""GPU parity of the rounding step (mxq_round_to_grid) against the oracle.

RTNE: every non-negative fp32 value below 2^(emax+1) (about 1.1e9 inputs) and
their negatives go through the GPU.  The GPU codes must be non-decreasing in
the magnitude; a non-decreasing step function is fixed by its values on both
sides of each step, and the oracle (nearest level, ties to even: monotone by
construction) is checked at exactly those points.  Together this proves the
two agree on every input.

SR: random (value, random bits) pairs against the oracle one by one."""
import numpy as np
import pytest

from gpuhelp import dev, say

pytestmark = pytest.mark.gpu

CHUNK = 1 << 27


GRIDS = [0, 1, 2, 3]
GRID_IDS = ["e2m1", "e1m2", "e2m1max4", "e2m1max3"]


@pytest.mark.parametrize("grid", GRIDS, ids=GRID_IDS)
def test_rtne_every_fp32_magnitude(orc, grid):
    import torch
    from fp4_microscaling_quantization_amd import mxq
    d = dev()
    top_bits = 0x41000000 if grid == 0 else 0x40800000      # 8.0 / 4.0
    T = orc.grid_top(grid)
    change = []            # (bits_before, bits_after, code_before, code_after)
    prev_last = None
    for start in range(0, top_bits, CHUNK):
        end = min(start + CHUNK, top_bits)
        say("rtne sweep", grid, hex(start))
        a = torch.arange(start, end, dtype=torch.int32, device=d).view(torch.float32)
        codes = mxq.round_to_grid(a, grid, mxq.RTNE)
        neg = mxq.round_to_grid(-a, grid, mxq.RTNE)
        # the sign bit is the only difference for negated inputs
        assert torch.equal(neg, codes | 8), "sign handling"
        assert bool((codes <= T).all())
        dif = codes[1:].to(torch.int16) - codes[:-1].to(torch.int16)
        assert bool((dif >= 0).all()), "not monotone"
        idx = torch.nonzero(dif).flatten().cpu().numpy()
        c = codes.cpu().numpy() if idx.size else None
        for i in idx:
            change.append((start + int(i), start + int(i) + 1, int(c[i]), int(c[i + 1])))
        first = int(codes[0].item())
        if prev_last is not None and first != prev_last:
            assert first > prev_last
            change.append((start - 1, start, prev_last, first))
        prev_last = int(codes[-1].item())
        del a, codes, neg, dif
    # the step points, and the values at the two ends
    assert len(change) == T, change
    f = lambda b: float(np.array([b], np.uint32).view(np.float32)[0])
    for b0, b1, c0, c1 in change:
        assert orc.round_rtne(grid, f(b0)) == c0, (hex(b0), c0)
        assert orc.round_rtne(grid, f(b1)) == c1, (hex(b1), c1)
    assert orc.round_rtne(grid, 0.0) == 0
    assert orc.round_rtne(grid, f(top_bits - 1)) == prev_last == T
    # beyond the range the scale allows: saturation
    big = torch.tensor([f(top_bits), 100.0, 3e38, float("inf")], device=d)
    assert (mxq.round_to_grid(big, grid, mxq.RTNE).cpu().numpy() == T).all()


@pytest.mark.parametrize("grid", GRIDS, ids=GRID_IDS)
@pytest.mark.parametrize("bits", [16, 8])
def test_sr_random_pairs(orc, grid, bits):
    import torch
    from fp4_microscaling_quantization_amd import mxq
    top = 8.0 if grid == 0 else 4.0
    g = np.random.Generator(np.random.PCG64(31 + grid + bits))
    n = 1 << 16
    a = g.uniform(0, top, n).astype(np.float32)
    # include exact levels, midpoints and values next to levels
    lv = np.array(orc.grid_levels(grid)[:orc.grid_top(grid) + 1], np.float32)
    edge = np.concatenate([lv, (lv[1:] + lv[:-1]) / 2, np.nextafter(lv, np.float32(0)),
                           np.nextafter(lv, np.float32(10))]).astype(np.float32)
    a[:edge.size] = edge
    sign = np.where(g.random(n) < 0.5, -1, 1).astype(np.float32)
    r = g.integers(0, 1 << bits, n).astype(np.uint16)
    say("sr pairs", grid, bits)
    got = mxq.round_to_grid(torch.from_numpy(sign * a).to(dev()), grid, mxq.SR,
                            rand=torch.from_numpy(r.view(np.int16)).to(dev()), sr_bits=bits)
    got = got.cpu().numpy()
    want = np.array([orc.round_sr(grid, float(v), int(ri), bits) for v, ri in zip(a, r)])
    want |= np.where(sign < 0, 8, 0)
    assert np.array_equal(got, want)
