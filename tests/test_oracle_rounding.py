"""CPU pins of the oracle's rounding: RTNE tie table, an exhaustive sweep of
every bf16 magnitude against numpy's round-half-to-even, the exact expectation
of stochastic rounding over all random values, and the closed-form
conditional bias (l_i - r_i)/2 by Monte Carlo."""
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")
GRID_NAMES = {"e2m1": 0, "e1m2": 1, "e2m1max4": 2, "e2m1max3": 3}


def _rows(name):
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            yield line.split()


def test_rtne_tie_table(orc):
    for grid, a, code in _rows("rtne_ties.txt"):
        assert orc.round_rtne(GRID_NAMES[grid], float(a)) == int(code), (grid, a)


def _numpy_rtne(grid: int, a: np.ndarray) -> np.ndarray:
    # piecewise-uniform segments of the grid, each rounded with numpy's
    # round-half-to-even; the segment offsets follow the level tables
    a = a.astype(np.float64)
    if grid == 1:
        return np.minimum(np.round(2 * a), 7).astype(np.int64)
    if grid in (2, 3):
        # E2M1 capped at 4 / 3: nearest of the levels up to the cap, i.e. the
        # E2M1 rounding with every code above the cap brought down to it
        return np.minimum(_numpy_rtne(0, a), 6 if grid == 2 else 5)
    lo = np.round(2 * a)                     # [0, 2): step 0.5, codes 0..4
    mid = np.round(a) + 2                    # [2, 4): step 1, codes 4..6
    hi = np.minimum(np.round(a / 2) + 4, 7)  # [4, inf): step 2, codes 6, 7
    return np.where(a < 2, lo, np.where(a < 4, mid, hi)).astype(np.int64)


@pytest.mark.parametrize("grid", [0, 1, 2, 3])
def test_rtne_exhaustive_bf16_magnitudes(orc, grid):
    # every non-negative finite bf16 value, shifted into the normalized range
    # [0, 2^(emax+1)) by a power of two, as the scale would
    bits = np.arange(0, 0x7F80, dtype=np.uint32)
    vals = (bits << 16).view(np.float32).astype(np.float64)
    top = 8.0 if grid == 0 else 4.0             # 2^(emax+1)
    # fold each value into [0, top) by its own power of two (keeps all
    # mantissa patterns), plus the raw tiny values
    with np.errstate(divide="ignore"):
        k = np.floor(np.log2(np.where(vals > 0, vals, 1.0)))
    folded = np.where(vals > 0, vals / 2.0 ** k * (top / 2), 0.0)
    folded = np.concatenate([folded, vals[vals < top]])
    want = _numpy_rtne(grid, folded)
    got = np.array([orc.round_rtne(grid, float(a)) for a in folded])
    assert np.array_equal(got, want)


@pytest.mark.parametrize("grid", [0, 1, 2, 3])
def test_rtne_invariants(orc, grid):
    T = orc.grid_top(grid)
    lv = np.array(orc.grid_levels(grid))[:T + 1]
    g = np.random.Generator(np.random.PCG64(1))
    a = np.sort(g.uniform(0, 2 * lv[T], 20000))
    m = np.array([orc.round_rtne(grid, x) for x in a])
    assert np.all(np.diff(m) >= 0)                       # monotone
    assert m.max() == T                                  # never above the top code
    inside = a <= lv[T]
    gaps = np.diff(lv)
    # nearest: never more than half the local gap away
    k = np.searchsorted(lv, a[inside], side="right") - 1
    k = np.clip(k, 0, T - 1)
    assert np.all(np.abs(lv[m[inside]] - a[inside]) <= gaps[k] / 2 + 1e-15)
    assert np.all(m[~inside] == T)                       # saturates


def _sr_expect(orc, grid, a, bits):
    lv = orc.grid_levels(grid)
    tot = 0.0
    for r in range(1 << bits):
        tot += lv[orc.round_sr(grid, a, r, bits)]
    return tot / (1 << bits)


@pytest.mark.parametrize("grid", [0, 1, 2, 3])
def test_sr_exact_expectation_all_random_values(orc, grid):
    T = orc.grid_top(grid)
    lv = orc.grid_levels(grid)[:T + 1]
    g = np.random.Generator(np.random.PCG64(7 + grid))
    pts = list(g.uniform(0, lv[T], 6)) + [0.1, 0.3, lv[3], (lv[T - 2] + lv[T - 1]) / 2]
    for a in pts:
        for bits in (8, 16):
            if bits == 16 and a not in pts[:3]:
                continue  # keep the 2^16 enumeration to a few points
            k = max(i for i in range(T + 1) if lv[i] <= a)
            gap = lv[k + 1] - lv[k] if k < T else 0.0
            e = _sr_expect(orc, grid, a, bits)
            # unbiased up to the resolution of B random bits
            assert abs(e - a) <= gap * 2.0 ** -(bits + 1) + 1e-15, (a, bits)


def test_sr_neighbours_only_and_top_clamp(orc):
    for grid in (0, 1, 2, 3):
        T = orc.grid_top(grid)
        lv = orc.grid_levels(grid)[:T + 1]
        g = np.random.Generator(np.random.PCG64(3))
        for a in g.uniform(0, lv[T], 200):
            k = max(i for i in range(T + 1) if lv[i] <= a)
            for r in (0, 1, 777, 32767, 65535):
                m = orc.round_sr(grid, a, r, 16)
                assert m in (k, min(k + 1, T))
        top = 2.0 ** (orc.grid_emax(grid) + 1)
        for a in np.linspace(lv[T], max(top, lv[T] + 1), 9)[:-1]:
            assert all(orc.round_sr(grid, a, r, 16) == T for r in (0, 65535))
        for m in range(T + 1):                   # exact levels stay put
            assert orc.round_sr(grid, lv[m], 0, 16) == m


def test_sr_round_up_count_closed_form(orc):
    # number of r in [0, 2^B) that round up is ceil(p*2^B - 1/2) for the
    # fraction p of the way from level k to level k+1 (uniform grid, step 0.5)
    grid = 1
    for k, p in ((2, 0.3), (0, 0.75), (6, 0.5), (4, 0.01)):
        a = 0.5 * k + 0.5 * p
        for bits in (8, 16):
            ups = sum(orc.round_sr(grid, a, r, bits) == k + 1 for r in range(1 << bits))
            assert ups == int(np.ceil(p * (1 << bits) - 0.5)), (k, p, bits)


def _bias_rows():
    return [(GRID_NAMES[g], int(c), float(lo), float(hi), float(b))
            for g, c, lo, hi, b in _rows("shrinkage_bias.txt")]


@pytest.mark.parametrize("row", _bias_rows(), ids=lambda r: f"g{r[0]}_m{r[1]}")
def test_closed_form_conditional_bias_monte_carlo(orc, row):
    grid, code, lo, hi, bias = row
    lv = orc.grid_levels(grid)
    g = np.random.Generator(np.random.PCG64(100 + 8 * grid + code))
    a = g.uniform(lo, hi, 20000)
    m = np.array([orc.round_rtne(grid, x) for x in a])
    inner = (a > lo) & (a < hi)
    assert np.all(m[inner] == code)          # the bin edges are the tie points
    err = lv[code] - a
    se = err.std() / np.sqrt(a.size)
    assert abs(err.mean() - bias) < 5 * se + 1e-12
    assert bias == (((lv[code] - lo) - (hi - lv[code])) / 2)
