"""Shared helpers of the GPU parity tests (not a test module)."""
import sys

import numpy as np

from fp4_microscaling_quantization_amd import synth


def say(*args):
    """Name the case about to run on the GPU (flushed, so a crash still shows it)."""
    print("[gpu-case]", *args, flush=True)
    sys.stdout.flush()


def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    return torch.device("cuda:0")


def to_dev_bf16(xbits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(xbits).view(np.int16)).to(dev()).view(torch.bfloat16)


def host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def special_matrix(rows: int, cols: int, seed: int) -> np.ndarray:
    """bf16 bits with whole blocks (along both axes) of special values."""
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal((rows, cols)).astype(np.float32)
    bits = synth.f32_to_bf16_bits(x)
    flat = bits.reshape(-1)
    n = flat.size
    pick = lambda k: g.choice(n, size=min(k, n), replace=False)
    flat[pick(n // 50)] = 0x0000                      # +0
    flat[pick(n // 50)] = 0x8000                      # -0
    flat[pick(n // 100)] = g.integers(1, 0x80, n // 100 if n >= 100 else 1, dtype=np.uint16)  # subnormal
    flat[pick(max(n // 400, 1))] = 0x7F80             # +inf
    flat[pick(max(n // 400, 1))] = 0xFF80             # -inf
    flat[pick(max(n // 400, 1))] = 0x7FC1             # nan
    flat[pick(n // 200)] = 0x7F7F                     # bf16 max (FWHT may overflow to inf)
    # whole zero rows / columns / tiny rows
    if rows > 3:
        bits[1, :] = 0
        bits[2, :] = (g.integers(1, 0x7F, cols) | (g.integers(0, 2, cols) << 15)).astype(np.uint16)
    if cols > 5:
        bits[:, 3] = 0x8000
        bits[:, 5] = 0x0001
    return bits


def check_product(got, ref, absref, k, what):
    """A GEMM output against the fp64 product of the dequantized operands.
    Each output sums k / 128 matrix-core steps of 128 products (four scaled
    blocks of 32 per step) in fp32: at most 5 roundings per step, each moving
    it by at most 2^-24 of the running sum of |a||b| (absref).  So every
    element lies within 5 (k / 128) 2^-24 absref of the fp64 value, and the
    relative Frobenius error must not exceed 1e-6."""
    bound = 5 * (k // 128) * 2.0 ** -24 * absref
    over = np.abs(got - ref) > bound
    assert not over.any(), (what, int(over.sum()), np.argwhere(over)[:4].tolist())
    err = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    assert err <= 1e-6, (what, err)
    return err


def stats_close(st, ref, top_err=2.0):
    """GPU statistics against the oracle's.  Counts must be equal.  The fp64
    sums add the same per-element terms (each term is the same fp64
    expression on both sides) in different orders: the GPU in per-lane sums,
    then a fixed tree; the oracle in element order.  Recursive summation of n
    terms in any order is within (n - 1) 2^-53 sum|t_i| of the exact sum, so
    the two differ by at most 2 (n - 1) 2^-53 sum|t_i|, with sum|t_i| bounded
    per sum: the sum itself for the non-negative ones (|y|, y^2, err^2),
    sqrt(n sum err^2) for the signed error (Cauchy-Schwarz), and top_err per
    element for the normalized errors |G_m - a| (at most 2, the largest
    saturation error of E2M1: a < 8 rounded to 6)."""
    for k in ("n", "n_saturated", "n_nonfinite_blocks", "level_count"):
        assert st[k] == ref[k], k
    n = max(ref["n"], 1)
    tol = lambda absum, cnt: 2.0 * max(cnt - 1, 0) * 2.0 ** -53 * absum
    bounds = {
        "sum_abs_y": tol(ref["sum_abs_y"], n),
        "sum_y2": tol(ref["sum_y2"], n),
        "sum_err2": tol(ref["sum_err2"], n),
        "sum_signed_err": tol(np.sqrt(n * ref["sum_err2"]), n),
        "sum_err_norm": tol(top_err * n, n),
        "sum_err_norm_sat": tol(top_err * ref["n_saturated"], ref["n_saturated"]),
    }
    for k, b in bounds.items():
        assert abs(st[k] - ref[k]) <= b, (k, st[k], ref[k], b)
    for m in range(8):
        c = ref["level_count"][m]
        assert abs(st["level_err_norm"][m] - ref["level_err_norm"][m]) <= tol(top_err * c, c), m
