"""CPU pins of the oracle's rotation (against scipy's Sylvester Hadamard
matrix in fp64), its Philox4x32-10 (against rocRAND's engine), the SR stream
layout, the transposed (column-wise) layout, and the fp64 GEMM (against
numpy's matmul)."""
import os
import shutil
import subprocess

import numpy as np
import pytest
import scipy.linalg

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("n", [16, 32])
def test_sylvester_hadamard_orthogonal(n):
    H = scipy.linalg.hadamard(n).astype(np.float64)
    assert np.array_equal(H @ H.T, n * np.eye(n))


@pytest.mark.parametrize("n", [2, 4, 8, 16, 32])
def test_fwht_equals_dense_hadamard(orc, n):
    H = scipy.linalg.hadamard(n).astype(np.float64)
    g = np.random.Generator(np.random.PCG64(n))
    # small integers: fp32 butterflies are exact, so equality
    xi = g.integers(-1000, 1000, n).astype(np.float32)
    assert np.array_equal(orc.fwht_f32(xi).astype(np.float64), H @ xi.astype(np.float64))
    # random reals: within the fp32 rounding of log2(n) stages
    for _ in range(50):
        x = g.standard_normal(n).astype(np.float32)
        ref = H @ x.astype(np.float64)
        got = orc.fwht_f32(x).astype(np.float64)
        assert np.linalg.norm(got - ref) <= 1e-6 * np.linalg.norm(ref)


@pytest.mark.parametrize("n", [16, 32])
def test_rotate_block_is_normalized_hadamard_of_signed_input(orc, n):
    H = scipy.linalg.hadamard(n).astype(np.float64) / np.sqrt(n)
    g = np.random.Generator(np.random.PCG64(40 + n))
    for trial in range(40):
        x = g.standard_normal(32).astype(np.float32) * np.float32(10.0 ** g.integers(-3, 3))
        mask = int(g.integers(0, 1 << n)) if trial % 2 else 0
        d = np.array([-1.0 if (mask >> (i % n)) & 1 else 1.0 for i in range(32)])
        ref = np.concatenate([H @ (d[s:s + n] * x[s:s + n]) for s in range(0, 32, n)])
        y = orc.rotate_block(x, n, mask).astype(np.float64)
        assert np.linalg.norm(y - ref) <= 2e-6 * np.linalg.norm(ref)
        # orthonormal: the norm is preserved
        assert abs(np.linalg.norm(y) - np.linalg.norm(x)) <= 2e-6 * np.linalg.norm(x)


def test_rotate_h16_acts_on_two_halves(orc):
    x = np.zeros(32, np.float32)
    x[16:] = np.arange(16, dtype=np.float32)
    y = orc.rotate_block(x, 16)
    assert np.all(y[:16] == 0)
    x2 = np.zeros(32, np.float32)
    x2[:16] = np.arange(16, dtype=np.float32)
    assert np.array_equal(orc.rotate_block(x2, 16)[:16], y[16:])


@pytest.fixture(scope="module")
def rocrand_philox(tmp_path_factory):
    src = os.path.join(HERE, "golden", "philox_rocrand.cpp")
    inc = "/opt/rocm/include"
    if not os.path.exists(os.path.join(inc, "rocrand", "rocrand_philox4x32_10.h")):
        pytest.skip("rocRAND headers not installed")
    if shutil.which("g++") is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("philox") / "philox_rocrand")
    subprocess.run(["g++", "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I", inc, src,
                    "-o", exe], check=True)
    return exe


def test_philox_matches_rocrand_engine(orc, rocrand_philox):
    g = np.random.Generator(np.random.PCG64(99))
    cases = [(0, 0, 0, 0, 0, 0), (0xFFFFFFFF, 0xFFFFFFFF, 0, 0, 0, 0),
             (7, 0, 3, 1, 5, 0), (0, 0, 0, 0, 0xFFFFFFFF, 0xFFFFFFFF)]
    for _ in range(200):
        k0, k1, c0, c2, c3 = (int(v) for v in g.integers(0, 1 << 32, 5))
        c1 = int(g.integers(0, 1 << 30))   # rocRAND takes ctr words 0-1 as offset/4
        cases.append((k0, k1, c0, c1, c2, c3))
    stdin = "".join("%x %x %x %x %x %x\n" % c for c in cases)
    out = subprocess.run([rocrand_philox], input=stdin, capture_output=True, text=True,
                         check=True).stdout.split("\n")
    for c, line in zip(cases, out):
        want = [int(w, 16) for w in line.split()]
        got = orc.philox4x32_10(c[2:], c[:2]).tolist()
        assert got == want, c


def test_sr_random_stream_layout(orc):
    seed = 0x0123456789ABCDEF
    key = [seed & 0xFFFFFFFF, seed >> 32]
    for b in (0, 1, 12345, (1 << 32) + 17):
        for j in range(32):
            w = orc.philox4x32_10([j >> 3, b & 0xFFFFFFFF, b >> 32, 9], key)
            assert orc.sr_random(seed, 9, b, j, 16) == (int(w[(j >> 1) & 3]) >> (16 * (j & 1))) & 0xFFFF
            w8 = orc.philox4x32_10([j >> 4, b & 0xFFFFFFFF, b >> 32, 9], key)
            assert orc.sr_random(seed, 9, b, j, 8) == (int(w8[(j >> 2) & 3]) >> (8 * (j & 3))) & 0xFF


def _rand_bf16(rows, cols, seed):
    from fp4_microscaling_quantization_amd import synth
    return synth.normal(rows, cols, seed)


@pytest.mark.parametrize("n,mask,rnd", [(0, 0, 0), (16, 0xA5C3, 0), (32, 0xDEADBEEF, 1)])
def test_column_layout_is_row_layout_of_transpose(orc, n, mask, rnd):
    x = _rand_bf16(64, 96, 3)
    p = orc.qparams(grid=1, round=rnd, hadamard_n=n, sign_mask=mask, sr_seed=11)
    for fmt in (orc.FMT_FP4, orc.FMT_E2M3):
        cc, cs = orc.quantize(x, orc.AXIS_COL, p, fmt)
        rc, rs = orc.quantize(np.ascontiguousarray(x.T), orc.AXIS_ROW, p, fmt)
        assert np.array_equal(cc, rc) and np.array_equal(cs, rs)


def test_quantize_matches_block_function_and_block_index(orc):
    # the tensor-level call quantizes block (line, j) with block index
    # line * nblocks + j, in row-major scale order
    from fp4_microscaling_quantization_amd import synth
    x = _rand_bf16(8, 128, 4)
    xf = synth.bf16_bits_to_f32(x)
    p = orc.qparams(grid=0, round=1, hadamard_n=16, sign_mask=0x1234, sr_seed=5, sr_stream=2)
    codes, scales = orc.quantize(x, orc.AXIS_ROW, p)
    for r in range(8):
        for j in range(4):
            nib, sc = orc.quantize_block(xf[r, 32 * j:32 * j + 32], p, r * 4 + j)
            assert sc == scales[r, j]
            packed = nib[0::2] | (nib[1::2] << 4)
            assert np.array_equal(packed, codes[r, 16 * j:16 * j + 16])


def test_dequantize_fp4_and_e2m3_agree(orc):
    x = _rand_bf16(32, 64, 6)
    for grid in (0, 1):
        p = orc.qparams(grid=grid, hadamard_n=32, sign_mask=0xF0F0F0F0)
        c4, s4 = orc.quantize(x, orc.AXIS_ROW, p, orc.FMT_FP4)
        c6, s6 = orc.quantize(x, orc.AXIS_ROW, p, orc.FMT_E2M3)
        assert np.array_equal(s4, s6)
        assert np.array_equal(orc.dequantize(c4, s4, grid, orc.FMT_FP4),
                              orc.dequantize(c6, s6, grid, orc.FMT_E2M3))


def test_gemm_matches_numpy(orc):
    g = np.random.Generator(np.random.PCG64(8))
    a = g.standard_normal((17, 64))
    b = g.standard_normal((9, 64))
    assert np.allclose(orc.gemm_abt_f64(a, b), a @ b.T, rtol=1e-13, atol=1e-13)


def test_gemm_of_dequantized_integer_codes_is_exact(orc):
    # levels are dyadic; at scale 2^0 products and sums of a few terms are exact
    g = np.random.Generator(np.random.PCG64(9))
    codes = g.integers(0, 256, (8, 64)).astype(np.uint8)
    scales = np.full((8, 4), 127, np.uint8)
    for grid in (0, 1):
        a = orc.dequantize(codes, scales, grid)
        c = orc.gemm_abt_f64(a, a)
        ref = (a.astype(np.float64) * 2 ** 4).astype(np.int64)
        assert np.array_equal(c * 2 ** 8, (ref @ ref.T).astype(np.float64))


def test_quantize_lines_matches_whole_tensor(orc):
    x = _rand_bf16(96, 64, 12)
    p = orc.qparams(grid=1, round=1, hadamard_n=16, sign_mask=0xBEEF, sr_seed=99)
    for axis in (orc.AXIS_ROW, orc.AXIS_COL):
        c, s = orc.quantize(x, axis, p)
        c2, s2 = orc.quantize_lines(x, axis, p, 17, 9)
        assert np.array_equal(c[17:26], c2) and np.array_equal(s[17:26], s2)


@pytest.mark.parametrize("n", [16, 32])
def test_rotate_block_signs_matches_dense_product(orc, n):
    # y = c_n H_n D x per n-sub-block, D = diag(-1 where bit (position in the
    # 32-block) of the sign word is set), against scipy's H in fp64
    H = scipy.linalg.hadamard(n).astype(np.float64) / np.sqrt(n)
    g = np.random.Generator(np.random.PCG64(90 + n))
    for _ in range(100):
        x = g.standard_normal(32).astype(np.float32)
        s = int(g.integers(0, 1 << 32))
        d = np.where((s >> np.arange(32)) & 1, -1.0, 1.0)
        want = np.concatenate([H @ (d[b:b + n] * x[b:b + n].astype(np.float64))
                               for b in range(0, 32, n)])
        got = orc.rotate_block_signs(x, n, s).astype(np.float64)
        assert np.max(np.abs(got - want)) <= 1e-6 * np.max(np.abs(want)) + 1e-12
    # one mask for every block is the sign word that repeats it per sub-block
    x = g.standard_normal(32).astype(np.float32)
    m = 0xBEEF if n == 16 else 0xDEADBEEF
    rep = (m | (m << 16)) if n == 16 else m
    assert np.array_equal(orc.rotate_block(x, n, m), orc.rotate_block_signs(x, n, rep))


def test_per_block_signs_vary_by_block_and_seed(orc):
    p = orc.qparams(hadamard_n=32, sign_mode=orc.SIGNS_PER_BLOCK, sign_seed=12345)
    words = [orc.block_signs(p, j) for j in range(4096)]
    assert len(set(words)) == 4096                       # a new draw per block
    bits = np.array([bin(w).count("1") for w in words])
    assert abs(bits.mean() - 16) < 0.5                   # fair signs (sd of the mean ~0.045)
    q = orc.qparams(hadamard_n=32, sign_mode=orc.SIGNS_PER_BLOCK, sign_seed=12346)
    assert sum(orc.block_signs(q, j) == w for j, w in enumerate(words)) == 0
    # mask mode ignores j and repeats the mask per sub-block
    m = orc.qparams(hadamard_n=16, sign_mask=0x1234)
    assert {orc.block_signs(m, j) for j in range(10)} == {0x12341234}


@pytest.mark.parametrize("n", [16, 32])
@pytest.mark.parametrize("mode", [0, 1])
def test_rotation_cancels_in_the_product(orc, n, mode):
    # A [m x K] rotated along K row-wise and B [K x p] rotated along K
    # column-wise with the same signs: the product is unchanged (the rotation
    # is orthogonal), which pins that both orientations give position k the
    # same sign, also when every block draws its own
    from fp4_microscaling_quantization_amd import synth
    m, K, p = 24, 256, 40
    A = synth.f32_to_bf16_bits(np.random.Generator(np.random.PCG64(5)).standard_normal((m, K)).astype(np.float32))
    B = synth.f32_to_bf16_bits(np.random.Generator(np.random.PCG64(6)).standard_normal((K, p)).astype(np.float32))
    kw = dict(sign_mask=0xA5C3F00F, sign_mode=mode, sign_seed=777)
    ra = orc.rotate(A, orc.AXIS_ROW, n, **kw).astype(np.float64)      # [m x K]
    rb = orc.rotate(B, orc.AXIS_COL, n, **kw).astype(np.float64)      # [p x K]
    want = synth.bf16_bits_to_f32(A).astype(np.float64) @ synth.bf16_bits_to_f32(B).astype(np.float64)
    got = ra @ rb.T
    assert np.linalg.norm(got - want) <= 1e-6 * np.linalg.norm(want)
    if mode == 1:
        # and the rotated operands differ from the single-mask ones
        r0 = orc.rotate(A, orc.AXIS_ROW, n, sign_mask=0xA5C3F00F)
        assert not np.array_equal(r0, ra.astype(np.float32))
