/*
 * mxq_oracle.c -- TEST INFRASTRUCTURE ONLY: the plain CPU definition the GPU
 * library is checked against.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the product path never does.
 *
 * Built with -O2 -ffp-contract=off -fno-fast-math so every float operation is
 * the single IEEE operation written here.  Citations name the web pages as in
 * mxq_oracle.h ([NEWS], [UFP4], [MXPT]).
 */
#include "mxq_oracle.h"

#include <math.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Philox4x32-10, from the SC'11 paper "Parallel Random Numbers: As Easy as  */
/* 1, 2, 3": ten rounds; each round multiplies counter words 0 and 2 by two  */
/* fixed odd constants into 64-bit products, and the high halves are xored   */
/* with the other counter words and the round key; the key is bumped by two  */
/* Weyl constants between rounds.                                            */
/* ------------------------------------------------------------------------ */
#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += PHILOX_W0;
            k1 += PHILOX_W1;
        }
        uint64_t p0 = (uint64_t)PHILOX_M0 * (uint64_t)c0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* ------------------------------------------------------------------------ */
/* Element grids.  [UFP4] "Declaracao do Problema" names E2M1 as 2 exponent  */
/* bits and 1 mantissa bit; "Metodologia 2" asks for a uniform E1M2 / INT4   */
/* style grid with equal spacing.  Both are decoded here from their bit      */
/* fields as small floats: E2M1 with exponent bias 1 (levels 0 .. 6) and     */
/* E1M2 with exponent bias 0 (levels 0, 0.5, ..., 3.5).                      */
/*                                                                           */
/* [UFP4] "Resultados Experimentais" (ablations) also tries E2M1 with its    */
/* range restricted, a cap on the largest value, as a stand-in for a uniform */
/* grid.  Those grids keep E2M1's codes and values and stop at a top code:   */
/* code 6 (value 4) or code 5 (value 3).                                     */
/* ------------------------------------------------------------------------ */
static double minifloat_value(int ebits, int mbits, int bias, int code)
{
    int m = code & ((1 << mbits) - 1);
    int e = code >> mbits;
    (void)ebits;
    double frac = (double)m / (double)(1 << mbits);
    if (e == 0)
        return ldexp(frac, 1 - bias);        /* subnormal */
    return ldexp(1.0 + frac, e - bias);
}

double orc_grid_level(int grid, int m)
{
    if (grid == ORC_GRID_E1M2)
        return minifloat_value(1, 2, 0, m);
    return minifloat_value(2, 1, 1, m);      /* E2M1 and its capped forms */
}

int orc_grid_top(int grid)
{
    if (grid == ORC_GRID_E2M1_MAX4)
        return 6;
    if (grid == ORC_GRID_E2M1_MAX3)
        return 5;
    return 7;
}

/* The block maximum is mapped into the binade (2^emax, 2^(emax+1)] that     */
/* holds the grid's top level: emax = ceil(log2(top)) - 1.  E2M1 (top 6)     */
/* gives 2 and E1M2 (top 3.5) gives 1, the usual floor(log2(top)); a cap of  */
/* 4 or 3 gives 1, so a capped E2M1 block spans [2, 4) before rounding.      */
int orc_grid_emax(int grid)
{
    int k;
    double f = frexp(orc_grid_level(grid, orc_grid_top(grid)), &k);   /* top = f * 2^k */
    return f == 0.5 ? k - 2 : k - 1;
}

/* ------------------------------------------------------------------------ */
/* Block Hadamard rotation.  [MXPT] "Metodologia": deterministic 16x16 (H16) */
/* and 32x32 (H32) Hadamard rotations; [NEWS] "Experimento de diagnostico":  */
/* the randomized variant flips signs at random before the Hadamard          */
/* transform.  Sylvester-ordered H, applied by the fast transform in fp32    */
/* with stages of ascending stride, then scaled by fl32(1/sqrt(n)) so the    */
/* rotation is orthonormal.                                                  */
/* ------------------------------------------------------------------------ */
void orc_fwht_f32(float *u, int n)
{
    for (int h = 1; h < n; h <<= 1) {
        for (int i = 0; i < n; ++i) {
            if ((i & h) == 0) {
                float a = u[i];
                float b = u[i + h];
                u[i] = a + b;
                u[i + h] = a - b;
            }
        }
    }
}

void orc_rotate_block_signs(const float x[32], int n, uint32_t signs, float y[32])
{
    if (n == 0) {
        for (int i = 0; i < 32; ++i)
            y[i] = x[i];
        return;
    }
    float c = (float)(1.0 / sqrt((double)n));
    for (int s = 0; s < 32; s += n) {
        float u[32];
        for (int i = 0; i < n; ++i) {
            float v = x[s + i];
            u[i] = ((signs >> (s + i)) & 1u) ? -v : v;
        }
        orc_fwht_f32(u, n);
        for (int i = 0; i < n; ++i)
            y[s + i] = u[i] * c;
    }
}

/* one mask for every block: position i takes bit (i mod n) */
static uint32_t mask_signs(int n, uint32_t mask)
{
    if (n == 16)
        return (mask & 0xFFFFu) | ((mask & 0xFFFFu) << 16);
    return n == 32 ? mask : 0u;
}

void orc_rotate_block(const float x[32], int n, uint32_t sign_mask, float y[32])
{
    orc_rotate_block_signs(x, n, mask_signs(n, sign_mask), y);
}

/* [NEWS] "Experimento de diagnostico": the signs are random; a sign vector as
 * long as the quantization axis gives every block its own draw. */
uint32_t orc_block_signs(const orc_qparams *p, uint64_t j)
{
    if (p->hadamard_n == 0)
        return 0u;
    if (p->sign_mode != ORC_SIGNS_PER_BLOCK)
        return mask_signs(p->hadamard_n, p->sign_mask);
    uint32_t key[2] = { (uint32_t)p->sign_seed, (uint32_t)(p->sign_seed >> 32) };
    uint32_t ctr[4] = { (uint32_t)j, (uint32_t)(j >> 32), 0xFFFFFFFFu, 0xFFFFFFFEu };
    uint32_t out[4];
    orc_philox4x32_10(ctr, key, out);
    return out[0];
}

/* ------------------------------------------------------------------------ */
/* Shared scale.  [NEWS] "Que es MXFP4?": one E8M0 exponent per block of 32, */
/* set by the largest exponent in the block.  Read as                       */
/* e = floor(log2(amax)) - emax (so the block maximum lands in the top      */
/* binade of the grid), clamped below at -127; stored as e + 127.  An      */
/* all-zero block takes e = -127 (code 0); a block holding NaN or Inf takes */
/* the E8M0 NaN code 0xFF.                                                  */
/* ------------------------------------------------------------------------ */
int orc_scale_code(int grid, const float y[32])
{
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) {
        if (!isfinite(y[i]))
            return 0xFF;
        double v = fabs((double)y[i]);
        if (v > amax)
            amax = v;
    }
    if (amax == 0.0)
        return 0;
    int k;
    frexp(amax, &k);                 /* amax = f * 2^k, f in [0.5, 1) */
    int e = (k - 1) - orc_grid_emax(grid);
    if (e < -127)
        e = -127;
    return e + 127;
}

/* ------------------------------------------------------------------------ */
/* Rounding.  [UFP4] "Metodologia 1": round-to-nearest-even onto the grid   */
/* (the source of shrinkage on E2M1); "Metodologia 2": stochastic rounding   */
/* on the upstream gradient, exact elsewhere.  [NEWS] "Experimento de        */
/* diagnostico": stochastic rounding has zero expected rounding error.       */
/* ------------------------------------------------------------------------ */
int orc_round_rtne(int grid, double a)
{
    /* nearest level; on a tie between neighbours k-1 and k, the even code */
    int best = 0;
    double bestd = fabs(a - orc_grid_level(grid, 0));
    for (int k = 1; k <= orc_grid_top(grid); ++k) {
        double d = fabs(a - orc_grid_level(grid, k));
        if (d < bestd || (d == bestd && (k % 2) == 0)) {
            best = k;
            bestd = d;
        }
    }
    return best;
}

int orc_round_sr(int grid, double a, uint32_t r, int bits)
{
    const int top = orc_grid_top(grid);
    if (a >= orc_grid_level(grid, top))
        return top;                             /* top bin clamps */
    int k = 0;
    while (k < top && orc_grid_level(grid, k + 1) <= a)
        ++k;
    double lo = orc_grid_level(grid, k);
    if (a == lo)
        return k;
    double hi = orc_grid_level(grid, k + 1);
    double p = (a - lo) / (hi - lo);            /* in (0, 1) */
    double thresh = p * ldexp(1.0, bits);
    return ((double)r + 0.5 < thresh) ? k + 1 : k;
}

uint32_t orc_sr_random(uint64_t seed, uint32_t stream, uint64_t b, int j, int bits)
{
    uint32_t key[2] = { (uint32_t)seed, (uint32_t)(seed >> 32) };
    uint32_t out[4];
    if (bits == 16) {
        uint32_t ctr[4] = { (uint32_t)(j >> 3), (uint32_t)b, (uint32_t)(b >> 32), stream };
        orc_philox4x32_10(ctr, key, out);
        uint32_t w = out[(j >> 1) & 3];
        return (w >> (16 * (j & 1))) & 0xFFFFu;
    } else {
        uint32_t ctr[4] = { (uint32_t)(j >> 4), (uint32_t)b, (uint32_t)(b >> 32), stream };
        orc_philox4x32_10(ctr, key, out);
        uint32_t w = out[(j >> 2) & 3];
        return (w >> (8 * (j & 3))) & 0xFFu;
    }
}

/* ------------------------------------------------------------------------ */
/* One block: rotate, scale, divide by 2^e, round, sign-magnitude nibble.    */
/* ------------------------------------------------------------------------ */
void orc_quantize_block(const float x[32], const orc_qparams *p, uint64_t block_index,
                        uint64_t j, uint8_t nib[32], uint8_t *scale)
{
    float y[32];
    orc_rotate_block_signs(x, p->hadamard_n, orc_block_signs(p, j), y);
    int sc = orc_scale_code(p->grid, y);
    *scale = (uint8_t)sc;
    if (sc == 0xFF) {
        memset(nib, 0, 32);
        return;
    }
    int e = sc - 127;
    for (int i = 0; i < 32; ++i) {
        double a = ldexp(fabs((double)y[i]), -e);   /* exact */
        int m;
        if (p->round == ORC_SR)
            m = orc_round_sr(p->grid, a, orc_sr_random(p->sr_seed, p->sr_stream, block_index,
                                                       i, (int)p->sr_bits),
                             (int)p->sr_bits);
        else
            m = orc_round_rtne(p->grid, a);
        nib[i] = (uint8_t)((signbit(y[i]) ? 8 : 0) | m);
    }
}

/* E2M3: 1 sign, 2 exponent bits (bias 1), 3 mantissa bits.  Find the code  */
/* whose decoded value equals the level exactly.                            */
int orc_e2m3_code(int grid, int nibble)
{
    double v = orc_grid_level(grid, nibble & 7);
    for (int c = 0; c < 32; ++c) {
        if (minifloat_value(2, 3, 1, c) == v)
            return ((nibble & 8) ? 32 : 0) | c;
    }
    return -1;
}

static int check_shape(int64_t rows, int64_t cols, int64_t ld, int axis)
{
    if (rows < 0 || cols < 0 || ld < cols)
        return -1;
    if (axis == ORC_AXIS_ROW && cols % 32)
        return -1;
    if (axis == ORC_AXIS_COL && rows % 32)
        return -1;
    return 0;
}

static float bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Gather block (line, jb) in axis order. */
static void gather_block(const uint16_t *x, int64_t ld, int axis, int64_t line, int64_t jb,
                         float out[32])
{
    for (int i = 0; i < 32; ++i) {
        int64_t r, c;
        if (axis == ORC_AXIS_ROW) { r = line; c = jb * 32 + i; }
        else                      { r = jb * 32 + i; c = line; }
        out[i] = bf16_to_f32(x[r * ld + c]);
    }
}

static void store_codes(uint8_t *dst, int fmt, int grid, const uint8_t nib[32])
{
    if (fmt == ORC_FMT_FP4) {
        for (int j = 0; j < 16; ++j)
            dst[j] = (uint8_t)(nib[2 * j] | (nib[2 * j + 1] << 4));
    } else {
        memset(dst, 0, 24);
        for (int i = 0; i < 32; ++i) {
            int code = orc_e2m3_code(grid, nib[i]);
            for (int b = 0; b < 6; ++b) {
                int bit = 6 * i + b;
                if ((code >> b) & 1)
                    dst[bit >> 3] |= (uint8_t)(1u << (bit & 7));
            }
        }
    }
}

static int load_nibbles(const uint8_t *src, int fmt, int grid, uint8_t nib[32])
{
    if (fmt == ORC_FMT_FP4) {
        for (int j = 0; j < 16; ++j) {
            nib[2 * j] = src[j] & 15;
            nib[2 * j + 1] = src[j] >> 4;
        }
        return 0;
    }
    for (int i = 0; i < 32; ++i) {
        int code = 0;
        for (int b = 0; b < 6; ++b) {
            int bit = 6 * i + b;
            code |= ((src[bit >> 3] >> (bit & 7)) & 1) << b;
        }
        int found = -1;
        for (int n = 0; n < 16; ++n)
            if (orc_e2m3_code(grid, n) == code)
                found = n;
        if (found < 0) {
            /* -0 and +0 share a value; only +0/-0 codes of level 0 may be absent */
            return -1;
        }
        nib[i] = (uint8_t)found;
    }
    return 0;
}

int orc_quantize_lines(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, int axis,
                       const orc_qparams *p, int fmt, int64_t line0, uint8_t *codes,
                       uint8_t *scales)
{
    if (check_shape(rows, cols, ld, axis) || line0 < 0)
        return -1;
    int64_t lines = axis == ORC_AXIS_ROW ? rows : cols;
    int64_t k = axis == ORC_AXIS_ROW ? cols : rows;
    int64_t nblk = k / 32;
    int64_t bbytes = fmt == ORC_FMT_FP4 ? 16 : 24;
    for (int64_t line = 0; line < lines; ++line) {
        for (int64_t jb = 0; jb < nblk; ++jb) {
            float xb[32];
            uint8_t nib[32];
            int64_t local = line * nblk + jb;
            uint64_t b = (uint64_t)((line0 + line) * nblk + jb);
            gather_block(x, ld, axis, line, jb, xb);
            orc_quantize_block(xb, p, b, (uint64_t)jb, nib, &scales[local]);
            store_codes(codes + local * bbytes, fmt, p->grid, nib);
        }
    }
    return 0;
}

int orc_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, int axis,
                 const orc_qparams *p, int fmt, uint8_t *codes, uint8_t *scales)
{
    return orc_quantize_lines(x, rows, cols, ld, axis, p, fmt, 0, codes, scales);
}

int orc_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t lines, int64_t k,
                   int grid, int fmt, double *out)
{
    if (k % 32)
        return -1;
    int64_t nblk = k / 32;
    int64_t bbytes = fmt == ORC_FMT_FP4 ? 16 : 24;
    for (int64_t b = 0; b < lines * nblk; ++b) {
        uint8_t nib[32];
        if (load_nibbles(codes + b * bbytes, fmt, grid, nib))
            return -1;
        int sc = scales[b];
        for (int i = 0; i < 32; ++i) {
            double v;
            if (sc == 0xFF)
                v = NAN;
            else
                v = ldexp(orc_grid_level(grid, nib[i] & 7), sc - 127);
            out[b * 32 + i] = (nib[i] & 8) ? -v : v;
        }
    }
    return 0;
}

/* [NEWS] "Experimento de diagnostico": the weight gradient is dY^T X.  With */
/* both operands stored along the token axis, dW[i][j] = sum_t A[i][t]B[j][t]. */
void orc_gemm_abt_f64(const double *a, const double *b, int64_t m, int64_t n, int64_t k,
                      double *c)
{
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t j = 0; j < n; ++j) {
            double s = 0.0;
            for (int64_t t = 0; t < k; ++t)
                s += a[i * k + t] * b[j * k + t];
            c[i * n + j] = s;
        }
    }
}

int orc_rotate(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, int axis,
               const orc_qparams *p, float *y)
{
    if (check_shape(rows, cols, ld, axis))
        return -1;
    int64_t lines = axis == ORC_AXIS_ROW ? rows : cols;
    int64_t k = axis == ORC_AXIS_ROW ? cols : rows;
    for (int64_t line = 0; line < lines; ++line) {
        for (int64_t jb = 0; jb < k / 32; ++jb) {
            float xb[32];
            gather_block(x, ld, axis, line, jb, xb);
            orc_rotate_block_signs(xb, p->hadamard_n, orc_block_signs(p, (uint64_t)jb),
                                   y + line * k + jb * 32);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Statistics.  [UFP4] "Metodologia 1": shrinkage is a negative expected     */
/* error in normalized magnitude space; "Resultados Experimentais": SQNR.   */
/* All sums are over the rotated values y and their reconstruction yhat.   */
/* ------------------------------------------------------------------------ */
int orc_stats(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, int axis,
              const orc_qparams *p, int fmt, const uint8_t *codes, const uint8_t *scales,
              orc_stats_t *out)
{
    if (check_shape(rows, cols, ld, axis))
        return -1;
    memset(out, 0, sizeof(*out));
    int64_t lines = axis == ORC_AXIS_ROW ? rows : cols;
    int64_t k = axis == ORC_AXIS_ROW ? cols : rows;
    int64_t nblk = k / 32;
    int64_t bbytes = fmt == ORC_FMT_FP4 ? 16 : 24;
    double top = orc_grid_level(p->grid, orc_grid_top(p->grid));
    for (int64_t line = 0; line < lines; ++line) {
        for (int64_t jb = 0; jb < nblk; ++jb) {
            int64_t b = line * nblk + jb;
            float xb[32], y[32];
            uint8_t nib[32];
            gather_block(x, ld, axis, line, jb, xb);
            orc_rotate_block_signs(xb, p->hadamard_n, orc_block_signs(p, (uint64_t)jb), y);
            int sc = scales[b];
            if (sc == 0xFF) {
                out->n_nonfinite_blocks++;
                continue;
            }
            if (load_nibbles(codes + b * bbytes, fmt, p->grid, nib))
                return -1;
            int e = sc - 127;
            for (int i = 0; i < 32; ++i) {
                double yv = (double)y[i];
                int m = nib[i] & 7;
                double g = orc_grid_level(p->grid, m);
                double yh = ldexp(g, e);
                if (nib[i] & 8)
                    yh = -yh;
                double a = ldexp(fabs(yv), -e);
                double sgn = yv < 0 ? -1.0 : (yv > 0 ? 1.0 : 0.0);
                double err = yh - yv;
                out->sum_abs_y += fabs(yv);
                out->sum_signed_err += sgn * err;
                out->sum_y2 += yv * yv;
                out->sum_err2 += err * err;
                out->sum_err_norm += g - a;
                if (a > top) {
                    out->n_saturated++;
                    out->sum_err_norm_sat += g - a;
                }
                out->level_count[m]++;
                out->level_err_norm[m] += g - a;
                out->n++;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Operand placement of the 16x16x128 block-scaled matrix cores.  A pure    */
/* byte permutation of the row layout, no arithmetic: K steps of 4 blocks,  */
/* tiles of 16 lines; block 4 s + g of line 16 t + r is lane 16 g + r of    */
/* fragment (s, t); the scale of step s sits in byte s % 4 of that lane's   */
/* word in scale group s / 4.  Untouched bytes keep their prior contents.  */
/* ------------------------------------------------------------------------ */
int orc_to_mfma_layout(const uint8_t *codes, const uint8_t *scales, int64_t lines, int64_t k,
                       int fmt, uint8_t *tcodes, uint8_t *tscales)
{
    if (lines < 0 || k < 0 || k % 128)
        return -1;
    int64_t nbk = k / 32;
    int64_t ntiles = (lines + 15) / 16;
    int64_t bb = fmt == ORC_FMT_FP4 ? 16 : 24;
    for (int64_t line = 0; line < lines; ++line) {
        for (int64_t jb = 0; jb < nbk; ++jb) {
            int64_t step = jb / 4, g = jb % 4, tile = line / 16, r = line % 16;
            int64_t lane = 16 * g + r;
            int64_t dst = (step * ntiles + tile) * 64 + lane;
            memcpy(tcodes + dst * bb, codes + (line * nbk + jb) * bb, (size_t)bb);
            int64_t group = step / 4;
            tscales[((group * ntiles + tile) * 64 + lane) * 4 + step % 4] = scales[line * nbk + jb];
        }
    }
    return 0;
}
