/*
 * mxq_oracle.h -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded CPU definition of MX block-32 FP4
 * quantization with an optional block-Hadamard rotation, the matching
 * dequantization, the fp64 weight-gradient product and the shrinkage-bias /
 * SQNR statistics.  It exists to check the GPU library against; only the
 * tests, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header, table or constant with the GPU library.
 *
 * Sources (web pages; the method has no published code):
 *  [NEWS]  htx.com (es-es) news article on "Pretraining large language models
 *          with MXFP4 on Native FP4 Hardware" (arXiv 2605.09825), sections
 *          "Que es MXFP4?" (block format) and "Experimento de diagnostico"
 *          (the three training GEMMs; stochastic rounding; Hadamard with
 *          random sign inversion).
 *  [UFP4]  gist.science (pt) summary "Repensando o Vies de Encolhimento
 *          (Shrinkage Bias) no Pre-treinamento de LLMs em FP4" (arXiv
 *          2606.20381), sections "Metodologia 1. Analise Teorica do Vies de
 *          Encolhimento", "Metodologia 2. A Receita UFP4" and "Resultados
 *          Experimentais / Diagnosticos de Quantizacao e GEMM".
 *  [MXPT]  gist.science (pt) summary "Pre-treinamento de Modelos de Linguagem
 *          Grandes com MXFP4" (arXiv 2605.09825), section "Metodologia"
 *          (deterministic H16 / H32 rotations).
 *
 * Parity status: every function below is pinned by CPU tests against values
 * fixed by the pages or by mathematics (see tests/test_oracle_*.py); none is
 * "parity unpinned".
 */
#ifndef MXQ_ORACLE_H
#define MXQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_GRID_E2M1 = 0, ORC_GRID_E1M2 = 1, ORC_GRID_E2M1_MAX4 = 2, ORC_GRID_E2M1_MAX3 = 3 };
enum { ORC_RTNE = 0, ORC_SR = 1 };
enum { ORC_FMT_FP4 = 0, ORC_FMT_E2M3 = 1 };
enum { ORC_AXIS_ROW = 0, ORC_AXIS_COL = 1 };
/* Random signs of the rotation: one n-bit mask shared by every block, or 32
 * signs per block drawn from Philox by the block's index along the
 * quantization axis (a sign vector as long as that axis). */
enum { ORC_SIGNS_MASK = 0, ORC_SIGNS_PER_BLOCK = 1 };

typedef struct {
    int32_t grid;        /* ORC_GRID_* */
    int32_t round;       /* ORC_RTNE or ORC_SR */
    int32_t hadamard_n;  /* 0 (no rotation), 16 or 32 */
    uint32_t sign_mask;  /* bit i set: negate block position i (mod n) before H */
    uint64_t sr_seed;    /* Philox key */
    uint32_t sr_stream;  /* Philox counter word 3 */
    uint32_t sr_bits;    /* random bits per element: 8 or 16 */
    uint32_t sign_mode;  /* ORC_SIGNS_MASK or ORC_SIGNS_PER_BLOCK */
    uint32_t pad_;
    uint64_t sign_seed;  /* Philox key of the per-block signs */
} orc_qparams;

typedef struct {
    double sum_abs_y;          /* sum |y| over finite blocks                     */
    double sum_signed_err;     /* sum sign(y) * (yhat - y)                        */
    double sum_y2;             /* sum y^2                                         */
    double sum_err2;           /* sum (yhat - y)^2                                */
    double sum_err_norm;       /* sum (|yhat| - |y|) * 2^-e   (normalized units)  */
    double sum_err_norm_sat;   /* same, only elements with a above the top level  */
    double level_err_norm[8];  /* per magnitude code m: sum (G_m - a)             */
    uint64_t n;                /* elements in finite blocks                       */
    uint64_t n_saturated;      /* elements with a > top level (clamped)           */
    uint64_t n_nonfinite_blocks;
    uint64_t level_count[8];   /* elements per magnitude code                     */
} orc_stats_t;

/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): out = bijection(ctr; key). */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

/* Grid level G_m (m = 0..7) decoded from the element format's bit fields
 * (the capped E2M1 grids decode their codes as E2M1). */
double orc_grid_level(int grid, int m);
/* Largest code the grid emits: 7, or 6 / 5 for E2M1 capped at 4 / 3. */
int orc_grid_top(int grid);
/* emax = ceil(log2(top level)) - 1: the block maximum is mapped into
 * (2^emax, 2^(emax+1)]; E2M1 (top 6) -> 2, E1M2 (top 3.5) -> 1, caps 4 and 3 -> 1. */
int orc_grid_emax(int grid);

/* In-place unnormalized fp32 fast Walsh-Hadamard transform, Sylvester order,
 * butterfly stages h = 1, 2, 4, ..., n/2. */
void orc_fwht_f32(float *u, int n);
/* Rotation of one 32-block: per n-sub-block, sign flip, FWHT, times fl32(1/sqrt n).
 * n = 0 copies. */
void orc_rotate_block(const float x[32], int n, uint32_t sign_mask, float y[32]);
/* The same with one sign bit per position of the 32-block (bit i: position i). */
void orc_rotate_block_signs(const float x[32], int n, uint32_t signs, float y[32]);
/* The 32 sign bits of block j (its index along the quantization axis) under p:
 * the mask repeated per n-sub-block, or word 0 of Philox4x32-10 with key
 * (lo32(sign_seed), hi32(sign_seed)) and counter (lo32(j), hi32(j),
 * 0xFFFFFFFF, 0xFFFFFFFE). */
uint32_t orc_block_signs(const orc_qparams *p, uint64_t j);

/* Shared E8M0 scale code of a rotated block (0xFF if any element is NaN/Inf). */
int orc_scale_code(int grid, const float y[32]);
/* Round a >= 0 (already divided by 2^e) to a magnitude code 0..7. */
int orc_round_rtne(int grid, double a);
int orc_round_sr(int grid, double a, uint32_t r, int bits);
/* The random value used for element j of block b under the SR stream. */
uint32_t orc_sr_random(uint64_t seed, uint32_t stream, uint64_t b, int j, int bits);

/* Quantize one 32-block.  nib[i] = sign<<3 | m.  block_index keys the SR
 * stream (the block's position in its scale array); j is the block's index
 * along the quantization axis (it keys per-block signs). */
void orc_quantize_block(const float x[32], const orc_qparams *p, uint64_t block_index,
                        uint64_t j, uint8_t nib[32], uint8_t *scale);

/* E2M3 6-bit code (sign in bit 5) holding the value (-1)^s * G_m exactly. */
int orc_e2m3_code(int grid, int nibble);

/* Quantize a bf16 matrix x[rows x cols] (leading dimension ld elements).
 * axis ROW: blocks along cols, outputs [rows x cols/32] blocks.
 * axis COL: blocks along rows, outputs transposed [cols x rows/32] blocks.
 * codes: FP4 -> 16 B per block (low nibble first); E2M3 -> 24 B per block
 * (code i at bits 6i..6i+5, little endian).  scales: 1 B per block.
 * Returns 0, or -1 on a bad shape. */
int orc_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, int axis,
                 const orc_qparams *p, int fmt, uint8_t *codes, uint8_t *scales);

/* The same for a slice: x holds only the lines line0 .. line0 + lines - 1 of a
 * larger tensor (the rows for axis ROW, the columns for axis COL); block
 * indices (which key the SR stream) are those of the whole tensor. */
int orc_quantize_lines(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, int axis,
                       const orc_qparams *p, int fmt, int64_t line0, uint8_t *codes,
                       uint8_t *scales);

/* Row layout -> the 16x16x128 matrix-core operand layout (a byte permutation;
 * bytes of padding lines / absent steps are left untouched). k % 128 == 0. */
int orc_to_mfma_layout(const uint8_t *codes, const uint8_t *scales, int64_t lines, int64_t k,
                       int fmt, uint8_t *tcodes, uint8_t *tscales);

/* Dequantize [lines x k] blocks (k along the block axis) to fp64. */
int orc_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t lines, int64_t k,
                   int grid, int fmt, double *out);

/* C[i][j] = sum_t A[i][t] * B[j][t] in fp64, A [m x k], B [n x k]. */
void orc_gemm_abt_f64(const double *a, const double *b, int64_t m, int64_t n, int64_t k,
                      double *c);

/* Bias / SQNR statistics of a quantized tensor against its rotated source. */
int orc_stats(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, int axis,
              const orc_qparams *p, int fmt, const uint8_t *codes, const uint8_t *scales,
              orc_stats_t *out);

/* The fp32 rotated values y in output (line-major) order: [lines x k]. */
int orc_rotate(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, int axis,
               const orc_qparams *p, float *y);

#ifdef __cplusplus
}
#endif
#endif
