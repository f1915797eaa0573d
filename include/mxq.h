/*
 * mxq.h -- C ABI of libmxq: MX block-32 FP4 quantization with a block
 * Hadamard rotation, and the block-scaled FP4 weight-gradient GEMM, for AMD
 * Instinct MI355X (gfx950).
 *
 * The method follows four web pages:
 *  - htx.com (es-es) news on "Pretraining large language models with MXFP4 on
 *    Native FP4 Hardware" (arXiv 2605.09825): section "Que es MXFP4?" (blocks
 *    of 32 elements with one shared E8M0 exponent, the block's largest
 *    exponent; 4-bit float elements) and section "Experimento de diagnostico"
 *    (the Fprop / Dgrad / Wgrad GEMMs Y = X W^T, dX = dY W, dW = dY^T X;
 *    stochastic rounding; Hadamard transform after random sign inversion).
 *  - gist.science (pt) summary "Pre-treinamento de Modelos de Linguagem
 *    Grandes com MXFP4": section "Metodologia" (deterministic H16 and H32
 *    rotations).
 *  - gist.science (pt, ko) summary "Repensando o Vies de Encolhimento
 *    (Shrinkage Bias) no Pre-treinamento de LLMs em FP4": "Metodologia 1"
 *    (RTNE on the non-uniform E2M1 grid and its shrinkage bias (l_i - r_i)/2),
 *    "Metodologia 2" (the uniform E1M2 / INT4-style grid; SR only on dY),
 *    "Resultados Experimentais" (SQNR diagnostics) and "Eficiencia" (fused
 *    rotation + quantization).
 *
 * Conventions for every call:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    allocates nothing and keeps no mutable global state, except the static
 *    per-device workspace of mxq_bias_stats_noalloc (below).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued asynchronously; nothing is synchronized.
 *  - Arguments are validated on the host before any launch; on failure the
 *    call returns a non-zero mxq_status and has no side effect.  A failed
 *    launch returns MXQ_ERR_DEVICE.  Faults inside kernels surface at the
 *    caller's next synchronization.  Nothing is printed.
 *  - Calls are thread-safe; calls that write the same output race.
 */
#ifndef MXQ_H
#define MXQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXQ_ABI_VERSION 5

typedef int32_t mxq_status;
#define MXQ_OK 0
#define MXQ_ERR_NULL 1          /* a required pointer is NULL                 */
#define MXQ_ERR_SHAPE 2         /* a size is negative / not a multiple of 32  */
#define MXQ_ERR_ALIGN 3         /* a pointer or leading dimension misaligned  */
#define MXQ_ERR_UNSUPPORTED 4   /* an enum value or combination not supported */
#define MXQ_ERR_DEVICE 5        /* the HIP launch failed                      */
#define MXQ_ERR_WORKSPACE 6     /* the workspace is missing or too small      */

/* Element grids (the 3-bit magnitude m of a sign-magnitude nibble s<<3|m):
 *   MXQ_GRID_E2M1: m -> {0, 0.5, 1, 1.5, 2, 3, 4, 6}; top-level exponent emax 2.
 *   MXQ_GRID_E1M2: m -> 0.5*m = {0, 0.5, ..., 3.5} (uniform); emax 1.
 *   MXQ_GRID_E2M1_MAX4, MXQ_GRID_E2M1_MAX3: E2M1 with its range restricted,
 *     the ablation of the gist.science summary "Repensando o Vies de
 *     Encolhimento ... em FP4", "Resultados Experimentais": E2M1's codes and
 *     values up to a cap of 4 (m <= 6) or 3 (m <= 5); larger magnitudes go to
 *     the cap.  emax 1 for both, so a block's normalized maximum lies in
 *     [2, 4).  Their codes are plain E2M1 nibbles (FP4 operands of the
 *     matrix cores as they stand).
 * In general emax = ceil(log2(top level)) - 1: the block maximum is mapped
 * into the binade (2^emax, 2^(emax+1)] that holds the grid's top level. */
#define MXQ_GRID_E2M1 0
#define MXQ_GRID_E1M2 1
#define MXQ_GRID_E2M1_MAX4 2
#define MXQ_GRID_E2M1_MAX3 3

/* Rounding of the normalized magnitude a = |y| / 2^e onto the grid:
 *   MXQ_ROUND_RTNE: nearest level, ties to the even code, saturating.
 *   MXQ_ROUND_SR:   between the neighbouring levels q_k <= a < q_(k+1), round
 *                   up iff r + 1/2 < p * 2^B with p = (a - q_k)/(q_(k+1) - q_k)
 *                   and r the element's B random bits (below); a at or above
 *                   the top level stays at the top level. */
#define MXQ_ROUND_RTNE 0
#define MXQ_ROUND_SR 1

/* Code storage of one 32-element block:
 *   MXQ_FMT_FP4:  16 bytes; byte j = nibble(2j) | nibble(2j+1) << 4.
 *   MXQ_FMT_E2M3: 24 bytes; element i is the OCP FP6 E2M3 code (sign in bit 5)
 *                 of the same value, at bits 6i..6i+5 of the little-endian
 *                 192-bit block.  Lossless for both grids; it is the operand
 *                 form the FP6 matrix cores read (E1M2 levels are not E2M1). */
#define MXQ_FMT_FP4 0
#define MXQ_FMT_E2M3 1

/* Placement of a block-quantized tensor's blocks in memory:
 *   MXQ_LAYOUT_ROWS:  codes [lines][k/32][block bytes], scales [lines][k/32].
 *   MXQ_LAYOUT_MFMA:  the operand order of the 16x16x128 block-scaled matrix
 *                     cores, so a GEMM streams each operand contiguously.
 *                     With T = ceil(lines/16) tiles of 16 lines, K steps of 4
 *                     blocks (s = b / 4) and lane l = 16 g + r for block
 *                     4 s + g of line 16 t + r:
 *                       codes  [k/128 steps][T][64 lanes][block bytes],
 *                       scales [ceil(k/512) groups][T][64 lanes][4 bytes],
 *                     byte j of a lane's scale word is the scale of step
 *                     4 q + j of group q.  Needs k % 128 == 0.  The bytes of
 *                     padding lines (lines..16T-1) and of absent steps in a
 *                     last partial group are never written or read. */
#define MXQ_LAYOUT_ROWS 0
#define MXQ_LAYOUT_MFMA 1

#define MXQ_AXIS_ROW 0          /* blocks run along the last (contiguous) dim */
#define MXQ_AXIS_COL 1          /* blocks run along the first dim; transposed */

#define MXQ_OUT_F32 0
#define MXQ_OUT_BF16 1

#define MXQ_SIGNS_MASK 0        /* one sign mask shared by every block        */
#define MXQ_SIGNS_PER_BLOCK 1   /* each block draws its own 32 signs          */

/* Quantizer knobs.
 * hadamard_n: 0 (no rotation), 16 or 32.  Each n-element sub-block of a
 *   32-block is replaced by fl32(1/sqrt(n)) * H_n * (D x), H_n the Sylvester
 *   Hadamard matrix in natural order, computed in fp32 by butterfly stages of
 *   stride 1, 2, 4, ... (the stage order fixes the fp32 rounding).
 * sign_mode, sign_mask, sign_seed: D = diag(d_i) for position i of the
 *   32-block, the random sign inversion before the transform (htx.com news,
 *   "Experimento de diagnostico").
 *   MXQ_SIGNS_MASK: d_i = -1 where bit (i mod n) of sign_mask is set, the
 *     same for every block; mask 0 gives the deterministic Hadamard
 *     rotation, a random mask the randomized one (RHT).
 *   MXQ_SIGNS_PER_BLOCK: a sign vector as long as the quantization axis.
 *     The block with index j along that axis (the same j on every line)
 *     takes d_i = -1 where bit i of word 0 of Philox4x32-10 is set, with key
 *     (lo32(sign_seed), hi32(sign_seed)) and counter (lo32(j), hi32(j),
 *     0xFFFFFFFF, 0xFFFFFFFE).
 *   Both operands of one GEMM must use the same signs along their shared
 *   axis (same mode and mask or seed); the rotation then cancels.
 * sr_seed, sr_stream, sr_bits: the stochastic-rounding stream.  Element j of
 *   the block with index b (its position in the scale array, row-major) takes
 *   Philox4x32-10 with key (lo32(seed), hi32(seed)):
 *     B = 16: counter (j>>3, lo32(b), hi32(b), stream), 16-bit half (j&1) of
 *             output word ((j>>1)&3);
 *     B = 8:  counter (j>>4, lo32(b), hi32(b), stream), byte (j&3) of word
 *             ((j>>2)&3). */
typedef struct {
    int32_t grid;
    int32_t round;
    int32_t hadamard_n;
    uint32_t sign_mask;
    uint64_t sr_seed;
    uint32_t sr_stream;
    uint32_t sr_bits;
    uint32_t sign_mode;   /* MXQ_SIGNS_* */
    uint32_t reserved;    /* 0 */
    uint64_t sign_seed;   /* key of the per-block signs */
} mxq_qconfig;

/* A block-quantized tensor of `lines` lines, each `k` elements long (k % 32
 * == 0): 16 (FP4) or 24 (E2M3) code bytes and one E8M0 scale byte (value
 * 2^(s-127); 0xFF marks a non-finite block) per 32-element block, placed as
 * `layout` says.  codes must be 4-byte aligned (16-byte for MXQ_LAYOUT_MFMA,
 * whose scales must be 4-byte aligned). */
typedef struct {
    void *codes;
    uint8_t *scales;
    int32_t fmt;     /* MXQ_FMT_* */
    int32_t grid;    /* MXQ_GRID_* of the stored values */
    int32_t layout;  /* MXQ_LAYOUT_* */
} mxq_qtensor;

/* Shrinkage-bias / SQNR sums over the rotated values y of the blocks with a
 * finite scale (fp64, fixed-order reduction, so repeatable).  e is the
 * block's scale exponent, a = |y| 2^-e, yhat the reconstruction. */
typedef struct {
    double sum_abs_y;          /* sum |y|                                     */
    double sum_signed_err;     /* sum sign(y) (yhat - y)                      */
    double sum_y2;             /* sum y^2                                     */
    double sum_err2;           /* sum (yhat - y)^2                            */
    double sum_err_norm;       /* sum (|yhat| - |y|) 2^-e                     */
    double sum_err_norm_sat;   /* the same over elements with a > top level   */
    double level_err_norm[8];  /* per magnitude code m: sum (G_m - a)         */
    uint64_t n;                /* elements counted                            */
    uint64_t n_saturated;      /* elements with a > top level                 */
    uint64_t n_nonfinite_blocks;
    uint64_t level_count[8];
} mxq_stats;

/* Fused rotate + scale + round + pack of a bf16 matrix x [rows x cols]
 * (row-major, leading dimension ld_x >= cols elements, x 2-byte aligned;
 * 128-bit loads are used when x is 16-byte aligned and ld_x % 8 == 0, else
 * 16-bit loads), the quantization of every GEMM operand in the three training
 * GEMMs (htx.com news, "Experimento de diagnostico"; the fused form follows
 * the "Eficiencia" section of the shrinkage-bias summary).
 *   row_out (may be NULL): blocks along cols, lines = rows, k = cols
 *                          (needs cols % 32 == 0).
 *   col_out (may be NULL): blocks along rows, written transposed: lines =
 *                          cols, k = rows (needs rows % 32 == 0).
 * At least one output is required; with both, one pass produces both (the
 * row output rotates along cols, the column output along rows, each with the
 * same mask).  Each output's grid must equal cfg->grid.
 * Errors: NULL cfg/x/outputs -> MXQ_ERR_NULL; bad sizes -> MXQ_ERR_SHAPE;
 * misaligned x/codes -> MXQ_ERR_ALIGN; bad knobs -> MXQ_ERR_UNSUPPORTED. */
mxq_status mxq_quantize(const mxq_qconfig *cfg, const void *x, int64_t rows, int64_t cols,
                        int64_t ld_x, const mxq_qtensor *row_out, const mxq_qtensor *col_out,
                        void *stream);

/* One tensor of mxq_quantize_batch: the arguments of one mxq_quantize call. */
typedef struct {
    const mxq_qconfig *cfg;
    const void *x;
    int64_t rows, cols, ld_x;
    const mxq_qtensor *row_out;  /* may be NULL */
    const mxq_qtensor *col_out;  /* may be NULL */
} mxq_quantize_job;

/* mxq_quantize for `count` tensors at once, e.g. the two operands of the
 * weight-gradient product, dY with SR and X with RTNE (htx.com news,
 * "Experimento de diagnostico").  The outputs are bit-identical to calling
 * mxq_quantize on each job in turn.  Every job is checked first, with
 * mxq_quantize's checks and status codes; on the first failure nothing is
 * launched and that status is returned.  Consecutive jobs that ask for a
 * column output only and share the grid family (E1M2, or the E2M1 grids),
 * hadamard_n and the column code format run as ONE launch (up to 8 jobs per
 * launch), their workgroups in job order; the rounding mode, seeds, signs,
 * shapes and layouts may differ.  Other jobs get their own launches, in
 * order.  No output may overlap another job's output or input (inputs may
 * be shared).  count == 0 does nothing; count < 0 -> MXQ_ERR_SHAPE; NULL
 * jobs with count > 0 -> MXQ_ERR_NULL.  A launch failure returns
 * MXQ_ERR_DEVICE; the launches before it stay enqueued. */
mxq_status mxq_quantize_batch(const mxq_quantize_job *jobs, int32_t count, void *stream);

/* Reconstruct yhat = (-1)^s G_m 2^(scale-127) (NaN for scale 0xFF) of a
 * block-quantized tensor into out [lines x k] (leading dimension ld_out
 * elements), as fp32 or bf16 (both exact).  The shared-exponent
 * reconstruction of the htx.com news, section "Que es MXFP4?". */
mxq_status mxq_dequantize(const mxq_qtensor *q, int64_t lines, int64_t k, int32_t out_dtype,
                          void *out, int64_t ld_out, void *stream);

/* The weight-gradient GEMM dW = dY^T X of the htx.com news ("Experimento de
 * diagnostico"), on block-quantized operands that both run along the token
 * axis: C [m x n] fp32 (leading dimension ldc) = A [m x k] * B [n x k]^T,
 * where A = dY quantized column-wise (m = its column count) and B = X
 * quantized column-wise.  Each product term carries both block scales; the
 * sum is accumulated in fp32 on the block-scaled matrix cores.
 * Operands: FP4 codes of the E2M1 grid, or E2M3 codes of either grid (A and
 * B may differ).  k % 128 == 0; m, n >= 0 (any).  C is fully overwritten.
 * Deterministic: no split-K, fixed summation order. */
mxq_status mxq_wgrad_gemm(const mxq_qtensor *a, const mxq_qtensor *b, int64_t m, int64_t n,
                          int64_t k, float *c, int64_t ldc, void *stream);

/* The rotation step of mxq_quantize on its own (the first kernel of the
 * unfused pipeline that the fused quantizer replaces, gist.science summary
 * "Repensando o Vies de Encolhimento (Shrinkage Bias) no Pre-treinamento de
 * LLMs em FP4", section "Eficiencia"): y = fl32(1/sqrt(n)) H_n (D x) on every
 * n-element sub-block of the 32-blocks along `axis` (MXQ_AXIS_ROW: along the
 * last dimension; MXQ_AXIS_COL: along the first), written to out in x's own
 * orientation [rows x cols], leading dimension ld_out elements.  out_dtype
 * MXQ_OUT_F32 gives exactly the values mxq_quantize rounds; MXQ_OUT_BF16
 * rounds them to nearest even.  cfg->hadamard_n must be 16 or 32 (cfg's
 * grid / rounding fields are ignored).  Requires the axis length % 32 == 0
 * and x, out aligned to their element size; 16-byte aligned rows
 * (out % 16 == 0, ld_out * element size % 16 == 0) take vector stores. */
mxq_status mxq_rotate(const mxq_qconfig *cfg, const void *x, int64_t rows, int64_t cols,
                      int64_t ld_x, int32_t axis, int32_t out_dtype, void *out, int64_t ld_out,
                      void *stream);

/* The same block-scaled product under its general name, for the three GEMMs
 * of a linear layer in the htx.com news ("Experimento de diagnostico"):
 *   Fprop  Y [T x N]  = X [T x K] W^T:  a = X row-wise,  b = W row-wise
 *          (m = T, n = N, k = K);
 *   Dgrad  dX [T x K] = dY [T x N] W:  a = dY row-wise, b = W column-wise
 *          (W's blocks run along N; m = T, n = K, k = N);
 *   Wgrad  dW [N x K] = dY^T X:        a = dY column-wise, b = X column-wise
 *          (m = N, n = K, k = T).
 * Both operands of one product must carry the same rotation along k (same
 * hadamard_n and sign_mask), which then cancels in the product.  Arguments,
 * requirements and errors as mxq_wgrad_gemm. */
mxq_status mxq_gemm_abt(const mxq_qtensor *a, const mxq_qtensor *b, int64_t m, int64_t n,
                        int64_t k, float *c, int64_t ldc, void *stream);

/* Bias / SQNR statistics of the shrinkage-bias summary ("Metodologia 1",
 * "Resultados Experimentais") for a tensor q produced by mxq_quantize from x
 * with the same cfg and axis; the rotated y is recomputed exactly as the
 * quantizer does.  `out` is a DEVICE pointer to one mxq_stats, fully
 * overwritten.  `workspace` is a device buffer of at least
 * mxq_bias_stats_workspace_size(rows, cols, axis) bytes. */
mxq_status mxq_bias_stats(const mxq_qconfig *cfg, const void *x, int64_t rows, int64_t cols,
                          int64_t ld_x, int32_t axis, const mxq_qtensor *q, mxq_stats *out,
                          void *workspace, size_t ws_bytes, void *stream);
/* Utility (no passage defines it): the workspace mxq_bias_stats needs, in
 * bytes (0 for negative sizes). */
size_t mxq_bias_stats_workspace_size(int64_t rows, int64_t cols, int32_t axis);

/* The effective bucket ratio that the shrinkage-bias summary ("Resultados
 * Experimentais") reports rising under the Hadamard rotation, which the
 * pages do not define; read here as exp(H) / L, with H the entropy (nats) of
 * the magnitude-code histogram stats->level_count and L the number of levels
 * `grid` emits (8; 7 and 6 for E2M1 capped at 4 and 3).  1 when all levels are
 * used equally, 1/L when all elements share one.  Host function: `stats` is a
 * HOST pointer (an mxq_stats copied back from the device).  Returns NaN for a
 * NULL pointer, an unknown grid or an empty histogram. */
double mxq_bucket_ratio(const mxq_stats *stats, int32_t grid);

/* mxq_bias_stats for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments without the workspace, the same checks, status codes and
 * results.  The workspace is a static device array of 204800 bytes that
 * each GPU holds until the process ends, found on the first call on a device
 * (with that device current; `stream` must belong to the current device).
 * A call that would need more returns MXQ_ERR_WORKSPACE (none does: the
 * workspace is at most 204800 bytes for any size).  The call allocates
 * nothing.  Every call on one GPU shares its array: calls that overlap on
 * one GPU race. */
mxq_status mxq_bias_stats_noalloc(const mxq_qconfig *cfg, const void *x, int64_t rows,
                                  int64_t cols, int64_t ld_x, int32_t axis, const mxq_qtensor *q,
                                  mxq_stats *out, void *stream);

/* The rounding step of mxq_quantize on its own, for checks of every input
 * value: codes[i] = the sign-magnitude nibble of a[i] (a value already
 * divided by its block scale 2^e, so |a| < 2^(emax+1) is the meaningful
 * range; larger magnitudes saturate) under the grid and rounding of the
 * shrinkage-bias summary ("Metodologia 1" RTNE, "Metodologia 2" SR).  For SR,
 * rand[i] holds element i's sr_bits random bits (the caller draws them);
 * rand may be NULL for RTNE.  a, rand, codes are device arrays of n items. */
mxq_status mxq_round_to_grid(int32_t grid, int32_t round, int32_t sr_bits, const float *a,
                             const uint16_t *rand, int64_t n, uint8_t *codes, void *stream);

/* A random sign mask for the randomized Hadamard rotation (RHT: random sign
 * inversion before the transform, htx.com news "Experimento de diagnostico";
 * gist.science summary "Pre-treinamento de Modelos de Linguagem Grandes com
 * MXFP4", "Metodologia"), drawn from a seed: the low n bits (n = 16 or 32) of
 * output word 0 of Philox4x32-10 with key (lo32(seed), hi32(seed)) and counter
 * (0, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF) -- a counter no block of the
 * stochastic-rounding stream uses.  Host function; returns 0 for other n. */
uint32_t mxq_rht_sign_mask(uint64_t seed, uint32_t n);

/* Utilities (no passage defines them): a static description of a status
 * code, and the ABI version the library was built with (MXQ_ABI_VERSION). */
const char *mxq_status_string(mxq_status s);
int32_t mxq_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MXQ_H */
