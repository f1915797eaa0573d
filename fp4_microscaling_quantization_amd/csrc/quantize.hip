// Host side of mxq_quantize (argument checks, dispatch to the row, column and
// dual kernels of quantize_col.hip) and mxq_round_to_grid with its kernel.
//
// The rotation, scale and rounding are the method of the htx.com news
// "Pretraining large language models with MXFP4" (section "Que es MXFP4?",
// "Experimento de diagnostico"), the gist.science summaries "Pre-treinamento
// de Modelos de Linguagem Grandes com MXFP4" ("Metodologia": H16 / H32) and
// "Repensando o Vies de Encolhimento ... em FP4" ("Metodologia 1", "2",
// "Eficiencia": the fused rotate + quantize).
#include "mxq_device.hpp"
#include "mxq_host.hpp"
#include "quant_out.hpp"

namespace mxq {

template <int GRID, int ROUND>
__global__ __launch_bounds__(256) void k_round_to_grid(const float *__restrict__ a,
                                                       const uint16_t *__restrict__ rnd, int64_t n,
                                                       int sr_bits, float top,
                                                       uint8_t *__restrict__ out)
{
    const int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
    if (i0 >= n)
        return;
    float v[8];
    uint32_t r[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        v[k] = (i0 + k < n) ? a[i0 + k] : 0.0f;
        r[k] = (ROUND == kSR && i0 + k < n) ? (uint32_t)rnd[i0 + k] : 0u;
    }
    const uint32_t w = round8<GRID, ROUND>(v, 1.0f, r, sr_bits == 16 ? 131072.0f : 512.0f, top);
#pragma unroll
    for (int k = 0; k < 8; ++k)
        if (i0 + k < n)
            out[i0 + k] = (uint8_t)((w >> (4 * k)) & 15u);
}

// ---- host side ---------------------------------------------------------------

mxq_status check_qconfig(const mxq_qconfig *cfg)
{
    if (!cfg)
        return MXQ_ERR_NULL;
    if (cfg->grid < MXQ_GRID_E2M1 || cfg->grid > MXQ_GRID_E2M1_MAX3)
        return MXQ_ERR_UNSUPPORTED;
    if (cfg->round != MXQ_ROUND_RTNE && cfg->round != MXQ_ROUND_SR)
        return MXQ_ERR_UNSUPPORTED;
    if (cfg->hadamard_n != 0 && cfg->hadamard_n != 16 && cfg->hadamard_n != 32)
        return MXQ_ERR_UNSUPPORTED;
    if (cfg->round == MXQ_ROUND_SR && cfg->sr_bits != 8 && cfg->sr_bits != 16)
        return MXQ_ERR_UNSUPPORTED;
    if (cfg->sign_mode != MXQ_SIGNS_MASK && cfg->sign_mode != MXQ_SIGNS_PER_BLOCK)
        return MXQ_ERR_UNSUPPORTED;
    return MXQ_OK;
}

mxq_status check_qtensor_out(const mxq_qtensor *t, int32_t grid, int64_t k)
{
    if (!t->codes || !t->scales)
        return MXQ_ERR_NULL;
    if (t->fmt != MXQ_FMT_FP4 && t->fmt != MXQ_FMT_E2M3)
        return MXQ_ERR_UNSUPPORTED;
    if (t->layout != MXQ_LAYOUT_ROWS && t->layout != MXQ_LAYOUT_MFMA)
        return MXQ_ERR_UNSUPPORTED;
    if (t->grid != grid)
        return MXQ_ERR_UNSUPPORTED;
    if (t->layout == MXQ_LAYOUT_MFMA && k % 128)
        return MXQ_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(t->codes) % (t->layout == MXQ_LAYOUT_MFMA ? 16 : 4))
        return MXQ_ERR_ALIGN;
    if (t->layout == MXQ_LAYOUT_MFMA && reinterpret_cast<uintptr_t>(t->scales) % 4)
        return MXQ_ERR_ALIGN;
    return MXQ_OK;
}

QKnobs make_knobs(const mxq_qconfig *cfg)
{
    QKnobs kn;
    // one sign bit per position of the 32-block: a 16-bit mask repeats
    kn.sign_mask = cfg->hadamard_n == 16 ? (cfg->sign_mask & 0xFFFFu) * 0x10001u
                   : cfg->hadamard_n == 32 ? cfg->sign_mask : 0u;
    kn.sign_mode = cfg->sign_mode;
    kn.skey_lo = (uint32_t)cfg->sign_seed;
    kn.skey_hi = (uint32_t)(cfg->sign_seed >> 32);
    kn.seed_lo = (uint32_t)cfg->sr_seed;
    kn.seed_hi = (uint32_t)(cfg->sr_seed >> 32);
    kn.stream = cfg->sr_stream;
    kn.sr_bits = cfg->sr_bits == 8 ? 8u : 16u;
    // the E2M1 family's scale exponent and (twice) its top level; the capped
    // grids map the block maximum into [2, 4) and stop at 4 or 3
    kn.emax = cfg->grid == MXQ_GRID_E2M1 ? 2 : 1;
    kn.top2 = cfg->grid == MXQ_GRID_E2M1_MAX4 ? 8.0f : cfg->grid == MXQ_GRID_E2M1_MAX3 ? 6.0f : 12.0f;
    return kn;
}

namespace {

// The checks of mxq_quantize, in its documented order.
mxq_status check_quantize(const mxq_qconfig *cfg, const void *x, int64_t rows, int64_t cols,
                          int64_t ld_x, const mxq_qtensor *row_out, const mxq_qtensor *col_out)
{
    mxq_status st = check_qconfig(cfg);
    if (st)
        return st;
    if (!x || (!row_out && !col_out))
        return MXQ_ERR_NULL;
    if (rows < 0 || cols < 0 || ld_x < cols)
        return MXQ_ERR_SHAPE;
    if (row_out && cols % 32)
        return MXQ_ERR_SHAPE;
    if (col_out && rows % 32)
        return MXQ_ERR_SHAPE;
    if (row_out && (st = check_qtensor_out(row_out, cfg->grid, cols)))
        return st;
    if (col_out && (st = check_qtensor_out(col_out, cfg->grid, rows)))
        return st;
    if (reinterpret_cast<uintptr_t>(x) % 2)
        return MXQ_ERR_ALIGN;
    // grid-size limits of the launches (2^31 workgroups / 65535 row tiles)
    if (col_out && (rows + 127) / 128 > 65535)
        return MXQ_ERR_SHAPE;
    return MXQ_OK;
}

OutDesc col_desc(const mxq_qtensor *col_out, int64_t rows, int64_t cols)
{
    return OutDesc{static_cast<uint8_t *>(col_out->codes), col_out->scales, col_out->fmt,
                   col_out->layout, (uint64_t)(rows / 32), (uint64_t)((cols + 15) / 16)};
}

// kernels come in two grid families: E1M2, and E2M1 with or without a cap
// (the cap and the scale exponent travel in the knobs)
int grid_family(const mxq_qconfig *cfg) { return cfg->grid == MXQ_GRID_E1M2 ? kE1M2 : kE2M1; }

// 8-byte loads of the column kernels when x and its rows are 8-byte aligned
int col_vec(const void *x, int64_t ld_x)
{
    return (reinterpret_cast<uintptr_t>(x) % 8 == 0 && ld_x % 4 == 0) ? 1 : 0;
}

// The launches of one checked mxq_quantize call.
mxq_status enqueue_quantize(const mxq_qconfig *cfg, const void *x, int64_t rows, int64_t cols,
                            int64_t ld_x, const mxq_qtensor *row_out, const mxq_qtensor *col_out,
                            hipStream_t s)
{
    if (rows == 0 || cols == 0)
        return MXQ_OK;
    OutDesc rout{}, cout{};
    if (row_out)
        rout = OutDesc{static_cast<uint8_t *>(row_out->codes), row_out->scales, row_out->fmt,
                       row_out->layout, (uint64_t)(cols / 32), (uint64_t)((rows + 15) / 16)};
    if (col_out)
        cout = col_desc(col_out, rows, cols);
    const uint16_t *xx = static_cast<const uint16_t *>(x);
    const uintptr_t xa = reinterpret_cast<uintptr_t>(x);
    const QKnobs kn = make_knobs(cfg);
    const int fam = grid_family(cfg);
    hipError_t e;
    if (!col_out) {
        // blocks along the contiguous dimension: 16-byte loads when aligned
        const uint64_t nbr = (uint64_t)cols / 32;
        RowLaunch r{xx, (uint64_t)rows * nbr, (uint32_t)nbr, ld_x, ld_x == cols ? 1 : 0,
                    (xa % 16 == 0 && ld_x % 8 == 0) ? 1 : 0, rout, kn, s};
        e = launch_quant_row16(fam, cfg->round, cfg->hadamard_n, r);
    } else {
        // blocks along rows (alone or with the row output): 8-byte loads when aligned
        const int vec8 = col_vec(x, ld_x);
        if (!row_out) {
            ColLaunch c{xx, rows, cols, ld_x, cout, vec8, kn, s};
            e = launch_quant_col(fam, cfg->round, cfg->hadamard_n, c);
        } else {
            DualLaunch d{xx, rows, cols, ld_x, rout, cout, vec8, kn, s};
            e = launch_quant_dual16(fam, cfg->round, cfg->hadamard_n, d);
        }
    }
    return e == hipSuccess ? MXQ_OK : MXQ_ERR_DEVICE;
}

// 128 x 128 tiles of a column job
int64_t col_tiles(const mxq_quantize_job &j) { return ((j.cols + 127) / 128) * ((j.rows + 127) / 128); }

// the most workgroups one 1-D launch of 256-lane workgroups may have
constexpr int64_t kMaxBatchTiles = (int64_t)0xFFFFFFFF / 256;

// Jobs that the batched column kernel can share a launch with: a column
// output only, something to do, and few enough tiles for a 1-D launch.
bool col_only(const mxq_quantize_job &j)
{
    return !j.row_out && j.col_out && j.rows > 0 && j.cols > 0 && col_tiles(j) <= kMaxBatchTiles;
}

bool same_col_kernel(const mxq_quantize_job &a, const mxq_quantize_job &b)
{
    return grid_family(a.cfg) == grid_family(b.cfg) && a.cfg->hadamard_n == b.cfg->hadamard_n &&
           a.col_out->fmt == b.col_out->fmt;
}

}  // namespace

}  // namespace mxq

using namespace mxq;

extern "C" mxq_status mxq_quantize(const mxq_qconfig *cfg, const void *x, int64_t rows,
                                   int64_t cols, int64_t ld_x, const mxq_qtensor *row_out,
                                   const mxq_qtensor *col_out, void *stream)
{
    const mxq_status st = check_quantize(cfg, x, rows, cols, ld_x, row_out, col_out);
    if (st)
        return st;
    return enqueue_quantize(cfg, x, rows, cols, ld_x, row_out, col_out,
                            static_cast<hipStream_t>(stream));
}

extern "C" mxq_status mxq_quantize_batch(const mxq_quantize_job *jobs, int32_t count, void *stream)
{
    if (count < 0)
        return MXQ_ERR_SHAPE;
    if (count == 0)
        return MXQ_OK;
    if (!jobs)
        return MXQ_ERR_NULL;
    for (int32_t i = 0; i < count; ++i) {
        const mxq_quantize_job &j = jobs[i];
        const mxq_status st =
            check_quantize(j.cfg, j.x, j.rows, j.cols, j.ld_x, j.row_out, j.col_out);
        if (st)
            return st;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int32_t i = 0; i < count;) {
        const mxq_quantize_job &j0 = jobs[i];
        if (!col_only(j0)) {
            const mxq_status st = enqueue_quantize(j0.cfg, j0.x, j0.rows, j0.cols, j0.ld_x,
                                                   j0.row_out, j0.col_out, s);
            if (st)
                return st;
            ++i;
            continue;
        }
        // a run of consecutive column-only jobs that share one kernel
        ColBatch b{};
        int64_t tiles = 0;
        int32_t n = 0;
        while (i + n < count && n < kColBatchMax && col_only(jobs[i + n]) &&
               same_col_kernel(j0, jobs[i + n]) && tiles + col_tiles(jobs[i + n]) <= kMaxBatchTiles) {
            const mxq_quantize_job &j = jobs[i + n];
            ColJob &q = b.job[n];
            q.x = static_cast<const uint16_t *>(j.x);
            q.rows = j.rows;
            q.cols = j.cols;
            q.ld = j.ld_x;
            q.out = col_desc(j.col_out, j.rows, j.cols);
            q.kn = make_knobs(j.cfg);
            q.first = tiles;
            q.gx = (j.cols + 127) / 128;
            q.vec = col_vec(j.x, j.ld_x);
            q.round = j.cfg->round == MXQ_ROUND_SR ? kSR : kRTNE;
            tiles += col_tiles(j);
            ++n;
        }
        b.n = n;
        const hipError_t e = launch_quant_col_batch(grid_family(j0.cfg), j0.cfg->hadamard_n,
                                                    j0.col_out->fmt, b, tiles, s);
        if (e != hipSuccess)
            return MXQ_ERR_DEVICE;
        i += n;
    }
    return MXQ_OK;
}

extern "C" mxq_status mxq_round_to_grid(int32_t grid, int32_t round, int32_t sr_bits,
                                        const float *a, const uint16_t *rand, int64_t n,
                                        uint8_t *codes, void *stream)
{
    if (grid < MXQ_GRID_E2M1 || grid > MXQ_GRID_E2M1_MAX3 ||
        (round != MXQ_ROUND_RTNE && round != MXQ_ROUND_SR) ||
        (round == MXQ_ROUND_SR && sr_bits != 8 && sr_bits != 16))
        return MXQ_ERR_UNSUPPORTED;
    if (n < 0)
        return MXQ_ERR_SHAPE;
    if (n == 0)
        return MXQ_OK;
    if (!a || !codes || (round == MXQ_ROUND_SR && !rand))
        return MXQ_ERR_NULL;
    const int64_t threads = (n + 7) / 8;
    const dim3 g((unsigned)((threads + 255) / 256));
    hipStream_t s = static_cast<hipStream_t>(stream);
    // top level of the E2M1 family: 6, or the cap
    const float top = grid == MXQ_GRID_E2M1_MAX4 ? 4.0f : grid == MXQ_GRID_E2M1_MAX3 ? 3.0f : 6.0f;
    if (grid != MXQ_GRID_E1M2) {
        if (round == MXQ_ROUND_RTNE)
            hipLaunchKernelGGL((k_round_to_grid<kE2M1, kRTNE>), g, dim3(256), 0, s, a, rand, n, sr_bits, top, codes);
        else
            hipLaunchKernelGGL((k_round_to_grid<kE2M1, kSR>), g, dim3(256), 0, s, a, rand, n, sr_bits, top, codes);
    } else {
        if (round == MXQ_ROUND_RTNE)
            hipLaunchKernelGGL((k_round_to_grid<kE1M2, kRTNE>), g, dim3(256), 0, s, a, rand, n, sr_bits, top, codes);
        else
            hipLaunchKernelGGL((k_round_to_grid<kE1M2, kSR>), g, dim3(256), 0, s, a, rand, n, sr_bits, top, codes);
    }
    return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_DEVICE;
}
