// Reconstruction (mxq_dequantize) and the shrinkage-bias / SQNR statistics
// (mxq_bias_stats) of block-quantized tensors.  Support kernels of the
// quantizer: memory-bound, one pass, no tuning beyond coalesced access.
//
// Reconstruction yhat = (-1)^s G_m 2^e follows the shared-exponent format of
// the htx.com news "Pretraining large language models with MXFP4", section
// "Que es MXFP4?".  The statistics are the diagnostics of the gist.science
// summary "Repensando o Vies de Encolhimento (Shrinkage Bias) no
// Pre-treinamento de LLMs em FP4": the signed error in normalized magnitude
// space of "Metodologia 1" and the SQNR of "Resultados Experimentais".
#include "mxq_device.hpp"
#include "mxq_host.hpp"

namespace mxq {

// Level magnitude of the 3-bit code m (E2M1: 0, .5, 1, 1.5, 2, 3, 4, 6; E1M2: m/2).
__device__ __forceinline__ float level_of(int grid, uint32_t m)
{
    if (grid == MXQ_GRID_E1M2)
        return 0.5f * (float)m;
    // E2M1 bit fields: exponent e = m >> 1 (bias 1), mantissa bit m & 1
    const uint32_t e = m >> 1, f = m & 1u;
    return e == 0 ? 0.5f * (float)f : ldexpf(1.0f + 0.5f * (float)f, (int)e - 1);
}

// Signed value of an FP6 E2M3 code (bias 1, 3 mantissa bits).
__device__ __forceinline__ float e2m3_value(uint32_t c)
{
    const uint32_t e = (c >> 3) & 3u, m = c & 7u;
    const float mag = e == 0 ? ldexpf((float)m, -3) : ldexpf((float)(8u + m), (int)e - 4);
    return (c & 32u) ? -mag : mag;
}

// Nibble (sign<<3 | m) of an E2M3 code holding a level of `grid`.
__device__ __forceinline__ uint32_t nibble_of_e2m3(int grid, uint32_t c)
{
    const uint32_t s = (c >> 2) & 8u, mag = c & 31u;
    uint32_t m;
    if (grid != MXQ_GRID_E1M2)
        m = mag >> 2;
    else
        m = mag < 16u ? (mag >> 2) : ((mag - 8u) >> 1);
    return s | m;
}

// The 8 elements 8*pos .. 8*pos+7 of block b, as nibbles.
__device__ __forceinline__ uint32_t load_nibbles8(const uint8_t *codes, int fmt, int grid,
                                                  uint64_t b, int pos)
{
    if (fmt == MXQ_FMT_FP4)
        return *reinterpret_cast<const uint32_t *>(codes + b * 16 + 4 * pos);
    const uint8_t *p = codes + b * 24 + 6 * pos;
    const uint64_t bits = (uint64_t)p[0] | ((uint64_t)p[1] << 8) | ((uint64_t)p[2] << 16) |
                          ((uint64_t)p[3] << 24) | ((uint64_t)p[4] << 32) | ((uint64_t)p[5] << 40);
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        w |= nibble_of_e2m3(grid, (uint32_t)(bits >> (6 * i)) & 63u) << (4 * i);
    return w;
}

// Block (line, jb) -> its block index in the code array and its scale byte
// offset, for both layouts (see MXQ_LAYOUT_MFMA in mxq.h).
__device__ __forceinline__ void block_place(int layout, int64_t line, int64_t jb, int64_t nbk,
                                            int64_t ntiles, uint64_t *cblk, uint64_t *soff)
{
    if (layout == MXQ_LAYOUT_ROWS) {
        *cblk = (uint64_t)(line * nbk + jb);
        *soff = *cblk;
    } else {
        const uint64_t lane = 16 * (uint64_t)(jb & 3) + (uint64_t)(line & 15);
        *cblk = ((uint64_t)(jb >> 2) * ntiles + (uint64_t)(line >> 4)) * 64 + lane;
        *soff = (((uint64_t)(jb >> 4) * ntiles + (uint64_t)(line >> 4)) * 64 + lane) * 4 +
                (uint64_t)((jb >> 2) & 3);
    }
}

__global__ __launch_bounds__(256) void k_dequant(const uint8_t *__restrict__ codes,
                                                 const uint8_t *__restrict__ scales, int fmt,
                                                 int grid, int layout, int64_t lines, int64_t nbk,
                                                 int out_bf16, void *__restrict__ out, int64_t ld_out)
{
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t b = gid >> 2;
    const int pos = (int)(gid & 3);
    if (b >= lines * nbk)
        return;
    const int64_t line = b / nbk, jb = b - line * nbk;
    uint64_t cblk, soff;
    block_place(layout, line, jb, nbk, (lines + 15) / 16, &cblk, &soff);
    const uint32_t sc = scales[soff];
    const uint32_t w = load_nibbles8(codes, fmt, grid, cblk, pos);
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t nib = (w >> (4 * i)) & 15u;
        float mag = sc == 0xFFu ? __builtin_nanf("") : ldexpf(level_of(grid, nib & 7u), (int)sc - 127);
        v[i] = (nib & 8u) ? -mag : mag;
    }
    const int64_t off = line * ld_out + jb * 32 + 8 * pos;
    if (out_bf16) {
        // every reconstructed value has <= 3 significant bits: truncation is exact
        uint32_t h[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            h[k] = (as_u(v[2 * k]) >> 16) | (as_u(v[2 * k + 1]) & 0xFFFF0000u);
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(out) + off) = make_uint4(h[0], h[1], h[2], h[3]);
    } else {
        float *o = static_cast<float *>(out) + off;
        *reinterpret_cast<float4 *>(o) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4 *>(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
}

// ---- statistics --------------------------------------------------------------

constexpr int kStatD = 14;   // doubles: 6 sums + 8 per-level error sums
constexpr int kStatU = 11;   // counts: n, n_sat, n_nonfinite_blocks, 8 per-level
constexpr int kStatN = kStatD + kStatU;
constexpr int kStatsMaxWG = 1024;

struct StatAcc {
    double d[kStatD];
    unsigned long long u[kStatU];
};

__device__ __forceinline__ double wave_sum(double x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        x += __shfl_xor(x, o, 64);
    return x;
}
__device__ __forceinline__ unsigned long long wave_sum(unsigned long long x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        x += __shfl_xor(x, o, 64);
    return x;
}

template <int HN>
__global__ __launch_bounds__(256) void k_stats(const uint16_t *__restrict__ x, int64_t rows,
                                               int64_t cols, int64_t ld, int axis,
                                               const uint8_t *__restrict__ codes,
                                               const uint8_t *__restrict__ scales, int fmt, int grid,
                                               QKnobs kn, double *__restrict__ partial)
{
    const int t = threadIdx.x, pos = t & 3;
    const int64_t lines = axis == MXQ_AXIS_ROW ? rows : cols;
    const int64_t k = axis == MXQ_AXIS_ROW ? cols : rows;
    const int64_t nbk = k / 32;
    const uint64_t nblocks = (uint64_t)(lines * nbk);
    const float top = grid == MXQ_GRID_E2M1 ? 6.0f
                      : grid == MXQ_GRID_E1M2 ? 3.5f
                      : grid == MXQ_GRID_E2M1_MAX4 ? 4.0f : 3.0f;
    const int emax = grid == MXQ_GRID_E2M1 ? 2 : 1;

    StatAcc acc;
#pragma unroll
    for (int i = 0; i < kStatD; ++i)
        acc.d[i] = 0.0;
#pragma unroll
    for (int i = 0; i < kStatU; ++i)
        acc.u[i] = 0;

    for (uint64_t base = (uint64_t)blockIdx.x * 64; base < nblocks; base += (uint64_t)gridDim.x * 64) {
        const uint64_t b = base + (uint64_t)(t >> 2);
        const bool valid = b < nblocks;
        float v[8];
        const int64_t line = valid ? (int64_t)(b / (uint64_t)nbk) : 0;
        const int64_t jb = valid ? (int64_t)b - line * nbk : 0;
        const uint32_t sg = (block_signs<HN>(kn, (uint64_t)jb) >> (8 * pos)) & 0xFFu;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t h = 0;
            if (valid) {
                const int64_t off = axis == MXQ_AXIS_ROW ? line * ld + jb * 32 + 8 * pos + i
                                                         : (jb * 32 + 8 * pos + i) * ld + line;
                h = x[off];
            }
            v[i] = as_f((h << 16) ^ (((sg >> i) & 1u) << 31));
        }
        rotate8<HN, 1, 2>(v, pos);
        if (!valid)
            continue;
        const uint32_t sc = scales[b];
        if (sc == 0xFFu) {
            if (pos == 0)
                acc.u[2] += 1;
            continue;
        }
        const uint32_t w = load_nibbles8(codes, fmt, grid, b, pos);
        const int e = (int)sc - 127;
        (void)emax;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t nib = (w >> (4 * i)) & 15u, m = nib & 7u;
            const double y = (double)v[i];
            const double g = (double)level_of(grid, m);
            double yh = ldexp(g, e);
            if (nib & 8u)
                yh = -yh;
            const double a = ldexp(fabs(y), -e);
            const double sgn = y < 0 ? -1.0 : (y > 0 ? 1.0 : 0.0);
            const double err = yh - y;
            acc.d[0] += fabs(y);
            acc.d[1] += sgn * err;
            acc.d[2] += y * y;
            acc.d[3] += err * err;
            acc.d[4] += g - a;
            if (a > (double)top) {
                acc.d[5] += g - a;
                acc.u[1] += 1;
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                if (m == (uint32_t)q) {
                    acc.d[6 + q] += g - a;
                    acc.u[3 + q] += 1;
                }
            }
            acc.u[0] += 1;
        }
    }
    // fixed-order reduction: wave butterflies, then the 4 waves in order
    __shared__ double sd[4][kStatD];
    __shared__ unsigned long long su[4][kStatU];
    const int wv = t >> 6, lane = t & 63;
#pragma unroll
    for (int i = 0; i < kStatD; ++i) {
        const double s = wave_sum(acc.d[i]);
        if (lane == 0)
            sd[wv][i] = s;
    }
#pragma unroll
    for (int i = 0; i < kStatU; ++i) {
        const unsigned long long s = wave_sum(acc.u[i]);
        if (lane == 0)
            su[wv][i] = s;
    }
    __syncthreads();
    if (t < kStatD) {
        partial[(int64_t)blockIdx.x * kStatN + t] = ((sd[0][t] + sd[1][t]) + sd[2][t]) + sd[3][t];
    } else if (t < kStatN) {
        const int i = t - kStatD;
        const unsigned long long s = su[0][i] + su[1][i] + su[2][i] + su[3][i];
        partial[(int64_t)blockIdx.x * kStatN + t] = __longlong_as_double((long long)s);
    }
}

__global__ __launch_bounds__(256) void k_stats_final(const double *__restrict__ partial, int nwg,
                                                     mxq_stats *__restrict__ out)
{
    const int t = threadIdx.x;
    if (t >= kStatN)
        return;
    double sd = 0.0;
    unsigned long long su = 0;
    for (int w = 0; w < nwg; ++w) {
        const double v = partial[(int64_t)w * kStatN + t];
        if (t < kStatD)
            sd += v;
        else
            su += (unsigned long long)__double_as_longlong(v);
    }
    double *od = reinterpret_cast<double *>(out);
    unsigned long long *ou = reinterpret_cast<unsigned long long *>(&out->n);
    // layout of mxq_stats: 6 sums, level_err_norm[8], then n, n_saturated,
    // n_nonfinite_blocks, level_count[8]
    if (t < kStatD)
        od[t] = sd;
    else
        ou[t - kStatD] = su;
}

namespace {
int stats_grid(int64_t nblocks)
{
    int64_t g = (nblocks + 63) / 64;
    if (g > kStatsMaxWG)
        g = kStatsMaxWG;
    if (g < 1)
        g = 1;
    return (int)g;
}
}  // namespace

}  // namespace mxq

using namespace mxq;

static_assert(sizeof(mxq_stats) == kStatN * 8, "mxq_stats layout");

extern "C" mxq_status mxq_dequantize(const mxq_qtensor *q, int64_t lines, int64_t k,
                                     int32_t out_dtype, void *out, int64_t ld_out, void *stream)
{
    if (!q || !out || !q->codes || !q->scales)
        return MXQ_ERR_NULL;
    if (q->fmt != MXQ_FMT_FP4 && q->fmt != MXQ_FMT_E2M3)
        return MXQ_ERR_UNSUPPORTED;
    if (q->grid < MXQ_GRID_E2M1 || q->grid > MXQ_GRID_E2M1_MAX3)
        return MXQ_ERR_UNSUPPORTED;
    if (out_dtype != MXQ_OUT_F32 && out_dtype != MXQ_OUT_BF16)
        return MXQ_ERR_UNSUPPORTED;
    if (q->layout != MXQ_LAYOUT_ROWS && q->layout != MXQ_LAYOUT_MFMA)
        return MXQ_ERR_UNSUPPORTED;
    if (lines < 0 || k < 0 || k % 32 || ld_out < k)
        return MXQ_ERR_SHAPE;
    if (q->layout == MXQ_LAYOUT_MFMA && k % 128)
        return MXQ_ERR_SHAPE;
    const int esz = out_dtype == MXQ_OUT_F32 ? 4 : 2;
    if (reinterpret_cast<uintptr_t>(out) % 16 || (ld_out * esz) % 16 ||
        reinterpret_cast<uintptr_t>(q->codes) % 4)
        return MXQ_ERR_ALIGN;
    if (lines == 0 || k == 0)
        return MXQ_OK;
    const int64_t threads = lines * (k / 32) * 4;
    hipLaunchKernelGGL(k_dequant, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint8_t *>(q->codes),
                       q->scales, q->fmt, q->grid, q->layout, lines, k / 32,
                       (int)(out_dtype == MXQ_OUT_BF16), out, ld_out);
    return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_DEVICE;
}

extern "C" size_t mxq_bias_stats_workspace_size(int64_t rows, int64_t cols, int32_t axis)
{
    if (rows < 0 || cols < 0)
        return 0;
    const int64_t lines = axis == MXQ_AXIS_ROW ? rows : cols;
    const int64_t k = axis == MXQ_AXIS_ROW ? cols : rows;
    return (size_t)stats_grid(lines * (k / 32)) * kStatN * sizeof(double);
}

extern "C" mxq_status mxq_bias_stats(const mxq_qconfig *cfg, const void *x, int64_t rows,
                                     int64_t cols, int64_t ld_x, int32_t axis, const mxq_qtensor *q,
                                     mxq_stats *out, void *workspace, size_t ws_bytes, void *stream)
{
    mxq_status st = check_qconfig(cfg);
    if (st)
        return st;
    if (!x || !q || !out || !q->codes || !q->scales)
        return MXQ_ERR_NULL;
    if (axis != MXQ_AXIS_ROW && axis != MXQ_AXIS_COL)
        return MXQ_ERR_UNSUPPORTED;
    if (q->fmt != MXQ_FMT_FP4 && q->fmt != MXQ_FMT_E2M3)
        return MXQ_ERR_UNSUPPORTED;
    if (q->grid != cfg->grid || q->layout != MXQ_LAYOUT_ROWS)
        return MXQ_ERR_UNSUPPORTED;
    if (rows < 0 || cols < 0 || ld_x < cols)
        return MXQ_ERR_SHAPE;
    if ((axis == MXQ_AXIS_ROW && cols % 32) || (axis == MXQ_AXIS_COL && rows % 32))
        return MXQ_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(q->codes) % 4 || reinterpret_cast<uintptr_t>(out) % 8)
        return MXQ_ERR_ALIGN;
    if (!workspace || ws_bytes < mxq_bias_stats_workspace_size(rows, cols, axis))
        return MXQ_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % 8)
        return MXQ_ERR_ALIGN;
    const int64_t lines = axis == MXQ_AXIS_ROW ? rows : cols;
    const int64_t k = axis == MXQ_AXIS_ROW ? cols : rows;
    const int nwg = stats_grid(lines * (k / 32));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const QKnobs kn = make_knobs(cfg);
    double *part = static_cast<double *>(workspace);
    const uint8_t *codes = static_cast<const uint8_t *>(q->codes);
    const uint16_t *xx = static_cast<const uint16_t *>(x);
    switch (cfg->hadamard_n) {
    case 0:
        hipLaunchKernelGGL(k_stats<0>, dim3(nwg), dim3(256), 0, s, xx, rows, cols, ld_x, axis, codes,
                           q->scales, q->fmt, q->grid, kn, part);
        break;
    case 16:
        hipLaunchKernelGGL(k_stats<16>, dim3(nwg), dim3(256), 0, s, xx, rows, cols, ld_x, axis, codes,
                           q->scales, q->fmt, q->grid, kn, part);
        break;
    default:
        hipLaunchKernelGGL(k_stats<32>, dim3(nwg), dim3(256), 0, s, xx, rows, cols, ld_x, axis, codes,
                           q->scales, q->fmt, q->grid, kn, part);
        break;
    }
    if (hipGetLastError() != hipSuccess)
        return MXQ_ERR_DEVICE;
    hipLaunchKernelGGL(k_stats_final, dim3(1), dim3(256), 0, s, part, nwg, out);
    return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_DEVICE;
}
