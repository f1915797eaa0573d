// Reconstruction (mxq_dequantize) and the shrinkage-bias / SQNR statistics
// (mxq_bias_stats) of block-quantized tensors.  Support kernels of the
// quantizer, one pass each: the reconstruction is memory-bound; the
// statistics are bound by their fp64 terms.
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
//
// One lane takes whole 32-element blocks: it loads the block's bf16 values,
// applies the signs and the rotation in fp32 exactly as the method defines
// them (butterfly stages of stride 1, 2, 4, ... inside each n-sub-block, then
// the product with fl32(1/sqrt(n))), reads the block's codes and scale, and
// adds the block's fp64 terms to its own sums.
//  * Row axis: a work item is one block; neighbouring lanes take neighbouring
//    blocks, so both the 64-byte input runs and the code runs of a wave are
//    contiguous.
//  * Column axis: a work item is kColRun consecutive blocks of one column;
//    neighbouring lanes take neighbouring columns, so each of a block's 32
//    row loads reads one contiguous run across the wave, and a lane's codes
//    for the item are one contiguous run (128 bytes for FP4).
// The sums are then reduced in a fixed order (wave butterflies, the 4 waves
// in order, then a fixed tree over the workgroups), so results repeat bit
// for bit.

constexpr int kStatD = 14;   // doubles: 6 sums + 8 per-level error sums
constexpr int kStatU = 11;   // counts: n, n_sat, n_nonfinite_blocks, 8 per-level
constexpr int kStatN = kStatD + kStatU;
constexpr int kStatsMaxWG = 1024;
constexpr int kColRun = 8;   // blocks per column work item

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

// y = fl32(1/sqrt(n)) H_n (D x) on each n-sub-block of the lane's block.
template <int HN>
__device__ __forceinline__ void rotate32(float (&v)[32])
{
    if constexpr (HN >= 16) {
#pragma unroll
        for (int h = 1; h < HN; h <<= 1) {
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                if (!(i & h)) {
                    const float a = v[i], b = v[i + h];
                    v[i] = a + b;
                    v[i + h] = a - b;
                }
            }
        }
        const float c = HN == 16 ? 0.25f : as_f(0x3E3504F3u);  // fl32(1/sqrt(n))
#pragma unroll
        for (int i = 0; i < 32; ++i)
            v[i] = v[i] * c;
    }
}

// The 32 nibbles of block b (element i at bits 4 (i % 8) of word i / 8).
// Codes are 4-byte aligned; an E2M3 block is six words, element i at bits
// 6i .. 6i + 5 of their little-endian concatenation.
__device__ __forceinline__ void load_nibbles32(const uint8_t *codes, int fmt, int grid, uint64_t b,
                                               uint32_t (&w)[4])
{
    if (fmt == MXQ_FMT_FP4) {
        const uint32_t *p = reinterpret_cast<const uint32_t *>(codes + b * 16);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            w[k] = p[k];
        return;
    }
    const uint32_t *p = reinterpret_cast<const uint32_t *>(codes + b * 24);
    uint32_t q[7];
#pragma unroll
    for (int k = 0; k < 6; ++k)
        q[k] = p[k];
    q[6] = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        w[k] = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const int o = 6 * i;
        const uint64_t pair = (uint64_t)q[o >> 5] | ((uint64_t)q[(o >> 5) + 1] << 32);
        const uint32_t c = (uint32_t)(pair >> (o & 31)) & 63u;
        w[i >> 3] |= nibble_of_e2m3(grid, c) << (4 * (i & 7));
    }
}

// Adds one block's terms: y its rotated values, sc its scale byte, w its
// nibbles, lut2 the grid's levels times 2 as 4-bit fields (level m = field m
// / 2).  Each term is the fp64 expression of the definition, computed
// exactly: for y != 0 the code carries y's sign, so sign(y) (yhat - y) =
// |yhat| - |y|, and for y = 0 both are 0.  The per-level error sums add
// G_m - a to level m's running sum, kept in the lane's own LDS slot `lvl +
// 256 m` by one LDS fp64 add per element: the slot receives exactly the
// matching terms in element order, as a register accumulator would, without
// the eight select-and-add steps per element that register sums need (24%
// faster, the same bytes).  The per-level counts go into a packed per-block
// histogram (8 bits per level, a block has 32 elements) that is unpacked once
// per block.
__device__ __forceinline__ void stat_block(StatAcc &acc, const float (&y)[32], uint32_t sc,
                                           const uint32_t (&w)[4], uint32_t lut2, double top,
                                           double *lvl)
{
    acc.u[2] += sc == 0xFFu ? 1u : 0u;   // non-finite blocks are counted, not summed
    if (sc == 0xFFu)
        return;
    const int e = (int)sc - 127;
    const double up = ldexp(1.0, e), down = ldexp(1.0, -e);   // exact powers of two
    uint32_t hist_lo = 0u, hist_hi = 0u;   // levels 0-3 and 4-7
    uint32_t nsat = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const uint32_t m = (w[i >> 3] >> (4 * (i & 7))) & 7u;
        const double ay = fabs((double)y[i]);
        const double g = 0.5 * (double)__builtin_amdgcn_ubfe(lut2, 4 * m, 4);
        const double t = g * up - ay;          // sign(y) (yhat - y)
        const double a = ay * down;
        const double dn = g - a;
        acc.d[0] += ay;
        acc.d[1] += t;
        acc.d[2] = __builtin_fma(ay, ay, acc.d[2]);
        acc.d[3] = __builtin_fma(t, t, acc.d[3]);
        acc.d[4] += dn;
        const bool sat = a > top;
        acc.d[5] += sat ? dn : 0.0;
        nsat += sat ? 1u : 0u;
        // the level's running sum: this lane's own LDS slot, added in element
        // order (a wave's LDS operations execute in order, so the slot sees
        // exactly the additions of a register accumulator, in the same order)
        __hip_atomic_fetch_add(lvl + 256 * m, dn, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const uint32_t inc = 1u << (8 * (m & 3u));
        hist_lo += m < 4u ? inc : 0u;
        hist_hi += m < 4u ? 0u : inc;
    }
    acc.u[0] += 32;
    // the block's count as one 32-bit value (left to itself the compiler adds
    // each element's 0 or 1 straight into the 64-bit sum)
    asm volatile("" : "+v"(nsat));
    acc.u[1] += nsat;
#pragma unroll
    for (int q = 0; q < 8; ++q)
        acc.u[3 + q] += ((q < 4 ? hist_lo : hist_hi) >> (8 * (q & 3))) & 0xFFu;
}

// The grid's 8 levels times 2, as 4-bit fields (E2M1: 0 1 2 3 4 6 8 12;
// E1M2: 0 .. 7); the capped E2M1 grids store E2M1 codes.
__device__ __forceinline__ uint32_t grid_lut2(int grid)
{
    return grid == MXQ_GRID_E1M2 ? 0x76543210u : 0xC8643210u;
}

__device__ __forceinline__ double grid_top(int grid)
{
    return grid == MXQ_GRID_E2M1 ? 6.0 : grid == MXQ_GRID_E1M2 ? 3.5
         : grid == MXQ_GRID_E2M1_MAX4 ? 4.0 : 3.0;
}

// The lane's per-level sums from its LDS slots into the accumulator (after
// its own last additions: the reads follow them in the wave's LDS order).
__device__ __forceinline__ void level_sums(StatAcc &acc, const double *lvl)
{
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int q = 0; q < 8; ++q)
        acc.d[6 + q] = __hip_atomic_load(lvl + 256 * q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Writes the workgroup's fixed-order sums to partial[blockIdx.x][kStatN]
// (counts as the bit patterns of doubles).
__device__ __forceinline__ void stats_flush(const StatAcc &acc, double *__restrict__ partial)
{
    __shared__ double sd[4][kStatD];
    __shared__ unsigned long long su[4][kStatU];
    const int t = threadIdx.x, wv = t >> 6, lane = t & 63;
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

__device__ __forceinline__ void stat_init(StatAcc &acc)
{
#pragma unroll
    for (int i = 0; i < kStatD; ++i)
        acc.d[i] = 0.0;
#pragma unroll
    for (int i = 0; i < kStatU; ++i)
        acc.u[i] = 0;
}

// Row axis: block b = line * nbk + jb, one per lane.  vec: x 16-byte
// aligned and ld % 8 == 0 (four 16-byte loads per block).
template <int HN>
__global__ __launch_bounds__(256) void k_stats_row(const uint16_t *__restrict__ x, int64_t lines,
                                                   int64_t nbk, int64_t ld, int vec,
                                                   const uint8_t *__restrict__ codes,
                                                   const uint8_t *__restrict__ scales, int fmt,
                                                   int grid, QKnobs kn, double *__restrict__ partial)
{
    const double top = grid_top(grid);
    const uint32_t lut2 = grid_lut2(grid);
    const uint64_t nblocks = (uint64_t)(lines * nbk);
    StatAcc acc;
    stat_init(acc);
    __shared__ double lvl_sh[8 * 256];                           // [level][thread]
    double *const lvl = lvl_sh + threadIdx.x;
#pragma unroll
    for (int q = 0; q < 8; ++q)
        lvl[256 * q] = 0.0;
    for (uint64_t b = (uint64_t)blockIdx.x * 256 + threadIdx.x; b < nblocks;
         b += (uint64_t)gridDim.x * 256) {
        const int64_t line = (int64_t)(b / (uint64_t)nbk), jb = (int64_t)b - line * nbk;
        const uint16_t *src = x + line * ld + jb * 32;
        uint32_t h[16];
        if (vec) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint4 q = reinterpret_cast<const uint4 *>(src)[k];
                h[4 * k] = q.x; h[4 * k + 1] = q.y; h[4 * k + 2] = q.z; h[4 * k + 3] = q.w;
            }
        } else {
#pragma unroll
            for (int k = 0; k < 16; ++k)
                h[k] = (uint32_t)src[2 * k] | ((uint32_t)src[2 * k + 1] << 16);
        }
        const uint32_t sg = block_signs<HN>(kn, (uint64_t)jb);
        float v[32];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            v[2 * k] = as_f((h[k] << 16) ^ (((sg >> (2 * k)) & 1u) << 31));
            v[2 * k + 1] = as_f((h[k] & 0xFFFF0000u) ^ (((sg >> (2 * k + 1)) & 1u) << 31));
        }
        rotate32<HN>(v);
        uint32_t w[4];
        load_nibbles32(codes, fmt, grid, b, w);
        stat_block(acc, v, scales[b], w, lut2, top, lvl);
    }
    level_sums(acc, lvl);
    stats_flush(acc, partial);
}

// Column axis: work item it = c + cols * gq covers blocks kColRun gq ..
// kColRun gq + kColRun - 1 of column c (line c; block index c * nbk + jb).
template <int HN>
__global__ __launch_bounds__(256) void k_stats_col(const uint16_t *__restrict__ x, int64_t cols,
                                                   int64_t nbk, int64_t ld,
                                                   const uint8_t *__restrict__ codes,
                                                   const uint8_t *__restrict__ scales, int fmt,
                                                   int grid, QKnobs kn, double *__restrict__ partial)
{
    const double top = grid_top(grid);
    const uint32_t lut2 = grid_lut2(grid);
    const int64_t ngroups = (nbk + kColRun - 1) / kColRun;
    const uint64_t nitems = (uint64_t)(cols * ngroups);
    StatAcc acc;
    stat_init(acc);
    __shared__ double lvl_sh[8 * 256];                           // [level][thread]
    double *const lvl = lvl_sh + threadIdx.x;
#pragma unroll
    for (int q = 0; q < 8; ++q)
        lvl[256 * q] = 0.0;
    for (uint64_t it = (uint64_t)blockIdx.x * 256 + threadIdx.x; it < nitems;
         it += (uint64_t)gridDim.x * 256) {
        const int64_t gq = (int64_t)(it / (uint64_t)cols), c = (int64_t)it - gq * cols;
        const int64_t jend = min(nbk, (gq + 1) * kColRun);
        for (int64_t jb = gq * kColRun; jb < jend; ++jb) {
            const uint16_t *src = x + jb * 32 * ld + c;
            const uint32_t sg = block_signs<HN>(kn, (uint64_t)jb);
            float v[32];
#pragma unroll
            for (int i = 0; i < 32; ++i)
                v[i] = as_f(((uint32_t)src[i * ld] << 16) ^ (((sg >> i) & 1u) << 31));
            rotate32<HN>(v);
            const uint64_t b = (uint64_t)(c * nbk + jb);
            uint32_t w[4];
            load_nibbles32(codes, fmt, grid, b, w);
            stat_block(acc, v, scales[b], w, lut2, top, lvl);
        }
    }
    level_sums(acc, lvl);
    stats_flush(acc, partial);
}

// Sum of the nwg workgroup partials in a fixed order: thread t adds the
// partials t, t + 256, t + 512, t + 768 in that order, then a binary tree
// over the 256 threads (stride 128, 64, ..., 1) in LDS.
__global__ __launch_bounds__(256) void k_stats_final(const double *__restrict__ partial, int nwg,
                                                     mxq_stats *__restrict__ out)
{
    __shared__ double shd[kStatD][256];
    __shared__ unsigned long long shu[kStatU][256];
    const int t = threadIdx.x;
    double d[kStatD];
    unsigned long long u[kStatU];
#pragma unroll
    for (int i = 0; i < kStatD; ++i)
        d[i] = 0.0;
#pragma unroll
    for (int i = 0; i < kStatU; ++i)
        u[i] = 0;
#pragma unroll
    for (int r = 0; r < kStatsMaxWG / 256; ++r) {
        const int w = t + 256 * r;
        if (w < nwg) {
            const double *p = partial + (int64_t)w * kStatN;
#pragma unroll
            for (int i = 0; i < kStatD; ++i)
                d[i] += p[i];
#pragma unroll
            for (int i = 0; i < kStatU; ++i)
                u[i] += (unsigned long long)__double_as_longlong(p[kStatD + i]);
        }
    }
#pragma unroll
    for (int i = 0; i < kStatD; ++i)
        shd[i][t] = d[i];
#pragma unroll
    for (int i = 0; i < kStatU; ++i)
        shu[i][t] = u[i];
    __syncthreads();
    for (int st = 128; st >= 1; st >>= 1) {
        for (int idx = t; idx < kStatN * st; idx += 256) {
            const int i = idx / st, j = idx - i * st;
            if (i < kStatD)
                shd[i][j] += shd[i][j + st];
            else
                shu[i - kStatD][j] += shu[i - kStatD][j + st];
        }
        __syncthreads();
    }
    // layout of mxq_stats: 6 sums, level_err_norm[8], then n, n_saturated,
    // n_nonfinite_blocks, level_count[8]
    double *od = reinterpret_cast<double *>(out);
    unsigned long long *ou = reinterpret_cast<unsigned long long *>(&out->n);
    if (t < kStatD)
        od[t] = shd[t][0];
    else if (t < kStatN)
        ou[t - kStatD] = shu[t - kStatD][0];
}

namespace {
// Work items of the statistics kernel: blocks (row axis) or runs of kColRun
// blocks of one column (column axis).
int64_t stats_items(int64_t rows, int64_t cols, int32_t axis)
{
    if (axis == MXQ_AXIS_ROW)
        return rows * (cols / 32);
    return cols * ((rows / 32 + kColRun - 1) / kColRun);
}

int stats_grid(int64_t items)
{
    int64_t g = (items + 255) / 256;
    if (g > kStatsMaxWG)
        g = kStatsMaxWG;
    if (g < 1)
        g = 1;
    return (int)g;
}

template <int HN>
hipError_t launch_stats_hn(const mxq_qconfig *cfg, const uint16_t *x, int64_t rows, int64_t cols,
                           int64_t ld, int32_t axis, const mxq_qtensor *q, double *part, int nwg,
                           hipStream_t s)
{
    const QKnobs kn = make_knobs(cfg);
    const uint8_t *codes = static_cast<const uint8_t *>(q->codes);
    if (axis == MXQ_AXIS_ROW) {
        const int vec = reinterpret_cast<uintptr_t>(x) % 16 == 0 && ld % 8 == 0;
        hipLaunchKernelGGL(k_stats_row<HN>, dim3(nwg), dim3(256), 0, s, x, rows, cols / 32, ld, vec,
                           codes, q->scales, q->fmt, q->grid, kn, part);
    } else {
        hipLaunchKernelGGL(k_stats_col<HN>, dim3(nwg), dim3(256), 0, s, x, cols, rows / 32, ld,
                           codes, q->scales, q->fmt, q->grid, kn, part);
    }
    return hipGetLastError();
}
}  // namespace

// The statistics kernels and the final reduction into `out`, with the
// workgroup partials in `part` (stats_grid(...) x kStatN doubles; every slot
// the reduction reads is written first, so `part` needs no clearing).
mxq_status launch_stats(const mxq_qconfig *cfg, const void *x, int64_t rows, int64_t cols,
                        int64_t ld_x, int32_t axis, const mxq_qtensor *q, mxq_stats *out,
                        double *part, hipStream_t s)
{
    const int nwg = stats_grid(stats_items(rows, cols, axis));
    const uint16_t *xx = static_cast<const uint16_t *>(x);
    hipError_t e;
    switch (cfg->hadamard_n) {
    case 0:
        e = launch_stats_hn<0>(cfg, xx, rows, cols, ld_x, axis, q, part, nwg, s);
        break;
    case 16:
        e = launch_stats_hn<16>(cfg, xx, rows, cols, ld_x, axis, q, part, nwg, s);
        break;
    default:
        e = launch_stats_hn<32>(cfg, xx, rows, cols, ld_x, axis, q, part, nwg, s);
        break;
    }
    if (e != hipSuccess)
        return MXQ_ERR_DEVICE;
    hipLaunchKernelGGL(k_stats_final, dim3(1), dim3(256), 0, s, part, nwg, out);
    return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_DEVICE;
}

// The argument checks of mxq_bias_stats other than the workspace's.
mxq_status check_stats(const mxq_qconfig *cfg, const void *x, int64_t rows, int64_t cols,
                       int64_t ld_x, int32_t axis, const mxq_qtensor *q, const mxq_stats *out)
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
    if (reinterpret_cast<uintptr_t>(q->codes) % 4 || reinterpret_cast<uintptr_t>(out) % 8 ||
        reinterpret_cast<uintptr_t>(x) % 2)
        return MXQ_ERR_ALIGN;
    return MXQ_OK;
}

size_t stats_workspace_bytes(int64_t rows, int64_t cols, int32_t axis)
{
    if (rows < 0 || cols < 0)
        return 0;
    return (size_t)stats_grid(stats_items(rows, cols, axis)) * kStatN * sizeof(double);
}

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
    return stats_workspace_bytes(rows, cols, axis);
}

extern "C" mxq_status mxq_bias_stats(const mxq_qconfig *cfg, const void *x, int64_t rows,
                                     int64_t cols, int64_t ld_x, int32_t axis, const mxq_qtensor *q,
                                     mxq_stats *out, void *workspace, size_t ws_bytes, void *stream)
{
    const mxq_status st = check_stats(cfg, x, rows, cols, ld_x, axis, q, out);
    if (st)
        return st;
    if (!workspace || ws_bytes < stats_workspace_bytes(rows, cols, axis))
        return MXQ_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % 8)
        return MXQ_ERR_ALIGN;
    return launch_stats(cfg, x, rows, cols, ld_x, axis, q, out, static_cast<double *>(workspace),
                        static_cast<hipStream_t>(stream));
}
