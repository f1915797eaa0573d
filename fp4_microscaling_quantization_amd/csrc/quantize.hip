// Fused block-Hadamard rotation + MX block-32 quantization kernels (gfx950)
// and the host side of mxq_quantize / mxq_round_to_grid.
//
// k_quant_tile writes both outputs from one read: blocks along rows (written
// transposed) and blocks along the contiguous dimension.  (Calls asking for
// one output go to k_quant_row16 / k_quant_col, quantize_col.hip.)  Each lane
// loads an 8x8
//    bf16 tile (8 rows x 128-bit); a 16-lane DPP row covers 32x32, so the
//    4 lanes of a column block (xor 1, 2) and of a row block (xor 4, 8) are
//    both reachable by DPP without going through LDS.
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

// Widen 8 bf16 (one uint4) to fp32 and flip the signs whose bit is set in `sg`.
__device__ __forceinline__ void widen8(const uint4 &q, uint32_t sg, float (&v)[8])
{
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        v[2 * k] = as_f((w[k] << 16) ^ (((sg >> (2 * k)) & 1u) << 31));
        v[2 * k + 1] = as_f((w[k] & 0xFFFF0000u) ^ (((sg >> (2 * k + 1)) & 1u) << 31));
    }
}

// 8 consecutive bf16 through 2-byte loads (rows that are not 16-byte aligned).
__device__ __forceinline__ uint4 load8_scalar(const uint16_t *__restrict__ p)
{
    uint32_t h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        h[j] = p[j];
    return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                      h[6] | (h[7] << 16));
}

// Store this lane's slice of block (line, jb): FP4 4 bytes at 4*pos, or E2M3
// in pairs (the even lane writes 12 bytes for itself and its XP partner).
// All lanes of the block must call it (the E2M3 path exchanges by DPP).
template <int GRID, int XP>
__device__ __forceinline__ void store_slice(const OutDesc &o, uint64_t line, uint64_t jb, int pos,
                                            uint32_t w, uint32_t sc, bool valid)
{
    if (o.fmt == MXQ_FMT_FP4) {
        if (valid)
            *reinterpret_cast<uint32_t *>(o.codes + code_offset(o, line, jb, 16) + 4 * pos) = w;
    } else {
        const uint64_t own = e2m3_pack8<GRID>(w);
        const uint32_t lo = (uint32_t)own, hi = (uint32_t)(own >> 32);
        const uint32_t plo = lane_xor<XP>(lo), phi = lane_xor<XP>(hi);
        if (valid && !(pos & 1)) {
            uint32_t *d = reinterpret_cast<uint32_t *>(o.codes + code_offset(o, line, jb, 24) +
                                                       12 * (pos >> 1));
            d[0] = lo;
            d[1] = hi | (plo << 16);
            d[2] = (plo >> 16) | (phi << 16);
        }
    }
    if (valid && pos == 0)
        o.scales[scale_offset(o, line, jb)] = (uint8_t)sc;
}

template <int GRID, int ROUND, int HN, bool ROWS, bool COLS>
__global__ __launch_bounds__(256) void k_quant_tile(const uint16_t *__restrict__ x, int64_t rows,
                                                    int64_t cols, int64_t ld, OutDesc rout,
                                                    OutDesc cout, int vec, QKnobs kn)
{
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int g = lane >> 4, l16 = lane & 15, qr = l16 & 3, qc = l16 >> 2;
    const int64_t rband = (int64_t)blockIdx.y * 128 + wv * 32;  // rows % 32 == 0
    if (rband >= rows)
        return;                                                   // whole wave
    const int64_t r0 = rband + 8 * qr;
    const int64_t c0 = (int64_t)blockIdx.x * 128 + 32 * g + 8 * qc;

    uint4 raw[8];
    if (vec && c0 + 8 <= cols) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            raw[i] = *reinterpret_cast<const uint4 *>(x + (r0 + i) * ld + c0);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t h[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                h[j] = (c0 + j < cols) ? (uint32_t)x[(r0 + i) * ld + c0 + j] : 0u;
            raw[i] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                h[6] | (h[7] << 16));
        }
    }

    if constexpr (COLS) {
        // column blocks: rows rband .. rband+31 of column c0 + j
        const uint64_t nbc = (uint64_t)rows / 32, jb = (uint64_t)rband / 32;
        const uint32_t sg = HN ? (kn.sign_mask >> ((8 * qr) % (HN ? HN : 32))) & 0xFFu : 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t wd = (&raw[i].x)[j >> 1];
                const uint32_t bits = (j & 1) ? (wd & 0xFFFF0000u) : (wd << 16);
                v[i] = as_f(bits ^ (((sg >> i) & 1u) << 31));
            }
            const int64_t c = c0 + j;
            const uint64_t blk = (uint64_t)c * nbc + jb;
            uint32_t sc;
            const uint32_t w = quant8<GRID, ROUND, HN, 1, 2>(v, qr, blk, kn, &sc);
            store_slice<GRID, 1>(cout, (uint64_t)c, jb, qr, w, sc, c < cols);
        }
    }
    if constexpr (ROWS) {
        // row blocks: columns 32 g .. 32 g + 31 of the tile, row r0 + i
        const uint64_t nbr = (uint64_t)cols / 32;
        const uint64_t jb = ((uint64_t)blockIdx.x * 128 + 32 * g) / 32;
        const uint32_t sg = HN ? (kn.sign_mask >> ((8 * qc) % (HN ? HN : 32))) & 0xFFu : 0u;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float v[8];
            widen8(raw[i], sg, v);
            const uint64_t blk = (uint64_t)(r0 + i) * nbr + jb;
            uint32_t sc;
            const uint32_t w = quant8<GRID, ROUND, HN, 4, 8>(v, qc, blk, kn, &sc);
            store_slice<GRID, 4>(rout, (uint64_t)(r0 + i), jb, qc, w, sc, c0 < cols);
        }
    }
}

template <int GRID, int ROUND>
__global__ __launch_bounds__(256) void k_round_to_grid(const float *__restrict__ a,
                                                       const uint16_t *__restrict__ rnd, int64_t n,
                                                       int sr_bits, uint8_t *__restrict__ out)
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
    const uint32_t w = round8<GRID, ROUND>(v, 1.0f, r, sr_bits == 16 ? 131072.0f : 512.0f);
#pragma unroll
    for (int k = 0; k < 8; ++k)
        if (i0 + k < n)
            out[i0 + k] = (uint8_t)((w >> (4 * k)) & 15u);
}

// ---- host side ---------------------------------------------------------------

namespace {

struct QuantLaunch {
    const uint16_t *x;
    int64_t rows, cols, ld;
    bool has_row, has_col;
    OutDesc rout, cout;
    int vec;  // x 16-byte aligned and ld % 8 == 0: 128-bit loads
    QKnobs kn;
    hipStream_t s;
};

template <int GRID, int ROUND, int HN>
hipError_t launch_quant(const QuantLaunch &q)
{
    // both outputs from one read (row-only and column-only calls have kernels of their own)
    const dim3 grid((unsigned)((q.cols + 127) / 128), (unsigned)((q.rows + 127) / 128));
    hipLaunchKernelGGL((k_quant_tile<GRID, ROUND, HN, true, true>), grid, dim3(256), 0, q.s, q.x,
                       q.rows, q.cols, q.ld, q.rout, q.cout, q.vec, q.kn);
    return hipGetLastError();
}

template <int GRID, int ROUND>
hipError_t launch_quant_hn(int hn, const QuantLaunch &q)
{
    switch (hn) {
    case 0: return launch_quant<GRID, ROUND, 0>(q);
    case 16: return launch_quant<GRID, ROUND, 16>(q);
    default: return launch_quant<GRID, ROUND, 32>(q);
    }
}

}  // namespace

mxq_status check_qconfig(const mxq_qconfig *cfg)
{
    if (!cfg)
        return MXQ_ERR_NULL;
    if (cfg->grid != MXQ_GRID_E2M1 && cfg->grid != MXQ_GRID_E1M2)
        return MXQ_ERR_UNSUPPORTED;
    if (cfg->round != MXQ_ROUND_RTNE && cfg->round != MXQ_ROUND_SR)
        return MXQ_ERR_UNSUPPORTED;
    if (cfg->hadamard_n != 0 && cfg->hadamard_n != 16 && cfg->hadamard_n != 32)
        return MXQ_ERR_UNSUPPORTED;
    if (cfg->round == MXQ_ROUND_SR && cfg->sr_bits != 8 && cfg->sr_bits != 16)
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
    kn.sign_mask = cfg->hadamard_n == 16 ? (cfg->sign_mask & 0xFFFFu) : cfg->sign_mask;
    kn.seed_lo = (uint32_t)cfg->sr_seed;
    kn.seed_hi = (uint32_t)(cfg->sr_seed >> 32);
    kn.stream = cfg->sr_stream;
    kn.sr_bits = cfg->sr_bits == 8 ? 8u : 16u;
    return kn;
}

}  // namespace mxq

using namespace mxq;

extern "C" mxq_status mxq_quantize(const mxq_qconfig *cfg, const void *x, int64_t rows,
                                   int64_t cols, int64_t ld_x, const mxq_qtensor *row_out,
                                   const mxq_qtensor *col_out, void *stream)
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
    if (rows == 0 || cols == 0)
        return MXQ_OK;

    QuantLaunch q;
    q.x = static_cast<const uint16_t *>(x);
    q.rows = rows;
    q.cols = cols;
    q.ld = ld_x;
    q.has_row = row_out != nullptr;
    q.has_col = col_out != nullptr;
    q.rout = OutDesc{};
    q.cout = OutDesc{};
    if (row_out)
        q.rout = OutDesc{static_cast<uint8_t *>(row_out->codes), row_out->scales, row_out->fmt,
                         row_out->layout, (uint64_t)(cols / 32), (uint64_t)((rows + 15) / 16)};
    if (col_out)
        q.cout = OutDesc{static_cast<uint8_t *>(col_out->codes), col_out->scales, col_out->fmt,
                         col_out->layout, (uint64_t)(rows / 32), (uint64_t)((cols + 15) / 16)};
    q.vec = (reinterpret_cast<uintptr_t>(x) % 16 == 0 && ld_x % 8 == 0) ? 1 : 0;
    q.kn = make_knobs(cfg);
    q.s = static_cast<hipStream_t>(stream);

    hipError_t e;
    if (!col_out) {
        const uint64_t nbr = (uint64_t)cols / 32;
        RowLaunch r{q.x, (uint64_t)rows * nbr, (uint32_t)nbr, ld_x, ld_x == cols ? 1 : 0, q.vec,
                    q.rout, q.kn, q.s};
        e = launch_quant_row16(cfg->grid, cfg->round, cfg->hadamard_n, r);
    } else if (!row_out) {
        ColLaunch c{q.x, rows, cols, ld_x, q.cout,
                    (reinterpret_cast<uintptr_t>(x) % 8 == 0 && ld_x % 4 == 0) ? 1 : 0, q.kn, q.s};
        e = launch_quant_col(cfg->grid, cfg->round, cfg->hadamard_n, c);
    } else if (cfg->grid == MXQ_GRID_E2M1)
        e = cfg->round == MXQ_ROUND_RTNE ? launch_quant_hn<kE2M1, kRTNE>(cfg->hadamard_n, q)
                                         : launch_quant_hn<kE2M1, kSR>(cfg->hadamard_n, q);
    else
        e = cfg->round == MXQ_ROUND_RTNE ? launch_quant_hn<kE1M2, kRTNE>(cfg->hadamard_n, q)
                                         : launch_quant_hn<kE1M2, kSR>(cfg->hadamard_n, q);
    return e == hipSuccess ? MXQ_OK : MXQ_ERR_DEVICE;
}

extern "C" mxq_status mxq_round_to_grid(int32_t grid, int32_t round, int32_t sr_bits,
                                        const float *a, const uint16_t *rand, int64_t n,
                                        uint8_t *codes, void *stream)
{
    if ((grid != MXQ_GRID_E2M1 && grid != MXQ_GRID_E1M2) ||
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
    if (grid == MXQ_GRID_E2M1) {
        if (round == MXQ_ROUND_RTNE)
            hipLaunchKernelGGL((k_round_to_grid<kE2M1, kRTNE>), g, dim3(256), 0, s, a, rand, n, sr_bits, codes);
        else
            hipLaunchKernelGGL((k_round_to_grid<kE2M1, kSR>), g, dim3(256), 0, s, a, rand, n, sr_bits, codes);
    } else {
        if (round == MXQ_ROUND_RTNE)
            hipLaunchKernelGGL((k_round_to_grid<kE1M2, kRTNE>), g, dim3(256), 0, s, a, rand, n, sr_bits, codes);
        else
            hipLaunchKernelGGL((k_round_to_grid<kE1M2, kSR>), g, dim3(256), 0, s, a, rand, n, sr_bits, codes);
    }
    return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_DEVICE;
}
