// The block rotation on its own: y = fl32(1/sqrt(n)) H_n (D x) on every
// n-block along one axis, written in x's orientation as fp32 or bf16.  This is
// the first kernel of the unfused pipeline (rotate, write, read back,
// quantize) that the fused quantizer replaces -- the gist.science summary
// "Repensando o Vies de Encolhimento (Shrinkage Bias) no Pre-treinamento de
// LLMs em FP4", section "Eficiencia", measures the fused rotation against the
// plain quantizer and against the unfused pair.
//
// Same work layouts as the quantizers: along rows of x (blocks in the
// contiguous dimension) 4 lanes per 32-block with one 16-byte load each and
// DPP butterflies across the quad; along columns 16 positions x 4 columns per
// lane (sixteen 8-byte loads), the butterflies inside the lane.
#include "mxq_device.hpp"
#include "mxq_host.hpp"

namespace mxq {

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t bf16_rne(float f)
{
    const uint32_t u = as_u(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int HN, int OUT>
__global__ __launch_bounds__(256) void k_rotate_row(const uint16_t *__restrict__ x, int64_t rows,
                                                    int64_t cols, int64_t ld, int vec, QKnobs kn,
                                                    uint8_t *__restrict__ out, int64_t ldo, int vst)
{
    const int t = threadIdx.x, pos = t & 3;
    const int64_t nbr = cols / 32;
    const int64_t b = (int64_t)blockIdx.x * 64 + (t >> 2);   // 32-block index, row-major
    const bool valid = b < rows * nbr;
    const int64_t r = valid ? b / nbr : 0, jb = valid ? b - r * nbr : 0;
    const int64_t off = r * ld + jb * 32 + 8 * pos;
    uint32_t w[4] = {0, 0, 0, 0};
    if (valid) {
        if (vec) {
            const uint4 q = *reinterpret_cast<const uint4 *>(x + off);
            w[0] = q.x; w[1] = q.y; w[2] = q.z; w[3] = q.w;
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                w[k] = (uint32_t)x[off + 2 * k] | ((uint32_t)x[off + 2 * k + 1] << 16);
        }
    }
    const uint32_t sg = (block_signs<HN>(kn, (uint64_t)jb) >> (8 * pos)) & 0xFFu;
    float v[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        v[2 * k] = as_f((w[k] << 16) ^ (((sg >> (2 * k)) & 1u) << 31));
        v[2 * k + 1] = as_f((w[k] & 0xFFFF0000u) ^ (((sg >> (2 * k + 1)) & 1u) << 31));
    }
    rotate8<HN, 1, 2>(v, pos);                  // all 4 lanes of the block take part
    if (!valid)
        return;
    const int64_t o = r * ldo + jb * 32 + 8 * pos;
    if constexpr (OUT == MXQ_OUT_F32) {
        float *d = reinterpret_cast<float *>(out) + o;
        if (vst) {
            reinterpret_cast<float4 *>(d)[0] = make_float4(v[0], v[1], v[2], v[3]);
            reinterpret_cast<float4 *>(d)[1] = make_float4(v[4], v[5], v[6], v[7]);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k)
                d[k] = v[k];
        }
    } else {
        uint16_t *d = reinterpret_cast<uint16_t *>(out) + o;
        if (vst) {
            uint32_t p[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                p[k] = bf16_rne(v[2 * k]) | (bf16_rne(v[2 * k + 1]) << 16);
            *reinterpret_cast<uint4 *>(d) = make_uint4(p[0], p[1], p[2], p[3]);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k)
                d[k] = (uint16_t)bf16_rne(v[k]);
        }
    }
}

template <int HN, int OUT>
__global__ __launch_bounds__(256) void k_rotate_col(const uint16_t *__restrict__ x, int64_t rows,
                                                    int64_t cols, int64_t ld, int vec, QKnobs kn,
                                                    uint8_t *__restrict__ out, int64_t ldo, int vst)
{
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int pos = lane & 1, cg = lane >> 1;
    const int64_t rband = (int64_t)blockIdx.y * 128 + wv * 32;  // rows % 32 == 0
    if (rband >= rows)
        return;                                                   // whole wave
    const int64_t r0 = rband + 16 * pos;
    const int64_t c0 = (int64_t)blockIdx.x * 128 + 4 * cg;
    const bool full = c0 + 4 <= cols;
    uint32_t lo[16], hi[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        if (vec && full) {
            const uint2 q = *reinterpret_cast<const uint2 *>(x + (r0 + i) * ld + c0);
            lo[i] = q.x;
            hi[i] = q.y;
        } else {
            uint32_t h[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                h[j] = (c0 + j < cols) ? (uint32_t)x[(r0 + i) * ld + c0 + j] : 0u;
            lo[i] = h[0] | (h[1] << 16);
            hi[i] = h[2] | (h[3] << 16);
        }
    }
    const uint32_t sg = block_signs<HN>(kn, (uint64_t)(rband >> 5)) >> (16 * pos);
    const float c = HN == 16 ? 0.25f : as_f(0x3E3504F3u);
    float y[4][16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t wd = (j < 2) ? lo[i] : hi[i];
            const uint32_t bits = (j & 1) ? (wd & 0xFFFF0000u) : (wd << 16);
            y[j][i] = as_f(bits ^ (((sg >> i) & 1u) << 31));
        }
        rotate16_raw<HN>(y[j], pos);
#pragma unroll
        for (int i = 0; i < 16; ++i)
            y[j][i] = y[j][i] * c;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t o = (r0 + i) * ldo + c0;
        if constexpr (OUT == MXQ_OUT_F32) {
            float *d = reinterpret_cast<float *>(out) + o;
            if (full && vst) {
                *reinterpret_cast<float4 *>(d) = make_float4(y[0][i], y[1][i], y[2][i], y[3][i]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (c0 + j < cols)
                        d[j] = y[j][i];
            }
        } else {
            uint16_t *d = reinterpret_cast<uint16_t *>(out) + o;
            if (full && vst) {
                *reinterpret_cast<uint2 *>(d) =
                    make_uint2(bf16_rne(y[0][i]) | (bf16_rne(y[1][i]) << 16),
                               bf16_rne(y[2][i]) | (bf16_rne(y[3][i]) << 16));
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (c0 + j < cols)
                        d[j] = (uint16_t)bf16_rne(y[j][i]);
            }
        }
    }
}

namespace {

template <int HN, int OUT>
void launch_rotate(int32_t axis, const uint16_t *x, int64_t rows, int64_t cols, int64_t ld,
                   const QKnobs &kn, uint8_t *out, int64_t ldo, hipStream_t s)
{
    // vector stores need every row's output to keep their alignment
    constexpr int esz = OUT == MXQ_OUT_F32 ? 4 : 2;
    const int vst = (reinterpret_cast<uintptr_t>(out) % 16 == 0 && (ldo * esz) % 16 == 0) ? 1 : 0;
    if (axis == MXQ_AXIS_ROW) {
        const int vec = (reinterpret_cast<uintptr_t>(x) % 16 == 0 && ld % 8 == 0) ? 1 : 0;
        const int64_t nblocks = rows * (cols / 32);
        hipLaunchKernelGGL((k_rotate_row<HN, OUT>), dim3((unsigned)((nblocks + 63) / 64)),
                           dim3(256), 0, s, x, rows, cols, ld, vec, kn, out, ldo, vst);
    } else {
        const int vec = (reinterpret_cast<uintptr_t>(x) % 8 == 0 && ld % 4 == 0) ? 1 : 0;
        const dim3 grid((unsigned)((cols + 127) / 128), (unsigned)((rows + 127) / 128));
        hipLaunchKernelGGL((k_rotate_col<HN, OUT>), grid, dim3(256), 0, s, x, rows, cols, ld, vec,
                           kn, out, ldo, vst);
    }
}

}  // namespace

}  // namespace mxq

using namespace mxq;

extern "C" mxq_status mxq_rotate(const mxq_qconfig *cfg, const void *x, int64_t rows, int64_t cols,
                                 int64_t ld_x, int32_t axis, int32_t out_dtype, void *out,
                                 int64_t ld_out, void *stream)
{
    if (!cfg || !x || !out)
        return MXQ_ERR_NULL;
    if (cfg->hadamard_n != 16 && cfg->hadamard_n != 32)
        return MXQ_ERR_UNSUPPORTED;
    if (cfg->sign_mode != MXQ_SIGNS_MASK && cfg->sign_mode != MXQ_SIGNS_PER_BLOCK)
        return MXQ_ERR_UNSUPPORTED;
    if ((axis != MXQ_AXIS_ROW && axis != MXQ_AXIS_COL) ||
        (out_dtype != MXQ_OUT_F32 && out_dtype != MXQ_OUT_BF16))
        return MXQ_ERR_UNSUPPORTED;
    if (rows < 0 || cols < 0 || ld_x < cols || ld_out < cols)
        return MXQ_ERR_SHAPE;
    if ((axis == MXQ_AXIS_ROW && cols % 32) || (axis == MXQ_AXIS_COL && rows % 32))
        return MXQ_ERR_SHAPE;
    if (axis == MXQ_AXIS_COL && (rows + 127) / 128 > 65535)
        return MXQ_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(x) % 2 ||
        reinterpret_cast<uintptr_t>(out) % (out_dtype == MXQ_OUT_F32 ? 4 : 2))
        return MXQ_ERR_ALIGN;
    if (rows == 0 || cols == 0)
        return MXQ_OK;
    const uint16_t *xx = static_cast<const uint16_t *>(x);
    uint8_t *o = static_cast<uint8_t *>(out);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const QKnobs kn = make_knobs(cfg);
    if (cfg->hadamard_n == 16) {
        if (out_dtype == MXQ_OUT_F32)
            launch_rotate<16, MXQ_OUT_F32>(axis, xx, rows, cols, ld_x, kn, o, ld_out, s);
        else
            launch_rotate<16, MXQ_OUT_BF16>(axis, xx, rows, cols, ld_x, kn, o, ld_out, s);
    } else {
        if (out_dtype == MXQ_OUT_F32)
            launch_rotate<32, MXQ_OUT_F32>(axis, xx, rows, cols, ld_x, kn, o, ld_out, s);
        else
            launch_rotate<32, MXQ_OUT_BF16>(axis, xx, rows, cols, ld_x, kn, o, ld_out, s);
    }
    return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_DEVICE;
}
