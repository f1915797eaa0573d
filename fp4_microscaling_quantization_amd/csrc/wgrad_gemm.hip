// Block-scaled FP4 / FP6 weight-gradient GEMM on the gfx950 scaled matrix
// cores: C [m x n] = A [m x k] * B [n x k]^T, both operands MX-quantized
// along k (32-element blocks, one E8M0 scale each), fp32 accumulation.
//
// The product is the Wgrad GEMM dW = dY^T X of the htx.com news "Pretraining
// large language models with MXFP4" (section "Experimento de diagnostico"),
// with both operands quantized along the token axis; the pages run it on the
// MI355X's native FP4 matrix cores (gist.science summary "Pre-treinamento de
// Modelos de Linguagem Grandes com MXFP4", "Metodologia").
//
// v_mfma_scale_f32_16x16x128_f8f6f4: lane l supplies row (l % 16) of its
// operand and 32 values (one whole MX block) for lane group g = l / 16; the
// product pairs lane group g / element t of A with the same of B, each side
// multiplied by its lane's E8M0 scale byte.  Which K block a lane group
// carries is free as long as A and B agree, so lane group g of K step s takes
// block 4 s + g.  Output: lane l holds C rows 4 (l / 16) + r, r = 0..3, of
// column l % 16.
#include "mxq_device.hpp"
#include "mxq_host.hpp"

namespace mxq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

enum : int { kMfmaFP6 = 2, kMfmaFP4 = 4 };  // cbsz / blgp operand format codes

// One lane's 32 values of block b: 16 bytes (FP4) or 24 bytes (FP6).
template <int FMT>
__device__ __forceinline__ v8i load_operand(const uint8_t *__restrict__ codes, uint64_t b)
{
    v8i r = {0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (FMT == kMfmaFP4) {
        const uint4 q = *reinterpret_cast<const uint4 *>(codes + b * 16);
        r[0] = (int)q.x; r[1] = (int)q.y; r[2] = (int)q.z; r[3] = (int)q.w;
    } else {
        const uint2 *p = reinterpret_cast<const uint2 *>(codes + b * 24);
        const uint2 q0 = p[0], q1 = p[1], q2 = p[2];
        r[0] = (int)q0.x; r[1] = (int)q0.y; r[2] = (int)q1.x;
        r[3] = (int)q1.y; r[4] = (int)q2.x; r[5] = (int)q2.y;
    }
    return r;
}

constexpr int kTM = 128, kTN = 128;  // workgroup tile; 4 waves of 64 x 64

template <int FA, int FB>
__global__ __launch_bounds__(256) void k_wgrad_simple(const uint8_t *__restrict__ ac,
                                                      const uint8_t *__restrict__ as,
                                                      const uint8_t *__restrict__ bc,
                                                      const uint8_t *__restrict__ bs, int64_t m,
                                                      int64_t n, int64_t k, float *__restrict__ c,
                                                      int64_t ldc)
{
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int g = lane >> 4, li = lane & 15;
    const int64_t m0 = (int64_t)blockIdx.y * kTM + (wv >> 1) * 64;
    const int64_t n0 = (int64_t)blockIdx.x * kTN + (wv & 1) * 64;
    const int64_t nbk = k / 32;

    int64_t arow[4], brow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        arow[i] = min(m0 + 16 * i + li, m - 1);   // clamp ragged rows; stores are masked
        brow[i] = min(n0 + 16 * i + li, n - 1);
    }
    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

    for (int64_t s = 0; s < k / 128; ++s) {
        v8i a[4], b[4];
        int sa[4], sb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint64_t ba = (uint64_t)(arow[i] * nbk + 4 * s + g);
            const uint64_t bb = (uint64_t)(brow[i] * nbk + 4 * s + g);
            a[i] = load_operand<FA>(ac, ba);
            b[i] = load_operand<FB>(bc, bb);
            sa[i] = (int)as[ba];
            sb[i] = (int)bs[bb];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    a[i], b[j], acc[i][j], FA, FB, 0, sa[i], 0, sb[j]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = n0 + 16 * j + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + 16 * i + 4 * g + r;
                if (row < m && col < n)
                    c[row * ldc + col] = acc[i][j][r];
            }
        }
}

__global__ __launch_bounds__(256) void k_zero_fill(float *__restrict__ c, int64_t m, int64_t n,
                                                   int64_t ldc)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < m * n)
        c[(i / n) * ldc + (i % n)] = 0.0f;
}

namespace {
int mfma_format(const mxq_qtensor *q)
{
    if (q->fmt == MXQ_FMT_E2M3)
        return kMfmaFP6;
    if (q->fmt == MXQ_FMT_FP4 && q->grid == MXQ_GRID_E2M1)
        return kMfmaFP4;
    return -1;  // E1M2 nibbles have no matrix-core type; use the E2M3 form
}
}  // namespace

}  // namespace mxq

using namespace mxq;

extern "C" mxq_status mxq_wgrad_gemm(const mxq_qtensor *a, const mxq_qtensor *b, int64_t m,
                                     int64_t n, int64_t k, float *c, int64_t ldc, void *stream)
{
    if (!a || !b || !c || !a->codes || !a->scales || !b->codes || !b->scales)
        return MXQ_ERR_NULL;
    const int fa = mfma_format(a), fb = mfma_format(b);
    if (fa < 0 || fb < 0)
        return MXQ_ERR_UNSUPPORTED;
    if (m < 0 || n < 0 || k < 0 || k % 128 || ldc < n)
        return MXQ_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(a->codes) % 8 || reinterpret_cast<uintptr_t>(b->codes) % 8 ||
        reinterpret_cast<uintptr_t>(c) % 4)
        return MXQ_ERR_ALIGN;
    if (fa == kMfmaFP4 && (reinterpret_cast<uintptr_t>(a->codes) % 16))
        return MXQ_ERR_ALIGN;
    if (fb == kMfmaFP4 && (reinterpret_cast<uintptr_t>(b->codes) % 16))
        return MXQ_ERR_ALIGN;
    if (m == 0 || n == 0)
        return MXQ_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (k == 0) {
        // empty reduction: C = 0 (a fill kernel, so the call stays graph-capturable)
        const int64_t total = m * n;
        hipLaunchKernelGGL(k_zero_fill, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, c,
                           m, n, ldc);
        return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_DEVICE;
    }
    const dim3 grid((unsigned)((n + kTN - 1) / kTN), (unsigned)((m + kTM - 1) / kTM));
    const uint8_t *ac = static_cast<const uint8_t *>(a->codes);
    const uint8_t *bc = static_cast<const uint8_t *>(b->codes);
    if (fa == kMfmaFP4 && fb == kMfmaFP4)
        hipLaunchKernelGGL((k_wgrad_simple<kMfmaFP4, kMfmaFP4>), grid, dim3(256), 0, s, ac, a->scales, bc, b->scales, m, n, k, c, ldc);
    else if (fa == kMfmaFP6 && fb == kMfmaFP6)
        hipLaunchKernelGGL((k_wgrad_simple<kMfmaFP6, kMfmaFP6>), grid, dim3(256), 0, s, ac, a->scales, bc, b->scales, m, n, k, c, ldc);
    else if (fa == kMfmaFP4)
        hipLaunchKernelGGL((k_wgrad_simple<kMfmaFP4, kMfmaFP6>), grid, dim3(256), 0, s, ac, a->scales, bc, b->scales, m, n, k, c, ldc);
    else
        hipLaunchKernelGGL((k_wgrad_simple<kMfmaFP6, kMfmaFP4>), grid, dim3(256), 0, s, ac, a->scales, bc, b->scales, m, n, k, c, ldc);
    return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_DEVICE;
}
