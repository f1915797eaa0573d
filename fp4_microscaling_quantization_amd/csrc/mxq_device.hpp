// Device building blocks of the fused rotate + quantize kernels (gfx950).
//
// Work layout: a 32-element MX block is spread over 4 lanes ("a quad" of the
// block), 8 consecutive block positions per lane; lane `pos` (0..3) holds
// positions 8*pos .. 8*pos+7.  The 4 lanes of a block sit in one 16-lane DPP
// row, at lane distances given by the template arguments XA (partner holding
// the other half of a 16-position half-block: pos ^ 1) and XB (the other
// 16-position half: pos ^ 2).  All cross-lane traffic is DPP (full-rate VALU).
//
// Method sources (web pages): MX blocks of 32 with one E8M0 exponent set by
// the largest exponent in the block -- htx.com news on "Pretraining large
// language models with MXFP4", section "Que es MXFP4?"; H16/H32 rotations --
// gist.science summary "Pre-treinamento de Modelos de Linguagem Grandes com
// MXFP4", section "Metodologia"; Hadamard after random sign inversion and
// stochastic rounding -- the htx.com news, section "Experimento de
// diagnostico"; RTNE onto E2M1 and the uniform E1M2 grid, SR only on dY --
// gist.science summary "Repensando o Vies de Encolhimento (Shrinkage Bias) no
// Pre-treinamento de LLMs em FP4", sections "Metodologia 1" and "2".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

enum : int { kE2M1 = 0, kE1M2 = 1 };
enum : int { kRTNE = 0, kSR = 1 };

// Runtime knobs handed to every quantize kernel.
struct QKnobs {
    uint32_t sign_mask;
    uint32_t seed_lo, seed_hi;
    uint32_t stream;
    uint32_t sr_bits;  // 8 or 16
    int32_t emax;      // E2M1 family: 2, or 1 with a cap (E1M2 kernels use 1)
    float top2;        // E2M1 family: twice the top level (12, or 8 / 6 with a cap)
    uint32_t sign_mode;          // MXQ_SIGNS_MASK: sign_mask holds the mask repeated per
                                 // n-sub-block; MXQ_SIGNS_PER_BLOCK: drawn per block
    uint32_t skey_lo, skey_hi;   // key of the per-block signs
};

// Global-memory views of generic pointers.  A pointer that reaches a kernel
// inside a structure picked at run time (a job of a batch, an output
// descriptor) is generic to the compiler, which then accesses it with flat
// instructions.  Those also count against the LDS and scalar-memory counter,
// so a wait for an LDS access waits for every load still in flight as well.
// Every tensor the kernels read or write lives in device global memory.
#define MXQ_GLOBAL __attribute__((address_space(1)))
template <class T> __device__ __forceinline__ MXQ_GLOBAL T *gmem(T *p) { return (MXQ_GLOBAL T *)p; }
// plain vector types for the wide accesses through such views (HIP's uint2 and
// uint4 have constructors that take generic references only)
typedef uint32_t gv2u __attribute__((ext_vector_type(2)));
typedef uint32_t gv4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float as_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }

// ---- lane exchange within a 16-lane DPP row: returns the value of lane ^ X --
template <int X> __device__ __forceinline__ uint32_t lane_xor(uint32_t v);
template <> __device__ __forceinline__ uint32_t lane_xor<1>(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
}
template <> __device__ __forceinline__ uint32_t lane_xor<2>(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
}
template <> __device__ __forceinline__ uint32_t lane_xor<4>(uint32_t v)
{
    // banks 0 and 2 read lane+4 (row_shl:4), banks 1 and 3 read lane-4 (row_shr:4)
    int t = __builtin_amdgcn_update_dpp((int)v, (int)v, 0x104, 0xF, 0x5, false);
    return (uint32_t)__builtin_amdgcn_update_dpp(t, (int)v, 0x114, 0xF, 0xA, false);
}
template <> __device__ __forceinline__ uint32_t lane_xor<8>(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);  // row_ror:8
}
template <int X> __device__ __forceinline__ float lane_xor_f(float v)
{
    return as_f(lane_xor<X>(as_u(v)));
}

// ---- Philox4x32-10 (Salmon et al., SC'11) -----------------------------------
struct Rand4 {
    uint32_t w[4];
};
__device__ __forceinline__ Rand4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        // three-input XOR in one gfx950 bitop3 (truth table 0x96)
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
        const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    Rand4 r;
    r.w[0] = c0; r.w[1] = c1; r.w[2] = c2; r.w[3] = c3;
    return r;
}

// The 32 sign bits of the block with index j along the quantization axis
// (bit i: position i of the 32-block): the mask, repeated per n-sub-block on
// the host, or word 0 of Philox4x32-10 at counter (lo32 j, hi32 j, ~0, ~1).
template <int HN>
__device__ __forceinline__ uint32_t block_signs(const QKnobs &kn, uint64_t j)
{
    if constexpr (HN == 0)
        return 0u;
    if (kn.sign_mode == 0)
        return kn.sign_mask;
    return philox4x32_10((uint32_t)j, (uint32_t)(j >> 32), 0xFFFFFFFFu, 0xFFFFFFFEu, kn.skey_lo,
                         kn.skey_hi).w[0];
}

// ---- rounding of a normalized magnitude a = |y| 2^-e (0 <= a < 2^(emax+1)) --
// E1M2 levels 0.5 m: m = RNE(2a) by one fused multiply-add against 2^23
// (single rounding of the exact 2a), saturated at 7.
__device__ __forceinline__ uint32_t rtne_e1m2(float a)
{
    const float t = __builtin_fmaf(a, 2.0f, 8388608.0f);
    return min(as_u(t) - 0x4B000000u, 7u);
}

// E2M1 segment of a: 0 for a < 2 (step 0.5), 1 for [2, 4) (step 1), 2 for
// a >= 4 (step 2); from the fp32 exponent field.
__device__ __forceinline__ int e2m1_segment(float a)
{
    return min(max((int)(as_u(a) >> 23) - 127, 0), 2);
}

// E2M1 in software: RNE(a / step) + segment offset, saturated at 7.
__device__ __forceinline__ uint32_t rtne_e2m1_soft(float a)
{
    const int d = e2m1_segment(a);
    const float s = as_f((uint32_t)(128 - d) << 23);          // 2^(1-d) = 1/step
    const float t = __builtin_fmaf(a, s, 8388608.0f);          // a*s exact
    return min(as_u(t) - 0x4B000000u + 2u * (uint32_t)d, 7u);
}

// SR: round up iff 2r + 1 < p 2^(B+1), p the exact fraction of the gap.
__device__ __forceinline__ uint32_t sr_e1m2(float a, uint32_t r, float two_pow_b1)
{
    const float x = a * 2.0f;
    const float k = floorf(x);
    const float p = x - k;                                     // exact
    const uint32_t up = (float)(2u * r + 1u) < p * two_pow_b1;
    return min((uint32_t)k + up, 7u);
}
__device__ __forceinline__ uint32_t sr_e2m1(float a, uint32_t r, float two_pow_b1)
{
    const int d = e2m1_segment(a);
    const float x = a * as_f((uint32_t)(128 - d) << 23);       // a / step, exact
    const float k = floorf(x);
    const float p = x - k;
    const uint32_t up = (float)(2u * r + 1u) < p * two_pow_b1;
    return min((uint32_t)k + 2u * (uint32_t)d + up, 7u);
}

// ---- block rotation of the lane's 8 values -----------------------------------
// y = fl32(1/sqrt(n)) * H_n * v on each n-position sub-block, H_n Sylvester,
// butterfly stages of stride 1, 2, 4 (in-lane), 8 (lane ^ XA) and, for n = 32,
// 16 (lane ^ XB) -- the same fp32 operations in the same stage order as the
// fast transform applied to the whole block.
template <int HN, int XA, int XB>
__device__ __forceinline__ void rotate8(float (&v)[8], int pos)
{
    if constexpr (HN >= 16) {
        // Butterfly stages of stride 1, 2, 4 inside the lane ...
#pragma unroll
        for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (!(i & h)) {
                    const float a = v[i], b = v[i + h];
                    v[i] = a + b;
                    v[i + h] = a - b;
                }
            }
        }
        // ... stride 8 across the pair (pos, pos^1): the lower lane keeps
        // u + u', the upper one u' - u (own value negated, then added).
        {
            const uint32_t neg = (pos & 1) ? 0x80000000u : 0u;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float p = lane_xor_f<XA>(v[i]);
                v[i] = p + as_f(as_u(v[i]) ^ neg);
            }
        }
        if constexpr (HN == 32) {
            const uint32_t neg = (pos & 2) ? 0x80000000u : 0u;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float p = lane_xor_f<XB>(v[i]);
                v[i] = p + as_f(as_u(v[i]) ^ neg);
            }
        }
        const float c = HN == 16 ? 0.25f : as_f(0x3E3504F3u);  // fl32(1/sqrt(n))
#pragma unroll
        for (int i = 0; i < 8; ++i)
            v[i] = v[i] * c;
    }
}

// ---- block rotation of 16 consecutive positions held by one lane -----------
// The fp32 butterfly stages of stride 1, 2, 4, 8 inside the lane and, for
// n = 32, stride 16 across the lane pair (pos, pos ^ 1) at DPP distance 1:
// the lower lane keeps u + u', the upper one u - u' (u lower, u' upper).
// No normalisation (the caller multiplies by fl32(1/sqrt(n)) or folds it).
template <int HN>
__device__ __forceinline__ void rotate16_raw(float (&v)[16], int pos)
{
    if constexpr (HN >= 16) {
#pragma unroll
        for (int s = 1; s < 16; s <<= 1) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (!(i & s)) {
                    const float p = v[i], q = v[i + s];
                    v[i] = p + q;
                    v[i + s] = p - q;
                }
            }
        }
        if constexpr (HN == 32) {
            const float beta = pos ? -1.0f : 1.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                v[i] = __builtin_fmaf(v[i], beta, lane_xor_f<1>(v[i]));
        }
    }
}

// ---- rounding of 8 signed values y * inv onto the grid --------------------
// Returns the sign-magnitude nibbles, element i in bits 4i..4i+3.  `r` and
// `tpb` = 2^(B+1) are only read for SR.
// `top` is the E2M1 family's top level (6, or the cap 4 / 3): larger
// magnitudes are brought down to it first.
template <int GRID, int ROUND>
__device__ __forceinline__ uint32_t round8(const float (&v)[8], float inv, const uint32_t (&r)[8],
                                           float tpb, float top)
{
    uint32_t w = 0;
    const bool capped = GRID == kE2M1 && top < 6.0f;
    if constexpr (GRID == kE2M1 && ROUND == kRTNE) {
        // the gfx950 FP4 convert rounds to nearest-even E2M1 with saturation
        // and keeps the sign (including -0); y * 2^-e is exact
        float s[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            s[i] = capped ? __builtin_amdgcn_fmed3f(v[i] * inv, -top, top) : v[i] * inv;
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, s[0], s[1], 1.0f, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, s[2], s[3], 1.0f, 1);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, s[4], s[5], 1.0f, 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, s[6], s[7], 1.0f, 3);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float a = capped ? fminf(fabsf(v[i]) * inv, top) : fabsf(v[i]) * inv;
            uint32_t m;
            if constexpr (ROUND == kRTNE)
                m = GRID == kE1M2 ? rtne_e1m2(a) : rtne_e2m1_soft(a);
            else
                m = GRID == kE1M2 ? sr_e1m2(a, r[i], tpb) : sr_e2m1(a, r[i], tpb);
            w |= (m | ((as_u(v[i]) >> 28) & 8u)) << (4 * i);
        }
    }
    return w;
}

}  // namespace mxq
