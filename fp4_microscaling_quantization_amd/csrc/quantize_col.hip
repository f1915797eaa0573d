// Column-wise fused rotate + quantize: blocks of 32 consecutive rows of one
// column, the kernel behind mxq_quantize when only the column-wise output is
// requested (the operands of the weight-gradient product dY^T X are both
// quantized along the token dimension, which is the row dimension of dY and X).
//
// Work layout.  A wave covers 32 rows x 128 columns, a workgroup 4 waves
// stacked along the rows (128 x 128).  Lane (cg, pos) = (lane >> 1, lane & 1)
// loads rows 16 pos .. 16 pos + 15 of its row band in the four columns
// 4 cg .. 4 cg + 3 (sixteen 8-byte loads), so it holds 16 consecutive block
// positions of four column blocks.  The size-16 rotation then runs entirely
// inside the lane; the two lanes of a block meet (by DPP) only for the block
// maximum and, for H32, the last butterfly stage.
//
// Arithmetic.  The fp32 operations of the method's definition (fp32 butterfly
// stages in order, then the scale and the rounding), up to exact rewrites:
//  * The 1/4 normalisation of H16 is folded into the power-of-two scale
//    multiplier (exact while the rotated value is a normal fp32 number, i.e.
//    for every block whose scale code is at least 40; lower blocks take the
//    unfused order).  The block maximum is taken on the unnormalised values
//    and divided by 4 once (monotone rounding).
//  * Rounding produces the chosen level as an fp32 value: RTNE by rint after
//    clamping, SR by ceil(x - (2r + 1) 2^-(B+1)), which rounds up exactly
//    when the fraction of x above its lower level exceeds (2r + 1) 2^-(B+1).
//  * The gfx950 scaled converts turn those grid values into FP4 or E2M3 codes
//    (a value on the grid converts exactly; the scale operand divides by a
//    power of two).
//
// Method sources (web pages): MX blocks of 32 sharing one E8M0 exponent taken
// from the block's largest magnitude -- htx.com news on "Pretraining large
// language models with MXFP4", section "Que es MXFP4?"; H16 / H32 rotations
// and the random sign flips -- gist.science summary "Pre-treinamento de
// Modelos de Linguagem Grandes com MXFP4", section "Metodologia", and the
// htx.com news, section "Experimento de diagnostico"; RTNE onto E2M1 or the
// uniform E1M2 grid and SR on the gradient -- gist.science summary
// "Repensando o Vies de Encolhimento (Shrinkage Bias) no Pre-treinamento de
// LLMs em FP4", sections "Metodologia 1" and "Metodologia 2".
#include "mxq_device.hpp"
#include "mxq_host.hpp"
#include "quant_out.hpp"

namespace mxq {

typedef float f16v __attribute__((ext_vector_type(16)));

// E2M3 codes of 32 fp32 values lying on the E2M3 grid after division by
// `scale`.  Code k of the 192-bit little-endian result (bits 6k .. 6k+5) is
// that of a[k / 2] for even k and of b[k / 2] for odd k.  The convert still
// reads its sources while it writes its destination, so the two must not
// share registers: the empty asm statement keeps both sources live past the
// convert, which keeps the register allocator from placing the result on top
// of them.
__device__ __forceinline__ void cvt_e2m3_32(const f16v &a, const f16v &b, float scale,
                                            uint32_t (&out)[6])
{
    const auto r = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(a, b, scale);
    asm volatile("" ::"v"(a), "v"(b));
#pragma unroll
    for (int i = 0; i < 6; ++i)
        out[i] = r[i];
}

// Philox4x32-10 output for the lane's positions 16 pos + 8 g .. + 7 with
// 16-bit draws: element j of block `blk` takes counter (j >> 3, blk lo,
// blk hi, stream), half j & 1 of word (j >> 1) & 3; with 8-bit draws
// (g = 0 only) element j takes counter (j >> 4, ...), byte j & 3 of word
// (j >> 2) & 3 (the definition in include/mxq.h).  The draws stay packed
// in the four output words until their position is rounded: sixteen fp32
// copies held at once would push the SR tile body past 128 VGPRs (three
// waves per SIMD instead of four).
__device__ __forceinline__ Rand4 sr_draw(const QKnobs &kn, int pos, int g, uint64_t blk)
{
    const uint32_t ctr = kn.sr_bits == 16 ? (uint32_t)(2 * pos + g) : (uint32_t)pos;
    return philox4x32_10(ctr, (uint32_t)blk, (uint32_t)(blk >> 32), kn.stream, kn.seed_lo,
                         kn.seed_hi);
}

// The convert scale that maps the values col16 leaves behind onto the grid.
template <int GRID, int ROUND>
constexpr float level_unit()
{
    return (GRID == kE2M1 && ROUND == kSR) ? 4.0f : 2.0f;
}

// One column block seen by one lane: v holds positions 16 pos .. 16 pos + 15
// (bf16 widened, random signs applied).  Rotates, finds the block's E8M0
// code (returned) and leaves in v the rounded levels times level_unit(), with
// the sign of the rotated value (for E2M1 with RTNE and FP4 output, the
// unrounded value times 2: the FP4 convert rounds it; for E1M2 with FP4
// output, the bits of the sign-magnitude nibble).
template <int GRID, int ROUND, int HN, bool EXACT_LEVEL>
__device__ __forceinline__ uint32_t col16(float (&v)[16], int pos, uint64_t blk, const QKnobs &kn,
                                          float h, float h2)
{
    const int EMAX = GRID == kE2M1 ? kn.emax : 1;
    // ---- rotation: fp32 butterflies of stride 1, 2, 4, 8 in the lane, 16 across
    rotate16_raw<HN>(v, pos);
    // H32's factor c = fl32(1/sqrt(32)).  Where the rounding below starts with
    // a plain product (RTNE; SR onto E2M1), c goes into the power-of-two
    // multiplier instead of a product of its own: fl(v (c 2^k)) = fl(v c) 2^k
    // while c 2^k is a normal number and the result is too (a result below
    // the normal range rounds to code 0 either way), and the block maximum of
    // |fl(v c)| is fl(max |v| c), rounding being monotone.  SR onto E1M2 starts
    // with a fused multiply-add, whose one rounding would then differ from the
    // rounded fl(v c): there c stays a product of its own.
    constexpr float c32 = __builtin_bit_cast(float, 0x3E3504F3u);  // fl32(1/sqrt(32))
    constexpr bool kFoldC = HN == 32 && (ROUND == kRTNE || GRID == kE2M1);
    if constexpr (HN == 32 && !kFoldC) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            v[i] = v[i] * c32;
    }
    // ---- block maximum of |y|
    uint32_t am;
    if constexpr (HN >= 16) {
        // Each output of a rotated sub-block mixes all its inputs: a NaN or Inf
        // input leaves no finite value in the lane, so fmax (which skips a NaN
        // operand) still returns a non-finite maximum for such a block.
        float m = fabsf(v[0]);
#pragma unroll
        for (int i = 1; i < 16; ++i)
            m = fmaxf(m, fabsf(v[i]));
        am = as_u(m);
    } else {
        // magnitude maximum on the bit patterns (NaN > Inf > finite): the
        // signed maximum finds the largest positive value, the unsigned one the
        // largest negative value
        uint32_t um = 0;
        int32_t sm = (int32_t)0x80000000u;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            um = max(um, as_u(v[i]));
            sm = max(sm, (int32_t)as_u(v[i]));
        }
        am = max(um & 0x7FFFFFFFu, (uint32_t)sm & 0x7FFFFFFFu);
    }
    am = max(am, lane_xor<1>(am));
    if constexpr (HN == 16)
        am = as_u(as_f(am) * 0.25f);  // fl(max|v| / 4) = max |fl(v / 4)|
    if constexpr (kFoldC)
        am = as_u(as_f(am) * c32);    // fl(max|v| c) = max |fl(v c)|
    const uint32_t sc = am >= 0x7F800000u ? 0xFFu : (uint32_t)max((int)(am >> 23) - EMAX, 0);

    // ---- multiplier m2 = 2 * 2^-e (times 1/4 for H16): v * m2 = 2 y 2^-e
    float m2;
    if (sc < 40u) {
        // low scale: the unfused order (y = v / 4 may be subnormal; 2^-e up to 2^127)
        const float inv = as_f((254u - sc) << 23);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if constexpr (HN == 16)
                v[i] = v[i] * 0.25f;
            if constexpr (kFoldC)
                v[i] = v[i] * c32;
            v[i] = v[i] * inv;
        }
        m2 = 2.0f;
    } else {
        m2 = as_f((255u - min(sc, 253u)) << 23);
        if constexpr (HN == 16)
            m2 *= 0.25f;
        if constexpr (kFoldC) {
            if (sc <= 251u) {
                m2 *= c32;  // c 2^(128 - sc) >= 2^-126: exact
            } else {
                // the top codes (and non-finite blocks): c 2^(128 - sc) would be
                // subnormal, so v takes c first
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    v[i] = v[i] * c32;
            }
        }
    }

    // ---- rounding
    if constexpr (ROUND == kRTNE) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float t = v[i] * m2;  // 2 a, signed
            if constexpr (GRID == kE1M2) {
                // levels 0.5 m: m = RNE(2a), saturated at 7
                const float c = __builtin_amdgcn_fmed3f(t, -7.0f, 7.0f);
                if constexpr (EXACT_LEVEL)
                    v[i] = rintf(c);
                else  // the FP4 nibble: RNE(|c|) is the low bits of 2^23 + |c|, and
                      // bit 3 of as_u(c) >> 28 (nothing above it) is c's sign;
                      // one bitop3 selects bits 0-2 from the first, the rest from
                      // the second (truth table 0xE4: s2 ? s0 : s1)
                    v[i] = as_f(__builtin_amdgcn_bitop3_b32(as_u(fabsf(c) + 8388608.0f),
                                                            as_u(c) >> 28, 7u, 0xE4));
            } else if constexpr (!EXACT_LEVEL) {
                // the FP4 convert rounds t / 2 to nearest even (saturating at 6);
                // a capped grid stops at its cap first
                v[i] = __builtin_amdgcn_fmed3f(t, -kn.top2, kn.top2);
            } else {
                // E2M1 in software: round 2a to a multiple of 2 step by adding and
                // subtracting 1.5 2^22 S (S = 2^max(floor(log2 2a), 1), whose ulp is 2 step)
                const float a2 = fminf(fabsf(t), kn.top2);
                const float S = as_f(max(as_u(a2) & 0x7F800000u, 0x40000000u));
                const float G = S * 6291456.0f;
                v[i] = copysignf((a2 + G) - G, t);
            }
        }
    } else {
        // round position i with its random integer r (as fp32)
        auto sr_one = [&](int i, float r) {
            if constexpr (GRID == kE1M2) {
                // x = min(2a, 7) - h; level index ceil(x - 2 h r)
                const float x = fminf(__builtin_fmaf(fabsf(v[i]), m2, -h), 7.0f - h);
                const float m = ceilf(__builtin_fmaf(r, -h2, x));
                if constexpr (EXACT_LEVEL)
                    v[i] = copysignf(m, v[i]);
                else  // the FP4 nibble, as for RTNE (m is an integer 0..7)
                    v[i] = as_f(__builtin_amdgcn_bitop3_b32(as_u(m + 8388608.0f),
                                                            as_u(v[i]) >> 28, 7u, 0xE4));
            } else {
                // a in units of the local step (S / 4 for 2a below 2 S): x = 2a * 2 / S
                const float a2 = fminf(fabsf(v[i]) * m2, kn.top2);
                const float S = as_f(max(as_u(a2) & 0x7F800000u, 0x40000000u));
                const float x = __builtin_fmaf(a2, as_f(0x7F800000u - as_u(S)), -h);
                v[i] = copysignf(ceilf(__builtin_fmaf(r, -h2, x)) * S, v[i]);
            }
        };
        if (kn.sr_bits == 16) {
            // both draws first: two independent Philox chains interleave
            const Rand4 q[2] = {sr_draw(kn, pos, 0, blk), sr_draw(kn, pos, 1, blk)};
#pragma unroll
            for (int i = 0; i < 16; ++i)
                sr_one(i, (float)((q[i >> 3].w[(i >> 1) & 3] >> (16 * (i & 1))) & 0xFFFFu));
        } else {
            const Rand4 q = sr_draw(kn, pos, 0, blk);
#pragma unroll
            for (int i = 0; i < 16; ++i)
                sr_one(i, (float)((q.w[i >> 2] >> (8 * (i & 3))) & 0xFFu));
        }
    }
    return sc;
}

// FP4 nibbles of the 16 values col16 left in v (element i at bits 4i of w).
template <int GRID, int ROUND>
__device__ __forceinline__ void pack_fp4(const float (&v)[16], uint32_t sc, uint32_t (&w)[2])
{
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        uint32_t x = 0;
        if constexpr (GRID == kE2M1) {
            constexpr float u = level_unit<GRID, ROUND>();
            x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[8 * d + 0], v[8 * d + 1], u, 0);
            x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[8 * d + 2], v[8 * d + 3], u, 1);
            x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[8 * d + 4], v[8 * d + 5], u, 2);
            x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[8 * d + 6], v[8 * d + 7], u, 3);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                x |= as_u(v[8 * d + i]) << (4 * i);  // col16 left the nibble itself
        }
        w[d] = sc == 0xFFu ? 0u : x;
    }
}

template <int N>
__device__ __forceinline__ void store_words(const OutDesc &o, uint64_t line, uint64_t jb, int pos,
                                            const uint32_t *w)
{
    MXQ_GLOBAL uint32_t *d = reinterpret_cast<MXQ_GLOBAL uint32_t *>(
        gmem(o.codes) + code_offset(o, line, jb, 8 * N) + 4 * N * pos);
#pragma unroll
    for (int k = 0; k < N; ++k)
        d[k] = w[k];
}

// The same words into the LDS image of a workgroup's 128 column x 4 block
// output tile: column cl (0..127), row band wv (0..3, i.e. block 4 by + wv).
// MFMA layout: the 8 tiles x 64 lane slots of one k-step (one contiguous run);
// row layout: column-major, each column's 4 blocks adjacent (one run each).
template <int N>
__device__ __forceinline__ void stage_words(uint32_t *stage, int layout, int cl, int wv, int pos,
                                            const uint32_t *w)
{
    const int slot = layout == MXQ_LAYOUT_MFMA ? (cl >> 4) * 64 + 16 * wv + (cl & 15) : 4 * cl + wv;
    uint32_t *d = stage + slot * (2 * N) + N * pos;
#pragma unroll
    for (int k = 0; k < N; ++k)
        d[k] = w[k];
}

// Write the staged output tile (after a barrier): line0 = 128 bx, block 4 by.
template <int BB>
__device__ __forceinline__ void flush_stage(const OutDesc &o, const uint32_t *stage, int t,
                                            uint64_t line0, uint64_t jb0)
{
    if (o.layout == MXQ_LAYOUT_MFMA) {
        // one run of 128 * BB bytes, 16-byte aligned; nontemporal stores: in
        // the batched column launch they made the weight-gradient pair 3-7%
        // faster (X's RTNE job first, as the step issues it), and the dual
        // kernel 2-3%
        MXQ_GLOBAL gv4u *dst =
            reinterpret_cast<MXQ_GLOBAL gv4u *>(gmem(o.codes) + code_offset(o, line0, jb0, BB));
        const gv4u *src = reinterpret_cast<const gv4u *>(stage);
#pragma unroll
        for (int k = 0; k < BB / 8; ++k)
            __builtin_nontemporal_store(src[k * 256 + t], dst + k * 256 + t);
    } else if ((reinterpret_cast<uintptr_t>(o.codes) & 15) == 0 && (BB == 16 || (o.nbk & 1) == 0)) {
        // 128 runs of 4 * BB bytes, each 16-byte aligned (E2M3 runs need an
        // even block count per line): 16-byte stores, 2 or 3 per thread instead
        // of 8 or 12 word stores (the column kernels 3-8% and the dual kernel 2%
        // faster).  Ordinary stores: on these half-line runs nontemporal ones
        // were slower.
        constexpr int U = BB / 4;          // 16-byte units per column run
        const gv4u *src = reinterpret_cast<const gv4u *>(stage);
#pragma unroll
        for (int k = 0; k < U / 2; ++k) {
            const int q = k * 256 + t, cl = q / U, u = q - cl * U;
            MXQ_GLOBAL gv4u *dst =
                reinterpret_cast<MXQ_GLOBAL gv4u *>(gmem(o.codes) + code_offset(o, line0 + cl, jb0, BB)) + u;
            *dst = src[q];
        }
    } else {
        // 128 runs of 4 * BB bytes, codes only 4-byte aligned
        constexpr int W = BB;              // words per column run (4 blocks x BB / 4)
#pragma unroll
        for (int k = 0; k < W / 2; ++k) {
            const int idx = k * 256 + t, cl = idx / W, q = idx % W;
            reinterpret_cast<MXQ_GLOBAL uint32_t *>(gmem(o.codes) +
                                                    code_offset(o, line0 + cl, jb0, BB))[q] =
                stage[cl * W + q];
        }
    }
}

// One 128 x 128 tile of the column-wise quantization: columns 128 bx ..,
// rows 128 by .. (rows % 32 == 0).  `stage` is the workgroup's LDS image of
// the tile's output (128 * BB words).
template <int GRID, int ROUND, int HN, int FMT>
__device__ __forceinline__ void col_tile(int64_t bx, int64_t by, const uint16_t *__restrict__ x,
                                         int64_t rows, int64_t cols, int64_t ld,
                                         const OutDesc &out, int vec, const QKnobs &kn,
                                         uint32_t *stage)
{
    // the wave index as a scalar (it is uniform across the wave): the row band
    // and the LDS offsets derived from it then take no vector registers, which
    // keeps the stochastic-rounding bodies at 4 waves per SIMD
    const int t = threadIdx.x, lane = t & 63, wv = __builtin_amdgcn_readfirstlane(t >> 6);
    const int pos = lane & 1, cg = lane >> 1;
    const int64_t rband = by * 128 + wv * 32;  // rows % 32 == 0
    // A full 128 x 128 tile stages its codes in LDS and writes them as long
    // runs (MFMA layout: one run; row layout: 4 blocks per column).  Every wave
    // of such a workgroup has rows, so none returns early.
    constexpr int BB = FMT == MXQ_FMT_E2M3 ? 24 : 16;           // bytes per block
    const bool staged = bx * 128 + 128 <= cols && by * 128 + 128 <= rows;
    if (rband >= rows)
        return;                                                   // whole wave
    const int64_t r0 = rband + 16 * pos;
    const int64_t c0 = bx * 128 + 4 * cg;
    const uint64_t jb = (uint64_t)rband >> 5, nbc = (uint64_t)rows >> 5;

    // lo[i]: columns c0, c0 + 1 of row r0 + i; hi[i]: columns c0 + 2, c0 + 3
    uint32_t lo[16], hi[16];
    if (vec && c0 + 4 <= cols) {
        // nontemporal: the tensor is read once (with the nontemporal code
        // stores: X's RTNE quantize 4-5% faster, the batched pair 1-2%; the
        // row kernel's 16-byte loads lose by it and stay ordinary)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const gv2u w = __builtin_nontemporal_load(
                reinterpret_cast<const MXQ_GLOBAL gv2u *>(gmem(x) + (r0 + i) * ld + c0));
            lo[i] = w.x;
            hi[i] = w.y;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            uint32_t hh[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                hh[j] = (c0 + j < cols) ? (uint32_t)gmem(x)[(r0 + i) * ld + c0 + j] : 0u;
            lo[i] = hh[0] | (hh[1] << 16);
            hi[i] = hh[2] | (hh[3] << 16);
        }
    }
    // random sign flips: position p = 16 pos + i takes bit p of the block's sign word
    if constexpr (HN > 0) {
        const uint32_t sg = block_signs<HN>(kn, jb) >> (16 * pos);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t f = ((sg >> i) & 1u) ? 0x80008000u : 0u;
            lo[i] ^= f;
            hi[i] ^= f;
        }
    }
    const float h = kn.sr_bits == 16 ? 0x1p-17f : 0x1p-9f;  // 2^-(B+1)
    const float h2 = 2.0f * h;
    constexpr bool kExact = FMT == MXQ_FMT_E2M3;

#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
        float a[16], b[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t w = jp ? hi[i] : lo[i];
            a[i] = as_f(w << 16);
            b[i] = as_f(w & 0xFFFF0000u);
        }
        const int64_t ca = c0 + 2 * jp, cb = ca + 1;
        const uint32_t sa =
            col16<GRID, ROUND, HN, kExact>(a, pos, (uint64_t)ca * nbc + jb, kn, h, h2);
        const uint32_t sb =
            col16<GRID, ROUND, HN, kExact>(b, pos, (uint64_t)cb * nbc + jb, kn, h, h2);
        if constexpr (FMT == MXQ_FMT_E2M3) {
            f16v s0, s1;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                s0[j] = a[2 * j];
                s1[j] = a[2 * j + 1];
                s0[8 + j] = b[2 * j];
                s1[8 + j] = b[2 * j + 1];
            }
            uint32_t o[6];
            cvt_e2m3_32(s0, s1, level_unit<GRID, ROUND>(), o);
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                o[k] = sa == 0xFFu ? 0u : o[k];
                o[3 + k] = sb == 0xFFu ? 0u : o[3 + k];
            }
            if (staged) {
                stage_words<3>(stage, out.layout, 4 * cg + 2 * jp, wv, pos, o);
                stage_words<3>(stage, out.layout, 4 * cg + 2 * jp + 1, wv, pos, o + 3);
            } else {
                if (ca < cols)
                    store_words<3>(out, (uint64_t)ca, jb, pos, o);
                if (cb < cols)
                    store_words<3>(out, (uint64_t)cb, jb, pos, o + 3);
            }
        } else {
            uint32_t wa[2], wb[2];
            pack_fp4<GRID, ROUND>(a, sa, wa);
            pack_fp4<GRID, ROUND>(b, sb, wb);
            if (staged) {
                stage_words<2>(stage, out.layout, 4 * cg + 2 * jp, wv, pos, wa);
                stage_words<2>(stage, out.layout, 4 * cg + 2 * jp + 1, wv, pos, wb);
            } else {
                if (ca < cols)
                    store_words<2>(out, (uint64_t)ca, jb, pos, wa);
                if (cb < cols)
                    store_words<2>(out, (uint64_t)cb, jb, pos, wb);
            }
        }
        if (pos == 0) {
            if (ca < cols)
                gmem(out.scales)[scale_offset(out, (uint64_t)ca, jb)] = (uint8_t)sa;
            if (cb < cols)
                gmem(out.scales)[scale_offset(out, (uint64_t)cb, jb)] = (uint8_t)sb;
        }
    }
    if (staged) {
        __syncthreads();
        flush_stage<BB>(out, stage, t, (uint64_t)bx * 128, (uint64_t)by * 4);
    }
}

template <int GRID, int ROUND, int HN, int FMT>
__global__ __launch_bounds__(256) void k_quant_col(const uint16_t *__restrict__ x, int64_t rows,
                                                   int64_t cols, int64_t ld, OutDesc out, int vec,
                                                   QKnobs kn)
{
    __shared__ uint32_t stage[128 * (FMT == MXQ_FMT_E2M3 ? 24 : 16)];  // 128 columns x 4 blocks
    col_tile<GRID, ROUND, HN, FMT>(blockIdx.x, blockIdx.y, x, rows, cols, ld, out, vec, kn, stage);
}

// Several column-wise quantizations in one launch (same grid family, rotation
// and code format; each job its own rounding): workgroup w takes tile
// w - first of the job whose tile range holds w, in the same x-fastest tile
// order as k_quant_col's 2-D grid.  Jobs run in the order given: the next
// job's tiles fill the last partial wave of the previous job's workgroups,
// and the launch gap between separate kernels goes.
// The job's fields in SGPRs, read by a few wide scalar loads at the start.
// Left to itself the compiler loads each field where it is first used, and
// every such load's wait then stalls the waves in the middle of the tile.
__device__ __forceinline__ ColJob load_job(const ColJob &src)
{
    constexpr int N = (int)(sizeof(ColJob) / 4);
    const uint32_t *s = reinterpret_cast<const uint32_t *>(&src);
    uint32_t v[N];
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] = s[i];
#pragma unroll
    for (int i = 0; i < N; ++i)
        asm volatile("" : "+s"(v[i]));
    ColJob q;
    uint32_t *d = reinterpret_cast<uint32_t *>(&q);
#pragma unroll
    for (int i = 0; i < N; ++i)
        d[i] = v[i];
    return q;
}

// RMODE: kRTNE or kSR when every job of the launch rounds that way (one
// tile body, so the kernel keeps that body's register budget and occupancy),
// kBatchMixed when both occur.
template <int GRID, int HN, int FMT, int RMODE>
__global__ __launch_bounds__(256) void k_quant_col_batch(ColBatch b)
{
    __shared__ uint32_t stage[128 * (FMT == MXQ_FMT_E2M3 ? 24 : 16)];
    // the host keeps a launch below 2^24 workgroups: tile indices fit 32 bits
    const uint32_t w = blockIdx.x;
    int j = 0;
#pragma unroll
    for (int i = 1; i < kColBatchMax; ++i)
        if (i < b.n && w >= (uint32_t)b.job[i].first)
            j = i;
    const ColJob q = load_job(b.job[j]);
    const uint32_t tile = w - (uint32_t)q.first, gx = (uint32_t)q.gx;
    const uint32_t by = tile / gx, bx = tile - by * gx;
    if constexpr (RMODE != kBatchMixed)
        col_tile<GRID, RMODE, HN, FMT>(bx, by, q.x, q.rows, q.cols, q.ld, q.out, q.vec, q.kn,
                                       stage);
    else if (q.round == kSR)
        col_tile<GRID, kSR, HN, FMT>(bx, by, q.x, q.rows, q.cols, q.ld, q.out, q.vec, q.kn, stage);
    else
        col_tile<GRID, kRTNE, HN, FMT>(bx, by, q.x, q.rows, q.cols, q.ld, q.out, q.vec, q.kn,
                                       stage);
}

// Row-wise fused rotate + quantize with the column kernel's per-lane work:
// two lanes per 32-block, each holding 16 consecutive positions (two 16-byte
// loads), the lane pair adjacent (DPP distance 1).  A wave handles 128
// consecutive blocks of the row-major block order as 4 rounds of 32 (so each
// load instruction reads 2 KB contiguously when rows are dense), a lane 4
// blocks; codes go out as 8 (FP4) or 12 (E2M3) contiguous bytes per lane.
template <int GRID, int ROUND, int HN, int FMT>
__global__ __launch_bounds__(256) void k_quant_row16(const uint16_t *__restrict__ x,
                                                     uint64_t nblocks, uint32_t nbr, int64_t ld,
                                                     int dense, int vec, OutDesc out, QKnobs kn)
{
    constexpr int U = 4;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int pos = lane & 1, pr = lane >> 1;
    const uint64_t base = ((uint64_t)blockIdx.x * 4 + wv) * (32 * U);
    const float h = kn.sr_bits == 16 ? 0x1p-17f : 0x1p-9f;  // 2^-(B+1)
    const float h2 = 2.0f * h;
    constexpr bool kExact = FMT == MXQ_FMT_E2M3;

    float v[U][16];
    uint64_t line[U], jbk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint64_t b = base + 32 * u + pr;
        const bool ok = b < nblocks;
        line[u] = ok ? b / nbr : 0;
        jbk[u] = ok ? b - line[u] * nbr : 0;
        const int64_t off = (dense ? (int64_t)b * 32 : (int64_t)line[u] * ld + (int64_t)jbk[u] * 32) + 16 * pos;
        uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (ok) {
            if (vec) {
                const gv4u q0 = *reinterpret_cast<const MXQ_GLOBAL gv4u *>(gmem(x) + off);
                const gv4u q1 = *reinterpret_cast<const MXQ_GLOBAL gv4u *>(gmem(x) + off + 8);
                w[0] = q0.x; w[1] = q0.y; w[2] = q0.z; w[3] = q0.w;
                w[4] = q1.x; w[5] = q1.y; w[6] = q1.z; w[7] = q1.w;
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    w[k] = (uint32_t)gmem(x)[off + 2 * k] | ((uint32_t)gmem(x)[off + 2 * k + 1] << 16);
            }
        }
        const uint32_t sg = block_signs<HN>(kn, jbk[u]) >> (16 * pos);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            v[u][2 * k] = as_f((w[k] << 16) ^ (((sg >> (2 * k)) & 1u) << 31));
            v[u][2 * k + 1] = as_f((w[k] & 0xFFFF0000u) ^ (((sg >> (2 * k + 1)) & 1u) << 31));
        }
    }
#pragma unroll
    for (int up = 0; up < U; up += 2) {
        uint32_t sc[2];
#pragma unroll
        for (int d = 0; d < 2; ++d)
            sc[d] = col16<GRID, ROUND, HN, kExact>(v[up + d], pos, base + 32 * (up + d) + pr, kn, h, h2);
        if constexpr (FMT == MXQ_FMT_E2M3) {
            f16v s0, s1;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                s0[j] = v[up][2 * j];
                s1[j] = v[up][2 * j + 1];
                s0[8 + j] = v[up + 1][2 * j];
                s1[8 + j] = v[up + 1][2 * j + 1];
            }
            uint32_t o[6];
            cvt_e2m3_32(s0, s1, level_unit<GRID, ROUND>(), o);
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                if (base + 32 * (up + d) + pr >= nblocks)
                    continue;
                uint32_t wd[3];
#pragma unroll
                for (int k = 0; k < 3; ++k)
                    wd[k] = sc[d] == 0xFFu ? 0u : o[3 * d + k];
                store_words<3>(out, line[up + d], jbk[up + d], pos, wd);
            }
        } else {
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                uint32_t wd[2];
                pack_fp4<GRID, ROUND>(v[up + d], sc[d], wd);
                if (base + 32 * (up + d) + pr < nblocks)
                    store_words<2>(out, line[up + d], jbk[up + d], pos, wd);
            }
        }
        if (pos == 0) {
#pragma unroll
            for (int d = 0; d < 2; ++d)
                if (base + 32 * (up + d) + pr < nblocks)
                    gmem(out.scales)[scale_offset(out, line[up + d], jbk[up + d])] = (uint8_t)sc[d];
        }
    }
}

// Row-wise quantize through LDS: a workgroup takes 16 lines (one 16-line tile
// of the matrix-core layout) by 32 blocks (8 k-steps), wave w lines 4 w ..
// 4 w + 3, a lane pair one block as in k_quant_row16.  Written straight to the
// matrix-core layout, each lane's half block lands in a different 16-byte
// slot; here the tile's 8 step runs (64 slots each) are assembled in LDS and
// leave as whole runs of 16-byte nontemporal stores, and the scale words of
// the tile's 2 groups as whole words.  In the row layout the same image
// leaves as 16 line runs of 32 blocks (512 or 768 bytes) and 16 runs of 32
// scale bytes.  The LDS image pads each 16-slot row (one block index g of the
// k-step) and each step so that the 64 lanes of a write land on spread banks
// (FP4: 272 / 1088 bytes, E2M3: 520 / 2080).  Needs rows % 16 == 0, 32 |
// blocks per row and 16-byte loads; in the row layout also 16-byte aligned
// codes and 4-byte aligned scales (the host checks).
template <int FMT> struct RowImg {
    static constexpr int BB = FMT == MXQ_FMT_E2M3 ? 24 : 16;   // bytes per block
    static constexpr int GP = FMT == MXQ_FMT_E2M3 ? 520 : 272; // bytes per 16-slot row
    static constexpr int SP = 4 * GP;                           // bytes per step
};

template <int GRID, int ROUND, int HN, int FMT>
__global__ __launch_bounds__(256) void k_quant_row16m(const uint16_t *__restrict__ x, uint32_t nbr,
                                                      int64_t ld, OutDesc out, QKnobs kn)
{
    constexpr int BB = RowImg<FMT>::BB, GP = RowImg<FMT>::GP, SP = RowImg<FMT>::SP;
    constexpr int N = BB / 8;                                    // words per half block
    __shared__ __align__(16) uint8_t img[8 * SP];
    __shared__ __align__(16) uint32_t simg[2 * 64];
    const int t = threadIdx.x, lane = t & 63, wv = __builtin_amdgcn_readfirstlane(t >> 6);
    const int pos = lane & 1, jj = lane >> 1;                    // the lane's block of the 32
    const uint32_t nbt = nbr / 32;
    const uint32_t tx = blockIdx.x % nbt, ty = blockIdx.x / nbt; // 32-block chunk, 16-line tile
    const uint64_t jb = (uint64_t)tx * 32 + jj;
    const int sl = jj >> 2, g = jj & 3;
    const bool rowl = out.layout == MXQ_LAYOUT_ROWS;
    const float h = kn.sr_bits == 16 ? 0x1p-17f : 0x1p-9f;
    const float h2 = 2.0f * h;
    constexpr bool kExact = FMT == MXQ_FMT_E2M3;

    const uint32_t sg = block_signs<HN>(kn, jb) >> (16 * pos);
    float v[4][16];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const uint64_t line = (uint64_t)ty * 16 + 4 * wv + u;
        const int64_t off = (int64_t)line * ld + (int64_t)jb * 32 + 16 * pos;
        const gv4u q0 = *reinterpret_cast<const MXQ_GLOBAL gv4u *>(gmem(x) + off);
        const gv4u q1 = *reinterpret_cast<const MXQ_GLOBAL gv4u *>(gmem(x) + off + 8);
        const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            v[u][2 * k] = as_f((w[k] << 16) ^ (((sg >> (2 * k)) & 1u) << 31));
            v[u][2 * k + 1] = as_f((w[k] & 0xFFFF0000u) ^ (((sg >> (2 * k + 1)) & 1u) << 31));
        }
    }
    uint8_t *const sb = reinterpret_cast<uint8_t *>(simg);
#pragma unroll
    for (int up = 0; up < 4; up += 2) {
        uint32_t sc[2];
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const uint64_t line = (uint64_t)ty * 16 + 4 * wv + up + d;
            sc[d] = col16<GRID, ROUND, HN, kExact>(v[up + d], pos, line * nbr + jb, kn, h, h2);
        }
        uint32_t wd[2][N];
        if constexpr (FMT == MXQ_FMT_E2M3) {
            f16v s0, s1;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                s0[j] = v[up][2 * j];
                s1[j] = v[up][2 * j + 1];
                s0[8 + j] = v[up + 1][2 * j];
                s1[8 + j] = v[up + 1][2 * j + 1];
            }
            uint32_t o[6];
            cvt_e2m3_32(s0, s1, level_unit<GRID, ROUND>(), o);
#pragma unroll
            for (int d = 0; d < 2; ++d)
#pragma unroll
                for (int k = 0; k < 3; ++k)
                    wd[d][k] = sc[d] == 0xFFu ? 0u : o[3 * d + k];
        } else {
#pragma unroll
            for (int d = 0; d < 2; ++d)
                pack_fp4<GRID, ROUND>(v[up + d], sc[d], wd[d]);
        }
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const int l = 4 * wv + up + d;                        // line within the tile
            uint32_t *dst = reinterpret_cast<uint32_t *>(img + sl * SP + g * GP + l * BB + pos * (BB / 2));
#pragma unroll
            for (int k = 0; k < N; ++k)
                dst[k] = wd[d][k];
            if (pos == 0)
                sb[rowl ? l * 32 + jj : ((jj >> 4) * 64 + 16 * g + l) * 4 + (sl & 3)] = (uint8_t)sc[d];
        }
    }
    __syncthreads();
    if (rowl) {
        // line runs: 16-byte unit u of line l (FP4: block u; E2M3: 8-byte
        // chunks 2 u and 2 u + 1, chunk c being bytes 8 (c % 3) of block c / 3)
        constexpr int U = 2 * BB;                                  // units per line run
        MXQ_GLOBAL uint8_t *const codes = gmem(out.codes);
#pragma unroll
        for (int k = 0; k < U / 16; ++k) {
            const int q = k * 256 + t, l = q / U, u = q - l * U;
            gv4u val;
            if constexpr (FMT == MXQ_FMT_E2M3) {
                typedef uint32_t u2v __attribute__((ext_vector_type(2)));
                u2v w2[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int c = 2 * u + e, b = c / 3;
                    w2[e] = *reinterpret_cast<const u2v *>(img + (b >> 2) * SP + (b & 3) * GP + l * BB +
                                                           (c - 3 * b) * 8);
                }
                val = gv4u{w2[0].x, w2[0].y, w2[1].x, w2[1].y};
            } else {
                val = *reinterpret_cast<const gv4u *>(img + (u >> 2) * SP + (u & 3) * GP + l * BB);
            }
            const uint64_t run = (((uint64_t)ty * 16 + l) * out.nbk + (uint64_t)tx * 32) * BB;
            __builtin_nontemporal_store(val, reinterpret_cast<MXQ_GLOBAL gv4u *>(codes + run) + u);
        }
        if (t < 128) {
            const int l = t >> 3, w = t & 7;
            reinterpret_cast<MXQ_GLOBAL uint32_t *>(
                gmem(out.scales) + ((uint64_t)ty * 16 + l) * out.nbk + (uint64_t)tx * 32)[w] = simg[t];
        }
        return;
    }
    // the 8 step runs: run r is step 8 tx + r of tile ty, 64 slots of BB bytes
    uint8_t *const codes = out.codes;
    if constexpr (FMT == MXQ_FMT_E2M3) {
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const int q = k * 256 + t, r = q / 96, uu = q - r * 96;   // 16-byte unit uu of run r
            const int gg = uu / 24, within = (uu - gg * 24) * 16;
            const uint8_t *src = img + r * SP + gg * GP + within;
            typedef uint32_t u2v __attribute__((ext_vector_type(2)));
            const u2v a = *reinterpret_cast<const u2v *>(src);
            const u2v b = *reinterpret_cast<const u2v *>(src + 8);
            const gv4u val = {a.x, a.y, b.x, b.y};
            const uint64_t run = (((uint64_t)tx * 8 + r) * out.ntiles + ty) * 64 * BB;
            __builtin_nontemporal_store(val, reinterpret_cast<MXQ_GLOBAL gv4u *>(gmem(codes) + run) + uu);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int q = k * 256 + t, r = q >> 6, L = q & 63;
            const gv4u val = *reinterpret_cast<const gv4u *>(img + r * SP + (L >> 4) * GP + (L & 15) * 16);
            const uint64_t run = (((uint64_t)tx * 8 + r) * out.ntiles + ty) * 64 * BB;
            __builtin_nontemporal_store(val, reinterpret_cast<MXQ_GLOBAL gv4u *>(gmem(codes) + run) + L);
        }
    }
    // the scale words of the tile's 2 groups
    if (t < 128) {
        const int grp = t >> 6, slot = t & 63;
        reinterpret_cast<MXQ_GLOBAL uint32_t *>(gmem(out.scales))
            [(((uint64_t)tx * 2 + grp) * out.ntiles + ty) * 64 + slot] = simg[t];
    }
}

// Both outputs from one read.  Phase 1 is k_quant_col's work on the tile
// (column blocks, 16 rows x 4 columns per lane); each lane also stores its raw
// bf16 words into an LDS image of the 128 x 128 tile.  After one barrier,
// phase 2 reads the tile's rows back from LDS and runs the row kernel's work
// on them (two lanes per row block, 16 consecutive columns each).  On a full
// tile the row codes then go back into the same LDS (after a second barrier)
// and leave like the column output: one contiguous run in the matrix-core
// layout, 128 line runs in the row layout, with the row layout's scales as
// one word per line (8.7% faster in the row layout, the same bytes).  The LDS
// image has no padding (32 KiB, so with FP4 column codes four workgroups fit
// in a CU); instead the 8-byte units of row r sit at unit ^ tile_swz(r).  The
// two 16-row halves a wave writes at once then fall 32 banks apart, and the
// 4 rows x 8 units of each 32-lane pass of a phase-2 read hit distinct banks.
constexpr int kTileRS = 256;   // LDS bytes per tile row (128 bf16)
__device__ __forceinline__ int tile_swz(int r) { return (r & 7) | (r & 16); }

template <int GRID, int ROUND, int HN, int FMTR, int FMTC>
__global__ __launch_bounds__(256) void k_quant_dual16(const uint16_t *__restrict__ x, int64_t rows,
                                                      int64_t cols, int64_t ld, OutDesc rout,
                                                      OutDesc cout, int vec, QKnobs kn)
{
    constexpr int BBC = FMTC == MXQ_FMT_E2M3 ? 24 : 16;
    __shared__ __align__(16) uint8_t tile[128 * kTileRS];
    __shared__ uint32_t stage[128 * BBC];
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int pos = lane & 1, cg = lane >> 1;
    const int64_t row0 = (int64_t)blockIdx.y * 128, col0 = (int64_t)blockIdx.x * 128;
    const int64_t rband = row0 + wv * 32;                         // rows % 32 == 0
    const bool live = rband < rows;                               // whole wave
    const bool staged = col0 + 128 <= cols && row0 + 128 <= rows;
    const float h = kn.sr_bits == 16 ? 0x1p-17f : 0x1p-9f;
    const float h2 = 2.0f * h;

    // ---- phase 1: load, stash, column blocks
    if (live) {
        const int64_t r0 = rband + 16 * pos;
        const int64_t c0 = col0 + 4 * cg;
        const uint64_t jb = (uint64_t)rband >> 5, nbc = (uint64_t)rows >> 5;
        uint32_t lo[16], hi[16];
        if (vec && c0 + 4 <= cols) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const gv2u w = *reinterpret_cast<const MXQ_GLOBAL gv2u *>(gmem(x) + (r0 + i) * ld + c0);
                lo[i] = w.x;
                hi[i] = w.y;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                uint32_t hh[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    hh[j] = (c0 + j < cols) ? (uint32_t)gmem(x)[(r0 + i) * ld + c0 + j] : 0u;
                lo[i] = hh[0] | (hh[1] << 16);
                hi[i] = hh[2] | (hh[3] << 16);
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = 32 * wv + 16 * pos + i;
            *reinterpret_cast<uint2 *>(tile + r * kTileRS + 8 * (cg ^ tile_swz(r))) =
                make_uint2(lo[i], hi[i]);
        }
        if constexpr (HN > 0) {
            const uint32_t sg = block_signs<HN>(kn, jb) >> (16 * pos);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint32_t f = ((sg >> i) & 1u) ? 0x80008000u : 0u;
                lo[i] ^= f;
                hi[i] ^= f;
            }
        }
        constexpr bool kExact = FMTC == MXQ_FMT_E2M3;
#pragma unroll
        for (int jp = 0; jp < 2; ++jp) {
            float a[16], b[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint32_t w = jp ? hi[i] : lo[i];
                a[i] = as_f(w << 16);
                b[i] = as_f(w & 0xFFFF0000u);
            }
            const int64_t ca = c0 + 2 * jp, cb = ca + 1;
            const uint32_t sa = col16<GRID, ROUND, HN, kExact>(a, pos, (uint64_t)ca * nbc + jb, kn, h, h2);
            const uint32_t sb = col16<GRID, ROUND, HN, kExact>(b, pos, (uint64_t)cb * nbc + jb, kn, h, h2);
            uint32_t wa[3], wb[3];
            if constexpr (FMTC == MXQ_FMT_E2M3) {
                f16v s0, s1;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    s0[j] = a[2 * j];
                    s1[j] = a[2 * j + 1];
                    s0[8 + j] = b[2 * j];
                    s1[8 + j] = b[2 * j + 1];
                }
                uint32_t o[6];
                cvt_e2m3_32(s0, s1, level_unit<GRID, ROUND>(), o);
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    wa[k] = sa == 0xFFu ? 0u : o[k];
                    wb[k] = sb == 0xFFu ? 0u : o[3 + k];
                }
            } else {
                uint32_t pa[2], pb[2];
                pack_fp4<GRID, ROUND>(a, sa, pa);
                pack_fp4<GRID, ROUND>(b, sb, pb);
                wa[0] = pa[0]; wa[1] = pa[1]; wb[0] = pb[0]; wb[1] = pb[1];
            }
            constexpr int N = BBC / 8;
            if (staged) {
                stage_words<N>(stage, cout.layout, 4 * cg + 2 * jp, wv, pos, wa);
                stage_words<N>(stage, cout.layout, 4 * cg + 2 * jp + 1, wv, pos, wb);
            } else {
                if (ca < cols)
                    store_words<N>(cout, (uint64_t)ca, jb, pos, wa);
                if (cb < cols)
                    store_words<N>(cout, (uint64_t)cb, jb, pos, wb);
            }
            if (pos == 0) {
                if (ca < cols)
                    gmem(cout.scales)[scale_offset(cout, (uint64_t)ca, jb)] = (uint8_t)sa;
                if (cb < cols)
                    gmem(cout.scales)[scale_offset(cout, (uint64_t)cb, jb)] = (uint8_t)sb;
            }
        }
    }
    __syncthreads();
    if (staged)
        flush_stage<BBC>(cout, stage, t, (uint64_t)col0, (uint64_t)blockIdx.y * 4);

    // ---- phase 2: row blocks of the tile from LDS: 128 rows x 4 blocks; lane pair
    // p = t >> 1 takes block p % 4 of rows p / 4 + 32 u, u = 0..3
    const uint64_t nbr = (uint64_t)cols >> 5;
    const int p = t >> 1;
    constexpr bool kExactR = FMTR == MXQ_FMT_E2M3;
    constexpr int BBR = FMTR == MXQ_FMT_E2M3 ? 24 : 16;
    // a full tile's row output is assembled in the tile's own LDS once every
    // wave has read its rows (codes in the flush order of the column output,
    // then, for the row layout, the 128 lines' scale words)
    uint32_t *const rimg = reinterpret_cast<uint32_t *>(tile);
    uint8_t *const rsb = reinterpret_cast<uint8_t *>(rimg + 128 * BBR);
    const bool swords = rout.layout == MXQ_LAYOUT_ROWS && (nbr & 3) == 0 &&
                        (reinterpret_cast<uintptr_t>(rout.scales) & 3) == 0;
    float v[4][16];
    bool ok[4];
    uint64_t rline[4], rjb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int lr = p / 4 + 32 * u, lb = p % 4;
        rline[u] = (uint64_t)(row0 + lr);
        rjb[u] = (uint64_t)(col0 / 32 + lb);
        ok[u] = (int64_t)rline[u] < rows && rjb[u] < nbr;
        const uint32_t sgr = block_signs<HN>(kn, rjb[u]) >> (16 * pos);
        const uint8_t *src = tile + lr * kTileRS;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint2 w = *reinterpret_cast<const uint2 *>(src + 8 * ((8 * lb + 4 * pos + k) ^ tile_swz(lr)));
            const uint32_t wd[2] = {w.x, w.y};
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int i = 4 * k + 2 * e;
                v[u][i] = as_f((wd[e] << 16) ^ (((sgr >> i) & 1u) << 31));
                v[u][i + 1] = as_f((wd[e] & 0xFFFF0000u) ^ (((sgr >> (i + 1)) & 1u) << 31));
            }
        }
    }
    if (staged)
        __syncthreads();                                          // the tile has been read
#pragma unroll
    for (int up = 0; up < 4; up += 2) {
        uint32_t sc[2];
#pragma unroll
        for (int d = 0; d < 2; ++d)
            sc[d] = col16<GRID, ROUND, HN, kExactR>(v[up + d], pos,
                                                    rline[up + d] * nbr + rjb[up + d], kn, h, h2);
        if constexpr (FMTR == MXQ_FMT_E2M3) {
            f16v s0, s1;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                s0[j] = v[up][2 * j];
                s1[j] = v[up][2 * j + 1];
                s0[8 + j] = v[up + 1][2 * j];
                s1[8 + j] = v[up + 1][2 * j + 1];
            }
            uint32_t o[6];
            cvt_e2m3_32(s0, s1, level_unit<GRID, ROUND>(), o);
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                uint32_t wd[3];
#pragma unroll
                for (int k = 0; k < 3; ++k)
                    wd[k] = sc[d] == 0xFFu ? 0u : o[3 * d + k];
                if (staged)
                    stage_words<3>(rimg, rout.layout, p / 4 + 32 * (up + d), p % 4, pos, wd);
                else if (ok[up + d])
                    store_words<3>(rout, rline[up + d], rjb[up + d], pos, wd);
            }
        } else {
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                uint32_t wd[2];
                pack_fp4<GRID, ROUND>(v[up + d], sc[d], wd);
                if (staged)
                    stage_words<2>(rimg, rout.layout, p / 4 + 32 * (up + d), p % 4, pos, wd);
                else if (ok[up + d])
                    store_words<2>(rout, rline[up + d], rjb[up + d], pos, wd);
            }
        }
        if (pos == 0) {
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                if (staged && swords)
                    rsb[(p / 4 + 32 * (up + d)) * 4 + p % 4] = (uint8_t)sc[d];
                else if (ok[up + d])
                    gmem(rout.scales)[scale_offset(rout, rline[up + d], rjb[up + d])] = (uint8_t)sc[d];
            }
        }
    }
    if (staged) {
        __syncthreads();
        flush_stage<BBR>(rout, rimg, t, (uint64_t)row0, (uint64_t)col0 >> 5);
        if (swords && t < 128)
            reinterpret_cast<MXQ_GLOBAL uint32_t *>(gmem(rout.scales))[((uint64_t)row0 + t) * (nbr >> 2) +
                                                                      ((uint64_t)col0 >> 7)] =
                reinterpret_cast<const uint32_t *>(rsb)[t];
    }
}

namespace {

template <int GRID, int ROUND, int HN, int FR>
void launch_dual_fc(const DualLaunch &q)
{
    const dim3 grid((unsigned)((q.cols + 127) / 128), (unsigned)((q.rows + 127) / 128));
    if (q.cout.fmt == MXQ_FMT_E2M3)
        hipLaunchKernelGGL((k_quant_dual16<GRID, ROUND, HN, FR, MXQ_FMT_E2M3>), grid, dim3(256), 0,
                           q.s, q.x, q.rows, q.cols, q.ld, q.rout, q.cout, q.vec, q.kn);
    else
        hipLaunchKernelGGL((k_quant_dual16<GRID, ROUND, HN, FR, MXQ_FMT_FP4>), grid, dim3(256), 0,
                           q.s, q.x, q.rows, q.cols, q.ld, q.rout, q.cout, q.vec, q.kn);
}

template <int GRID, int ROUND, int HN>
void launch_dual_fmt(const DualLaunch &q)
{
    if (q.rout.fmt == MXQ_FMT_E2M3)
        launch_dual_fc<GRID, ROUND, HN, MXQ_FMT_E2M3>(q);
    else
        launch_dual_fc<GRID, ROUND, HN, MXQ_FMT_FP4>(q);
}

template <int GRID, int ROUND>
void launch_dual_hn(int hn, const DualLaunch &q)
{
    switch (hn) {
    case 0: launch_dual_fmt<GRID, ROUND, 0>(q); break;
    case 16: launch_dual_fmt<GRID, ROUND, 16>(q); break;
    default: launch_dual_fmt<GRID, ROUND, 32>(q); break;
    }
}

template <int GRID, int ROUND, int HN>
void launch_row16_fmt(const RowLaunch &q)
{
    const uint64_t rows = q.nbr ? q.nblocks / q.nbr : 0;
    const bool out_ok = q.out.layout == MXQ_LAYOUT_MFMA ||
                        (reinterpret_cast<uintptr_t>(q.out.codes) % 16 == 0 &&
                         reinterpret_cast<uintptr_t>(q.out.scales) % 4 == 0);
    if (out_ok && q.vec && q.nbr % 32 == 0 && rows % 16 == 0 && rows > 0) {
        const unsigned g = (unsigned)((q.nbr / 32) * (rows / 16));
        if (q.out.fmt == MXQ_FMT_E2M3)
            hipLaunchKernelGGL((k_quant_row16m<GRID, ROUND, HN, MXQ_FMT_E2M3>), dim3(g), dim3(256), 0,
                               q.s, q.x, q.nbr, q.ld, q.out, q.kn);
        else
            hipLaunchKernelGGL((k_quant_row16m<GRID, ROUND, HN, MXQ_FMT_FP4>), dim3(g), dim3(256), 0,
                               q.s, q.x, q.nbr, q.ld, q.out, q.kn);
        return;
    }
    const unsigned grid = (unsigned)((q.nblocks + 511) / 512);
    if (q.out.fmt == MXQ_FMT_E2M3)
        hipLaunchKernelGGL((k_quant_row16<GRID, ROUND, HN, MXQ_FMT_E2M3>), dim3(grid), dim3(256),
                           0, q.s, q.x, q.nblocks, q.nbr, q.ld, q.dense, q.vec, q.out, q.kn);
    else
        hipLaunchKernelGGL((k_quant_row16<GRID, ROUND, HN, MXQ_FMT_FP4>), dim3(grid), dim3(256),
                           0, q.s, q.x, q.nblocks, q.nbr, q.ld, q.dense, q.vec, q.out, q.kn);
}

template <int GRID, int ROUND>
void launch_row16_hn(int hn, const RowLaunch &q)
{
    switch (hn) {
    case 0: launch_row16_fmt<GRID, ROUND, 0>(q); break;
    case 16: launch_row16_fmt<GRID, ROUND, 16>(q); break;
    default: launch_row16_fmt<GRID, ROUND, 32>(q); break;
    }
}

template <int GRID, int ROUND, int HN>
void launch_col_fmt(const ColLaunch &q)
{
    const dim3 grid((unsigned)((q.cols + 127) / 128), (unsigned)((q.rows + 127) / 128));
    if (q.out.fmt == MXQ_FMT_E2M3)
        hipLaunchKernelGGL((k_quant_col<GRID, ROUND, HN, MXQ_FMT_E2M3>), grid, dim3(256), 0, q.s,
                           q.x, q.rows, q.cols, q.ld, q.out, q.vec, q.kn);
    else
        hipLaunchKernelGGL((k_quant_col<GRID, ROUND, HN, MXQ_FMT_FP4>), grid, dim3(256), 0, q.s,
                           q.x, q.rows, q.cols, q.ld, q.out, q.vec, q.kn);
}

template <int GRID, int ROUND>
void launch_col_hn(int hn, const ColLaunch &q)
{
    switch (hn) {
    case 0: launch_col_fmt<GRID, ROUND, 0>(q); break;
    case 16: launch_col_fmt<GRID, ROUND, 16>(q); break;
    default: launch_col_fmt<GRID, ROUND, 32>(q); break;
    }
}

template <int GRID, int HN, int FMT>
void launch_col_batch_rmode(int rmode, const ColBatch &b, int64_t tiles, hipStream_t s)
{
    const dim3 grid((unsigned)tiles);
    if (rmode == kRTNE)
        hipLaunchKernelGGL((k_quant_col_batch<GRID, HN, FMT, kRTNE>), grid, dim3(256), 0, s, b);
    else if (rmode == kSR)
        hipLaunchKernelGGL((k_quant_col_batch<GRID, HN, FMT, kSR>), grid, dim3(256), 0, s, b);
    else
        hipLaunchKernelGGL((k_quant_col_batch<GRID, HN, FMT, kBatchMixed>), grid, dim3(256), 0,
                           s, b);
}

template <int GRID, int HN>
void launch_col_batch_fmt(int fmt, int rmode, const ColBatch &b, int64_t tiles, hipStream_t s)
{
    if (fmt == MXQ_FMT_E2M3)
        launch_col_batch_rmode<GRID, HN, MXQ_FMT_E2M3>(rmode, b, tiles, s);
    else
        launch_col_batch_rmode<GRID, HN, MXQ_FMT_FP4>(rmode, b, tiles, s);
}

template <int GRID>
void launch_col_batch_hn(int hn, int fmt, int rmode, const ColBatch &b, int64_t tiles,
                         hipStream_t s)
{
    switch (hn) {
    case 0: launch_col_batch_fmt<GRID, 0>(fmt, rmode, b, tiles, s); break;
    case 16: launch_col_batch_fmt<GRID, 16>(fmt, rmode, b, tiles, s); break;
    default: launch_col_batch_fmt<GRID, 32>(fmt, rmode, b, tiles, s); break;
    }
}

}  // namespace

hipError_t launch_quant_col_batch(int grid, int hn, int fmt, const ColBatch &b, int64_t tiles,
                                  hipStream_t s)
{
    bool sr = false, rtne = false;
    for (int i = 0; i < b.n; ++i)
        (b.job[i].round == kSR ? sr : rtne) = true;
    const int rmode = sr && rtne ? kBatchMixed : sr ? kSR : kRTNE;
    if (grid == kE2M1)
        launch_col_batch_hn<kE2M1>(hn, fmt, rmode, b, tiles, s);
    else
        launch_col_batch_hn<kE1M2>(hn, fmt, rmode, b, tiles, s);
    return hipGetLastError();
}

hipError_t launch_quant_dual16(int grid, int round, int hn, const DualLaunch &q)
{
    if (grid == kE2M1)
        round == kRTNE ? launch_dual_hn<kE2M1, kRTNE>(hn, q) : launch_dual_hn<kE2M1, kSR>(hn, q);
    else
        round == kRTNE ? launch_dual_hn<kE1M2, kRTNE>(hn, q) : launch_dual_hn<kE1M2, kSR>(hn, q);
    return hipGetLastError();
}

hipError_t launch_quant_row16(int grid, int round, int hn, const RowLaunch &q)
{
    if (grid == kE2M1)
        round == kRTNE ? launch_row16_hn<kE2M1, kRTNE>(hn, q) : launch_row16_hn<kE2M1, kSR>(hn, q);
    else
        round == kRTNE ? launch_row16_hn<kE1M2, kRTNE>(hn, q) : launch_row16_hn<kE1M2, kSR>(hn, q);
    return hipGetLastError();
}

hipError_t launch_quant_col(int grid, int round, int hn, const ColLaunch &q)
{
    if (grid == kE2M1)
        round == kRTNE ? launch_col_hn<kE2M1, kRTNE>(hn, q) : launch_col_hn<kE2M1, kSR>(hn, q);
    else
        round == kRTNE ? launch_col_hn<kE1M2, kRTNE>(hn, q) : launch_col_hn<kE1M2, kSR>(hn, q);
    return hipGetLastError();
}

}  // namespace mxq
