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
#include <type_traits>

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

// ---- LDS-staged kernel -----------------------------------------------------
// Workgroup tile 256 x 256 (4 waves of 128 x 128 = 8 x 8 MFMA tiles of
// 16 x 16); one K step = 128 = 4 blocks per row.
//
// Block assignment: K steps come in groups of 4 (16 blocks = 512 K).  At step
// s' of group q, lane group g takes block 16 q + 4 g + s'.  A lane's 4 scale
// bytes for the group are then the contiguous dword at scales[row][16 q + 4 g],
// with byte s' for step s'; A and B use the same assignment, so the product is
// unchanged (only the fp32 summation order depends on it).
//
// Staging: operand bytes go from global memory straight into LDS with
// global_load_lds, which writes lane L's 16 (dwordx4) or 12 (dwordx3) bytes at
// 16 L.  Layout "fragment-major": for each 16-row tile, fragment lane
// l = 16 g + r's block bytes sit at 16 l -- one 1 KB region for an FP4 block,
// two (bytes 0-11 and 12-23) for an FP6 block -- so every fragment read is a
// contiguous, bank-conflict-free 128-bit sweep.  Two stages alternate: the next step's loads are
// in flight during this step's MFMAs.  Scales are staged per group, [row][16 B].
constexpr int kBM = 256, kBN = 256;

template <int F> constexpr int blk_bytes() { return F == kMfmaFP4 ? 16 : 24; }

template <int F> constexpr int tile_bytes() { return F == kMfmaFP4 ? 1024 : 2048; }

template <int FA, int FB>
constexpr int lds_bytes() { return 2 * 16 * (tile_bytes<FA>() + tile_bytes<FB>()) + 2 * 2 * 4096; }

typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void glb_void;

__device__ __forceinline__ void g2l16(const uint8_t *g, uint8_t *l)
{
    __builtin_amdgcn_global_load_lds((glb_void *)g, (lds_void *)l, 16, 0, 0);
}
__device__ __forceinline__ void g2l12(const uint8_t *g, uint8_t *l)
{
    __builtin_amdgcn_global_load_lds((glb_void *)g, (lds_void *)l, 12, 0, 0);
}

// This wave's share (4 of the 16 row tiles) of one operand's K step.
template <int F>
__device__ __forceinline__ void stage_step(const uint8_t *__restrict__ codes, int64_t row0,
                                           int64_t rows, int64_t nbk, int64_t q, int sp,
                                           uint8_t *lds_stage, int wv, int lane)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rt = 4 * wv + i;
        if constexpr (F == kMfmaFP4) {
            const int g = lane >> 4, rr = lane & 15;
            const int64_t rg = min(row0 + 16 * rt + rr, rows - 1);
            g2l16(codes + (rg * nbk + 16 * q + 4 * g + sp) * 16, lds_stage + rt * 1024);
        } else {
            const int g = lane >> 4, rr = lane & 15;
            const int64_t rg = min(row0 + 16 * rt + rr, rows - 1);
            const uint8_t *src = codes + (rg * nbk + 16 * q + 4 * g + sp) * 24;
            g2l12(src, lds_stage + rt * 2048);
            g2l12(src + 12, lds_stage + rt * 2048 + 1024);
        }
    }
}

// This wave's 64 rows of one operand's scale group (16 bytes per row).
__device__ __forceinline__ void stage_scales(const uint8_t *__restrict__ scales, int64_t row0,
                                             int64_t rows, int64_t nbk, int64_t q, uint8_t *lds,
                                             int wv, int lane)
{
    const int64_t rg = min(row0 + 64 * wv + lane, rows - 1);
    g2l16(scales + rg * nbk + 16 * q, lds + 64 * wv * 16);
}

template <int F>
__device__ __forceinline__ v8i lds_fragment(const uint8_t *__restrict__ lds, int rt, int lane)
{
    v8i r = {0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (F == kMfmaFP4) {
        const uint4 q = *reinterpret_cast<const uint4 *>(lds + rt * 1024 + lane * 16);
        r[0] = (int)q.x; r[1] = (int)q.y; r[2] = (int)q.z; r[3] = (int)q.w;
    } else {
        const uint4 a = *reinterpret_cast<const uint4 *>(lds + rt * 2048 + lane * 16);
        const uint4 b = *reinterpret_cast<const uint4 *>(lds + rt * 2048 + 1024 + lane * 16);
        r[0] = (int)a.x; r[1] = (int)a.y; r[2] = (int)a.z;
        r[3] = (int)b.x; r[4] = (int)b.y; r[5] = (int)b.z;
    }
    return r;
}

// Tile order: workgroups go round-robin over the 8 XCDs; give each XCD a
// contiguous run of tiles, grouped 4 tile-rows deep, so the tiles sharing an
// XCD's L2 share A and B panels.
__device__ __forceinline__ void tile_of(int w, int ntm, int ntn, int &tm, int &tn)
{
    const int total = ntm * ntn;
    if (total % 8 == 0)
        w = (w % 8) * (total / 8) + w / 8;
    constexpr int GM = 4;
    const int gsize = GM * ntn;
    const int grp = w / gsize;
    const int first = grp * GM;
    const int gm = min(ntm - first, GM);
    const int loc = w - grp * gsize;
    tm = first + loc % gm;
    tn = loc / gm;
}

template <int FA, int FB>
__global__ __launch_bounds__(256, 1) void k_wgrad_lds(const uint8_t *__restrict__ ac,
                                                      const uint8_t *__restrict__ as,
                                                      const uint8_t *__restrict__ bc,
                                                      const uint8_t *__restrict__ bs, int64_t m,
                                                      int64_t n, int64_t k, float *__restrict__ c,
                                                      int64_t ldc)
{
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int SA = 16 * tile_bytes<FA>(), SB = 16 * tile_bytes<FB>();
    constexpr int STAGE = SA + SB;
    uint8_t *const scl = smem + 2 * STAGE;     // [2 groups][A 4 KB | B 4 KB]

    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int wm = wv >> 1, wn = wv & 1, g = lane >> 4, li = lane & 15;
    int tm, tn;
    tile_of(blockIdx.x, (int)((m + kBM - 1) / kBM), (int)((n + kBN - 1) / kBN), tm, tn);
    const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
    const int64_t nbk = k / 32, nsteps = k / 128;

    v4f acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

    // prologue: scales of group 0, operands of step 0
    stage_scales(as, m0, m, nbk, 0, scl, wv, lane);
    stage_scales(bs, n0, n, nbk, 0, scl + 4096, wv, lane);
    stage_step<FA>(ac, m0, m, nbk, 0, 0, smem, wv, lane);
    stage_step<FB>(bc, n0, n, nbk, 0, 0, smem + SA, wv, lane);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    uint32_t sca[8], scb[8];
    for (int64_t s = 0; s < nsteps; ++s) {
        const int cur = (int)(s & 1);
        const int64_t q = s >> 2;
        const int sp = (int)(s & 3);
        if (s + 1 < nsteps) {
            const int64_t q1 = (s + 1) >> 2;
            const int sp1 = (int)((s + 1) & 3);
            uint8_t *nxt = smem + (cur ^ 1) * STAGE;
            stage_step<FA>(ac, m0, m, nbk, q1, sp1, nxt, wv, lane);
            stage_step<FB>(bc, n0, n, nbk, q1, sp1, nxt + SA, wv, lane);
        }
        if (sp == 0) {
            const uint8_t *sgA = scl + (q & 1) * 8192, *sgB = sgA + 4096;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                sca[i] = *reinterpret_cast<const uint32_t *>(sgA + (128 * wm + 16 * i + li) * 16 + 4 * g);
                scb[i] = *reinterpret_cast<const uint32_t *>(sgB + (128 * wn + 16 * i + li) * 16 + 4 * g);
            }
            if (4 * (q + 1) < nsteps) {
                // the other group buffer was last read at step 4 (q - 1)
                uint8_t *sg1 = scl + ((q + 1) & 1) * 8192;
                stage_scales(as, m0, m, nbk, q + 1, sg1, wv, lane);
                stage_scales(bs, n0, n, nbk, q + 1, sg1 + 4096, wv, lane);
            }
        }
        const uint8_t *stg = smem + cur * STAGE;
        const int sh = 8 * sp;
        v8i bf[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            bf[j] = lds_fragment<FB>(stg + SA, 8 * wn + j, lane);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const v8i af = lds_fragment<FA>(stg, 8 * wm + i, lane);
            const int sai = (int)((sca[i] >> sh) & 0xFFu);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    af, bf[j], acc[i][j], FA, FB, 0, sai, 0, (int)((scb[j] >> sh) & 0xFFu));
        }
        __builtin_amdgcn_s_waitcnt(0);   // this wave's loads into the other stage landed
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t col = n0 + 128 * wn + 16 * j + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + 128 * wm + 16 * i + 4 * g + r;
                if (row < m && col < n)
                    c[row * ldc + col] = acc[i][j][r];
            }
        }
}

// ---- MFMA-tiled operands -----------------------------------------------------
// Both operands in MXQ_LAYOUT_MFMA: a K step of one 16-row tile is one
// contiguous 1 KB (FP4) or 1.5 KB (FP6) fragment, already in lane order, and
// the 16 tiles a workgroup needs for a step are adjacent.  8 waves (2 per
// SIMD) of 128 x 64 output each cover a 256 x 256 tile.  The step's operand
// bytes are copied verbatim into LDS with 16-byte direct loads (lane order ==
// memory order), issued one step ahead into a second buffer.  The copies are
// issued from inline asm so the compiler, which cannot tell them apart from
// the buffer being read, does not drain them before every LDS read; their
// completion is awaited explicitly (vmcnt) before the barrier that publishes
// the buffer.  A lane's 4 scale bytes per 4-step group come straight from
// global memory, one dword per fragment row, a group ahead.
// k_wgrad_tiled is that 2-stage form; it serves scale arrays that are not
// 16-byte aligned.  Aligned ones take k_wgrad_ring3 below (3 stages, scale
// words copied through LDS), which issues the same products in the same order.
constexpr int kWaves = 8;

// M0 is a register the compiler reserves (it may hold a live value of its own
// across this statement, e.g. for an LDS instruction it emitted), so the copy
// saves it into an SGPR of its own, points it at the LDS destination, and puts
// the saved value back before the statement ends.  The load takes M0 when it
// is issued, so the restore right behind it does not change the copy.  The
// build treats -Winline-asm as an error, so a reserved register can never sit
// on a clobber list unnoticed.
__device__ __forceinline__ void dma16(const uint8_t *g, const uint8_t *l)
{
    const uint32_t la = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const uint8_t *)l);
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\t"
                 "s_mov_b32 m0, %2\n\t"
                 "s_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, off\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(g), "s"(__builtin_amdgcn_readfirstlane(la))
                 : "memory");
}

// The same copy with the global address split into a wave-uniform 64-bit base
// (scalar registers) and a 32-bit per-lane offset, so a step's new base is
// scalar arithmetic only.
__device__ __forceinline__ void dma16_so(const uint8_t *base, uint32_t off, const uint8_t *l)
{
    const uint32_t la = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const uint8_t *)l);
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\t"
                 "s_mov_b32 m0, %3\n\t"
                 "s_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, %2\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(off), "s"(base), "s"(__builtin_amdgcn_readfirstlane(la))
                 : "memory");
}

__device__ __forceinline__ void wait_all_vm()
{
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt/lgkmcnt untouched
}

__device__ __forceinline__ void barrier_no_fence()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int F>
__device__ __forceinline__ v8i tiled_fragment(const uint8_t *__restrict__ lds, int rt, int lane)
{
    v8i r = {0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (F == kMfmaFP4) {
        const uint4 q = *reinterpret_cast<const uint4 *>(lds + rt * 1024 + lane * 16);
        r[0] = (int)q.x; r[1] = (int)q.y; r[2] = (int)q.z; r[3] = (int)q.w;
    } else {
        // three 8-byte reads off one base with immediate offsets; volatile keeps
        // the compiler from pairing words of different fragments into one
        // read (whose halves then need register moves)
        typedef __attribute__((address_space(3))) const volatile uint64_t lds_u64;
        lds_u64 *p = (lds_u64 *)(__attribute__((address_space(3))) const uint8_t *)(lds + rt * 1536 + lane * 24);
        const uint64_t a = p[0], b = p[1], c = p[2];
        r[0] = (int)(uint32_t)a; r[1] = (int)(uint32_t)(a >> 32);
        r[2] = (int)(uint32_t)b; r[3] = (int)(uint32_t)(b >> 32);
        r[4] = (int)(uint32_t)c; r[5] = (int)(uint32_t)(c >> 32);
    }
    return r;
}

template <int FA, int FB>
constexpr int tiled_lds_bytes() { return 2 * 16 * 64 * (blk_bytes<FA>() + blk_bytes<FB>()); }

template <int FA, int FB>
__global__ __launch_bounds__(64 * kWaves, 1) void k_wgrad_tiled(const uint8_t *__restrict__ ac,
                                                                const uint8_t *__restrict__ as,
                                                                const uint8_t *__restrict__ bc,
                                                                const uint8_t *__restrict__ bs,
                                                                int64_t m, int64_t n, int64_t k,
                                                                float *__restrict__ c, int64_t ldc)
{
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int SA = 16 * 64 * blk_bytes<FA>(), SB = 16 * 64 * blk_bytes<FB>();
    constexpr int STAGE = SA + SB;
    constexpr int CA = SA / 1024, CB = SB / 1024;          // 1 KB chunks per operand
    constexpr int PER = (CA + CB) / kWaves;                // chunks per wave per step

    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int wm = wv >> 2, wn = wv & 3, g = lane >> 4, li = lane & 15;
    int tm, tn;
    tile_of(blockIdx.x, (int)((m + kBM - 1) / kBM), (int)((n + kBN - 1) / kBN), tm, tn);
    const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
    const int64_t ntA = (m + 15) / 16, ntB = (n + 15) / 16;
    const int64_t nsteps = k / 128;

    // This wave's chunks: a contiguous run over [A chunks | B chunks].  Each
    // lane's source offset inside a step and its LDS slot are the same for
    // every step, so they are computed once; a step only adds its stride.
    constexpr int TBA = 64 * blk_bytes<FA>(), TBB = 64 * blk_bytes<FB>();
    uint32_t goff[PER];      // byte offset inside the operand's step
    bool isA[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int ch = wv * PER + i;
        isA[i] = ch < CA;
        const int cc = isA[i] ? ch : ch - CA;
        const int tb = isA[i] ? TBA : TBB;
        const int o = cc * 1024 + lane * 16;
        // clamp tiles past the operand's last one (their rows are never stored)
        const int64_t tile = isA[i] ? min(m0 / 16 + o / TBA, ntA - 1) : min(n0 / 16 + o / TBB, ntB - 1);
        goff[i] = (uint32_t)(tile * tb + o % tb);
    }
    auto stage = [&](int64_t s, uint8_t *buf) {
        const uint8_t *sa_ = ac + s * ntA * TBA, *sb_ = bc + s * ntB * TBB;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int ch = wv * PER + i;
            dma16((isA[i] ? sa_ : sb_) + goff[i], buf + (isA[i] ? ch * 1024 : SA + (ch - CA) * 1024));
        }
    };
    const uint32_t *sA = reinterpret_cast<const uint32_t *>(as);
    const uint32_t *sB = reinterpret_cast<const uint32_t *>(bs);
    const int64_t ta0 = m0 / 16 + 8 * wm, tb0 = n0 / 16 + 4 * wn;
    uint32_t ca[8], cb[4], na[8], nb[4];
    auto scales = [&](int64_t q, uint32_t (&xa)[8], uint32_t (&xb)[4]) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            xa[i] = sA[(q * ntA + min(ta0 + i, ntA - 1)) * 64 + lane];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            xb[j] = sB[(q * ntB + min(tb0 + j, ntB - 1)) * 64 + lane];
    };

    v4f acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

    scales(0, ca, cb);
    stage(0, smem);
    for (int64_t s = 0; s < nsteps; ++s) {
        const int cur = (int)(s & 1);
        wait_all_vm();                 // this wave's copies for step s (and scale loads) landed
        barrier_no_fence();            // ... and everyone's; step s-1's buffer is free
        if ((s & 3) == 0 && s > 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                ca[i] = na[i];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                cb[j] = nb[j];
        }
        if (s + 1 < nsteps)
            stage(s + 1, smem + (cur ^ 1) * STAGE);
        if ((s & 3) == 0 && 4 * (s / 4 + 1) < nsteps)
            scales(s / 4 + 1, na, nb);
        const uint8_t *st = smem + cur * STAGE;
        const int sh = 8 * (int)(s & 3);
        v8i bf[4];
        int sb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bf[j] = tiled_fragment<FB>(st + SA, 4 * wn + j, lane);
            sb[j] = (int)((cb[j] >> sh) & 0xFFu);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const v8i af = tiled_fragment<FA>(st, 8 * wm + i, lane);
            const int sa = (int)((ca[i] >> sh) & 0xFFu);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    af, bf[j], acc[i][j], FA, FB, 0, sa, 0, sb[j]);
        }
    }

#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = n0 + 64 * wn + 16 * j + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + 128 * wm + 16 * i + 4 * g + r;
                if (row < m && col < n)
                    c[row * ldc + col] = acc[i][j][r];
            }
        }
}

// ---- 3-stage ring ------------------------------------------------------------
// The product and tiling of k_wgrad_tiled, with each step's copies issued two
// steps ahead into a 3-stage LDS ring.  A copy reaches LDS about a microsecond
// after it is issued, longer than one step's products take, so with one step of
// lead the waves wait on the copies at every barrier; two steps of lead hide
// that.  Each step waits only for its own copies (vmcnt = the number of copies
// issued since, i.e. those of the next step), so the next step's copies stay in
// flight across the barrier.  That holds only while the loop has no other
// vector-memory load outstanding: a compiler-generated wait for such a load
// would also drain every copy issued after it.  So the scale words come through
// LDS too: with a 4-step group's first step, the 16 A and 16 B tiles' scale
// words of that group (2 x 4 KiB, one 1 KiB copy per wave) go into one of two
// group buffers, and each lane reads its 12 words from there.
// Between the products the loop holds almost no vector (VALU) instructions,
// which share the issue slots of the matrix cores: the scale byte of a step is
// picked by the product instruction itself (op_sel), and the copy addresses are
// a scalar base per step plus a fixed per-lane offset.
// A step reads all twelve of its fragments before it issues its copies, in the
// order the products use them: LDS answers a wave's reads in order, so the
// first product waits for two fragments only, and the copies, whose issue can
// hold a wave while the address unit is busy, come after the reads instead of
// in front of them (3-4% faster than reading A fragment i + 1 during row i).
// A wave's 128 x 64 accumulator tile to C through 4 KiB of LDS, 16 rows at a
// time.  Lane (g, li) holds rows 4 g .. 4 g + 3 of column 16 j + li; the rows
// go back out as 16-byte pieces (lane L: row 4 k + L / 16, columns
// 4 (L % 16) .. + 3), so each store writes four 256-byte row runs instead of
// sixteen 64-byte ones.  Element (R, C) of the 16 x 64 slab sits at
// R * 64 + 4 ((C / 4) ^ (4 (R / 4))) + C % 4, which puts the four row quads of
// a write on distinct banks.  The stores are nontemporal: C is not read again
// here, and the operand panels that other workgroups still read keep the cache.
__device__ __forceinline__ void store_tile_lds(const v4f (&acc)[8][4], float *lw, float *c,
                                               int64_t ldc, int64_t row0, int64_t col0, int lane)
{
    const int g = lane >> 4, li = lane & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                lw[(4 * g + r) * 64 + 4 * ((4 * j + (li >> 2)) ^ (4 * g)) + (li & 3)] = acc[i][j][r];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int R = 4 * k + g;
            const v4f v = *reinterpret_cast<const v4f *>(lw + R * 64 + 4 * (li ^ (4 * k)));
            __builtin_nontemporal_store(
                v, reinterpret_cast<v4f *>(c + (row0 + 16 * i + R) * ldc + col0 + 4 * li));
        }
    }
}

template <int FA, int FB>
constexpr int ring3_lds_bytes() { return 3 * 16 * 64 * (blk_bytes<FA>() + blk_bytes<FB>()) + 2 * 8192; }

template <int FA, int FB>
__global__ __launch_bounds__(64 * kWaves, 1) void k_wgrad_ring3(const uint8_t *__restrict__ ac,
                                                                const uint8_t *__restrict__ as,
                                                                const uint8_t *__restrict__ bc,
                                                                const uint8_t *__restrict__ bs,
                                                                int64_t m, int64_t n, int64_t k,
                                                                float *__restrict__ c, int64_t ldc)
{
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int SA = 16 * 64 * blk_bytes<FA>(), SB = 16 * 64 * blk_bytes<FB>();
    constexpr int STAGE = SA + SB;
    constexpr int CA = SA / 1024, CB = SB / 1024;          // 1 KB chunks per operand
    constexpr int PER = (CA + CB) / kWaves;                // chunks per wave per step
    static_assert(PER * kWaves == CA + CB, "chunks split evenly over the waves");
    static_assert(kWaves == 8, "one scale chunk per wave: 4 of A, 4 of B");
    static_assert(STAGE >= kWaves * 4096, "a ring slot holds every wave's 4 KiB output slab");
    uint8_t *const scl = smem + 3 * STAGE;                 // 2 group buffers of 8 KiB

    // the wave index is uniform across the wave: taken into a scalar register so
    // the copy addresses are scalar arithmetic
    const int t = threadIdx.x, lane = t & 63, wv = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wv >> 2, wn = wv & 3, g = lane >> 4, li = lane & 15;
    int tm, tn;
    tile_of(blockIdx.x, (int)((m + kBM - 1) / kBM), (int)((n + kBN - 1) / kBN), tm, tn);
    const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
    const int64_t ntA = (m + 15) / 16, ntB = (n + 15) / 16;
    const int nsteps = (int)(k / 128);

    // operand chunks, as in k_wgrad_tiled
    constexpr int TBA = 64 * blk_bytes<FA>(), TBB = 64 * blk_bytes<FB>();
    uint32_t goff[PER];
    bool isA[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int ch = wv * PER + i;
        isA[i] = ch < CA;
        const int cc = isA[i] ? ch : ch - CA;
        const int tb = isA[i] ? TBA : TBB;
        const int o = cc * 1024 + lane * 16;
        const int64_t tile = isA[i] ? min(m0 / 16 + o / TBA, ntA - 1) : min(n0 / 16 + o / TBB, ntB - 1);
        goff[i] = (uint32_t)(tile * tb + o % tb);
    }
    // this wave's scale chunk of a group: wave w < 4 copies A tiles 4w .. 4w + 3
    // of the workgroup's 16, wave w >= 4 B tiles 4 (w - 4) ..; lane L carries
    // the words of lanes 4 (L % 16) .. + 3 of tile 4 (w % 4) + L / 16, so the
    // buffer holds [A 16 tiles | B 16 tiles][64 lanes][4 B] (tiles past the
    // operand's last are clamped, as for the codes)
    const bool sIsA = wv < 4;
    const int64_t stile = sIsA ? min(m0 / 16 + 4 * (wv & 3) + lane / 16, ntA - 1)
                               : min(n0 / 16 + 4 * (wv & 3) + lane / 16, ntB - 1);
    const int64_t sstride = (sIsA ? ntA : ntB) * 256;    // bytes per group
    // copy sources as a wave-uniform base (scalar registers) plus a 32-bit
    // per-lane offset (the host keeps one step of an operand below 4 GiB)
    const uint8_t *const sbase0 = sIsA ? as : bs;
    const uint32_t soffl = (uint32_t)(stile * 256 + (lane & 15) * 16);
    auto stage = [&](int s, uint8_t *buf) {
        const uint8_t *sa_ = ac + (int64_t)s * ntA * TBA, *sb_ = bc + (int64_t)s * ntB * TBB;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int ch = wv * PER + i;
            dma16_so(isA[i] ? sa_ : sb_, goff[i], buf + (isA[i] ? ch * 1024 : SA + (ch - CA) * 1024));
        }
        if ((s & 3) == 0)
            dma16_so(sbase0 + (int64_t)(s >> 2) * sstride, soffl, scl + ((s >> 2) & 1) * 8192 + wv * 1024);
    };

    v4f acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

    stage(0, smem);
    if (nsteps > 1)
        stage(1, smem + STAGE);
    uint32_t ca[8], cb[4];
    int cur = 0, nxt2 = 2;                  // ring slots of steps s and s + 2
    // One step.  Q = s % 4 is the byte of the scale words the matrix cores use,
    // selected by the instruction's op_sel, so no scale byte is extracted by a
    // vector instruction between the products (the loop below unrolls the four
    // steps of a scale group).
    auto step = [&](int s, auto QC) {
        constexpr int Q = decltype(QC)::value;
        // this wave's copies for step s landed (those of step s + 1, issued
        // after them, may still be in flight) ...
        if (s + 1 >= nsteps)
            wait_all_vm();
        else if (((s + 1) & 3) == 0)
            __builtin_amdgcn_s_waitcnt(0x0F70 | (PER + 1));
        else
            __builtin_amdgcn_s_waitcnt(0x0F70 | PER);
        barrier_no_fence();                 // ... and everyone's; step s-1's slot is free
        if constexpr (Q == 0) {
            const uint32_t *sg = reinterpret_cast<const uint32_t *>(scl + ((s >> 2) & 1) * 8192);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                ca[i] = sg[(8 * wm + i) * 64 + lane];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                cb[j] = sg[1024 + (4 * wn + j) * 64 + lane];
        }
        const uint8_t *st = smem + cur * STAGE;
        // every fragment of the step read up front, in the order of use, then
        // the copies of step s + 2
        v8i bf[4];
        v8i af[8];
        af[0] = tiled_fragment<FA>(st, 8 * wm, lane);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bf[j] = tiled_fragment<FB>(st + SA, 4 * wn + j, lane);
#pragma unroll
        for (int i = 1; i < 8; ++i)
            af[i] = tiled_fragment<FA>(st, 8 * wm + i, lane);
        __builtin_amdgcn_sched_barrier(0);
        if (s + 2 < nsteps)
            stage(s + 2, smem + nxt2 * STAGE);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    af[i], bf[j], acc[i][j], FA, FB, Q, (int)ca[i], Q, (int)cb[j]);
        }
        cur = cur == 2 ? 0 : cur + 1;
        nxt2 = nxt2 == 2 ? 0 : nxt2 + 1;
    };
    for (int s = 0; s < nsteps; s += 4) {
        step(s, std::integral_constant<int, 0>{});
        if (s + 1 < nsteps) step(s + 1, std::integral_constant<int, 1>{});
        if (s + 2 < nsteps) step(s + 2, std::integral_constant<int, 2>{});
        if (s + 3 < nsteps) step(s + 3, std::integral_constant<int, 3>{});
    }

    // a whole tile leaves through LDS as 16-byte row pieces: the ring slot of
    // step nsteps (that of step nsteps - 3, read by every wave before the last
    // barrier, with no copy pending) holds each wave's 4 KiB
    if (m0 + kBM <= m && n0 + kBN <= n && (ldc & 3) == 0 && ((uintptr_t)c & 15) == 0) {
        float *lw = reinterpret_cast<float *>(smem + cur * STAGE) + wv * 1024;
        store_tile_lds(acc, lw, c, ldc, m0 + 128 * wm, n0 + 64 * wn, lane);
        return;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = n0 + 64 * wn + 16 * j + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + 128 * wm + 16 * i + 4 * g + r;
                if (row < m && col < n)
                    c[row * ldc + col] = acc[i][j][r];
            }
        }
}

// The ring kernel for FP4 operands with the fragment reads one step ahead.
// In k_wgrad_ring3 every wave reads a step's fragments right after the step's
// barrier and then issues its products, so all waves read the LDS at the same
// time and then all keep the matrix cores busy at the same time: the reads
// and copies add to the products instead of overlapping them.  Here a wave
// reads step s + 1's fragments into a second register set right after the
// barrier of step s and then issues step s's products (whose fragments it
// read during step s - 1), so the LDS reads and the copies run while the
// products do.  Two fragment sets take 2 x 48 registers with FP4 operands
// (FP6 would need 2 x 72 and no longer fit two waves per SIMD), and the reads
// of step s + 1 need its copies landed by the barrier of step s, so the ring
// has four slots (copies of step s + 3 issued in step s: a two-step lead
// again).  The loop has no branches (a branch would make the compiler's
// counter bookkeeping assume the products wait for the reads just issued):
// k is a multiple of 512, and past the last step the reads are unused and
// the copies rewrite step s - 1's bytes into its own slot.
template <int FA, int FB>
constexpr int ra4_lds_bytes() { return 4 * 16 * 64 * (blk_bytes<FA>() + blk_bytes<FB>()) + 2 * 8192; }

template <int FA, int FB>
__global__ __launch_bounds__(64 * kWaves, 1) void k_wgrad_ra4(const uint8_t *__restrict__ ac,
                                                                const uint8_t *__restrict__ as,
                                                                const uint8_t *__restrict__ bc,
                                                                const uint8_t *__restrict__ bs,
                                                                int64_t m, int64_t n, int64_t k,
                                                                float *__restrict__ c, int64_t ldc)
{
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int SA = 16 * 64 * blk_bytes<FA>(), SB = 16 * 64 * blk_bytes<FB>();
    constexpr int STAGE = SA + SB;
    constexpr int CA = SA / 1024, CB = SB / 1024;          // 1 KB chunks per operand
    constexpr int PER = (CA + CB) / kWaves;                // chunks per wave per step
    static_assert(PER * kWaves == CA + CB, "chunks split evenly over the waves");
    static_assert(kWaves == 8, "one scale chunk per wave: 4 of A, 4 of B");
    static_assert(STAGE >= kWaves * 4096, "a ring slot holds every wave's 4 KiB output slab");
    uint8_t *const scl = smem + 4 * STAGE;                 // 2 group buffers of 8 KiB

    // the wave index is uniform across the wave: taken into a scalar register so
    // the copy addresses are scalar arithmetic
    const int t = threadIdx.x, lane = t & 63, wv = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wv >> 2, wn = wv & 3, g = lane >> 4, li = lane & 15;
    int tm, tn;
    tile_of(blockIdx.x, (int)((m + kBM - 1) / kBM), (int)((n + kBN - 1) / kBN), tm, tn);
    const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
    const int64_t ntA = (m + 15) / 16, ntB = (n + 15) / 16;
    const int nsteps = (int)(k / 128);

    // operand chunks: with FP4 a 1 KiB chunk is one 16-row tile, so a chunk's
    // source is a wave-uniform tile offset plus 16 bytes per lane
    static_assert(FA == kMfmaFP4 && FB == kMfmaFP4, "FP4 operands only");
    uint32_t gsc[PER];
    bool isA[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int ch = wv * PER + i;
        isA[i] = ch < CA;
        const int cc = isA[i] ? ch : ch - CA;
        const int64_t tile = isA[i] ? min(m0 / 16 + cc, ntA - 1) : min(n0 / 16 + cc, ntB - 1);
        gsc[i] = (uint32_t)(tile * 1024);
    }
    const uint32_t lofs = (uint32_t)lane * 16;
    // this wave's scale chunk of a group: wave w < 4 copies A tiles 4w .. 4w + 3
    // of the workgroup's 16, wave w >= 4 B tiles 4 (w - 4) ..; lane L carries
    // the words of lanes 4 (L % 16) .. + 3 of tile 4 (w % 4) + L / 16, so the
    // buffer holds [A 16 tiles | B 16 tiles][64 lanes][4 B] (tiles past the
    // operand's last are clamped, as for the codes)
    const bool sIsA = wv < 4;
    const int64_t stile = sIsA ? min(m0 / 16 + 4 * (wv & 3) + lane / 16, ntA - 1)
                               : min(n0 / 16 + 4 * (wv & 3) + lane / 16, ntB - 1);
    const int64_t sstride = (sIsA ? ntA : ntB) * 256;    // bytes per group
    // copy sources as a wave-uniform base (scalar registers) plus a 32-bit
    // per-lane offset (the host keeps one step of an operand below 4 GiB)
    const uint8_t *const sbase0 = sIsA ? as : bs;
    const uint32_t soffl = (uint32_t)(stile * 256 + (lane & 15) * 16);
    auto stage = [&](int s, uint8_t *buf) {
        const uint8_t *sa_ = ac + (int64_t)s * ntA * 1024, *sb_ = bc + (int64_t)s * ntB * 1024;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int ch = wv * PER + i;
            dma16_so((isA[i] ? sa_ : sb_) + gsc[i], lofs, buf + (isA[i] ? ch * 1024 : SA + (ch - CA) * 1024));
        }
        if ((s & 3) == 0)
            dma16_so(sbase0 + (int64_t)(s >> 2) * sstride, soffl, scl + ((s >> 2) & 1) * 8192 + wv * 1024);
    };

    v4f acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

    // k % 512 == 0 and k >= 512 (the host checks): nsteps is a multiple of 4
    stage(0, smem);
    stage(1, smem + STAGE);
    stage(2, smem + 2 * STAGE);
    __builtin_amdgcn_s_waitcnt(0x0070 | (2 * PER));  // step 0's copies landed
    barrier_no_fence();
    uint32_t ca[8], cb[4];
    auto read_scales = [&](int grp) {
        const uint32_t *sg = reinterpret_cast<const uint32_t *>(scl + (grp & 1) * 8192);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            ca[i] = sg[(8 * wm + i) * 64 + lane];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            cb[j] = sg[1024 + (4 * wn + j) * 64 + lane];
    };
    v8i af[2][8], bf[2][4];
    auto read_frags = [&](int set, const uint8_t *st) {
        af[set][0] = tiled_fragment<FA>(st, 8 * wm, lane);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bf[set][j] = tiled_fragment<FB>(st + SA, 4 * wn + j, lane);
#pragma unroll
        for (int i = 1; i < 8; ++i)
            af[set][i] = tiled_fragment<FA>(st, 8 * wm + i, lane);
    };
    read_scales(0);
    read_frags(0, smem);
    // One step, without branches.  Its fragments were read during the previous
    // step; after the barrier the wave reads those of step s + 1 into the other
    // register set and issues the copies of step s + 3, then the products of
    // step s run while those reads and copies are in flight.  Past the last
    // step the reads are left unused and the copies rewrite step s - 1 into
    // its own slot (the same bytes, and the same number of copies, so the
    // waits stay exact).
    auto step = [&](int s, auto QC) {
        constexpr int Q = decltype(QC)::value;
        constexpr int P = Q & 1;
        __builtin_amdgcn_sched_barrier(0);
        // this wave's copies of step s + 1 landed (those of s + 2 may not
        // have), and its reads of step s's fragments, issued a step ago
        if constexpr (((Q + 2) & 3) == 0)
            __builtin_amdgcn_s_waitcnt(0x0070 | (PER + 1));
        else
            __builtin_amdgcn_s_waitcnt(0x0070 | PER);
        // ... and everyone's; every wave is past the products of step s - 1,
        // so slot (s - 1) % 4 is free
        barrier_no_fence();
        __builtin_amdgcn_sched_barrier(0);
        read_frags(P ^ 1, smem + ((Q + 1) & 3) * STAGE);
        __builtin_amdgcn_sched_barrier(0);
        stage(s + 3 < nsteps ? s + 3 : s - 1, smem + ((Q + 3) & 3) * STAGE);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    af[P][i], bf[P][j], acc[i][j], FA, FB, Q, (int)ca[i], Q, (int)cb[j]);
        }
        if constexpr (Q == 3) {
            // the next group's scale words (copied with step s + 1, which landed)
            __builtin_amdgcn_sched_barrier(0);
            read_scales((s + 1) >> 2);
        }
    };
    for (int s = 0; s < nsteps; s += 4) {
        step(s, std::integral_constant<int, 0>{});
        step(s + 1, std::integral_constant<int, 1>{});
        step(s + 2, std::integral_constant<int, 2>{});
        step(s + 3, std::integral_constant<int, 3>{});
    }
    // every wave's copies and reads are done before a slot takes the output
    __builtin_amdgcn_s_waitcnt(0x0070);
    barrier_no_fence();
    const int cur = 0;

    // a whole tile leaves through LDS as 16-byte row pieces: the ring slot of
    // step nsteps (that of step nsteps - 3, read by every wave before the last
    // barrier, with no copy pending) holds each wave's 4 KiB
    if (m0 + kBM <= m && n0 + kBN <= n && (ldc & 3) == 0 && ((uintptr_t)c & 15) == 0) {
        float *lw = reinterpret_cast<float *>(smem + cur * STAGE) + wv * 1024;
        store_tile_lds(acc, lw, c, ldc, m0 + 128 * wm, n0 + 64 * wn, lane);
        return;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = n0 + 64 * wn + 16 * j + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + 128 * wm + 16 * i + 4 * g + r;
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

template <int FA, int FB>
hipError_t launch_staged(int64_t tiles, hipStream_t s, const uint8_t *ac, const uint8_t *as,
                         const uint8_t *bc, const uint8_t *bs, int64_t m, int64_t n, int64_t k,
                         float *c, int64_t ldc)
{
    constexpr int lds = lds_bytes<FA, FB>();
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&k_wgrad_lds<FA, FB>),
        hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (attr != hipSuccess)
        return attr;
    hipLaunchKernelGGL((k_wgrad_lds<FA, FB>), dim3((unsigned)tiles), dim3(256), lds, s, ac, as, bc,
                       bs, m, n, k, c, ldc);
    return hipGetLastError();
}

template <int FA, int FB>
hipError_t launch_tiled(int64_t tiles, hipStream_t s, const uint8_t *ac, const uint8_t *as,
                        const uint8_t *bc, const uint8_t *bs, int64_t m, int64_t n, int64_t k,
                        float *c, int64_t ldc)
{
    const bool offsets32 = ((m + 15) / 16) * 64 * blk_bytes<FA>() < (int64_t(1) << 32) &&
                           ((n + 15) / 16) * 64 * blk_bytes<FB>() < (int64_t(1) << 32) &&
                           k / 128 <= 0x7FFFFFFF;
    if (offsets32 && reinterpret_cast<uintptr_t>(as) % 16 == 0 &&
        reinterpret_cast<uintptr_t>(bs) % 16 == 0) {
        // scale words copied 16 bytes per lane: the 3-stage ring
        if constexpr (FA == kMfmaFP4 && FB == kMfmaFP4) {
            if (k % 512 == 0) {
                constexpr int lds = ra4_lds_bytes<FA, FB>();
                static const hipError_t attr = hipFuncSetAttribute(
                    reinterpret_cast<const void *>(&k_wgrad_ra4<FA, FB>),
                    hipFuncAttributeMaxDynamicSharedMemorySize, lds);
                if (attr != hipSuccess)
                    return attr;
                hipLaunchKernelGGL((k_wgrad_ra4<FA, FB>), dim3((unsigned)tiles), dim3(64 * kWaves),
                                   lds, s, ac, as, bc, bs, m, n, k, c, ldc);
                return hipGetLastError();
            }
        }
        constexpr int lds = ring3_lds_bytes<FA, FB>();
        static const hipError_t attr = hipFuncSetAttribute(
            reinterpret_cast<const void *>(&k_wgrad_ring3<FA, FB>),
            hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (attr != hipSuccess)
            return attr;
        hipLaunchKernelGGL((k_wgrad_ring3<FA, FB>), dim3((unsigned)tiles), dim3(64 * kWaves), lds,
                           s, ac, as, bc, bs, m, n, k, c, ldc);
        return hipGetLastError();
    }
    constexpr int lds = tiled_lds_bytes<FA, FB>();
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&k_wgrad_tiled<FA, FB>),
        hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (attr != hipSuccess)
        return attr;
    hipLaunchKernelGGL((k_wgrad_tiled<FA, FB>), dim3((unsigned)tiles), dim3(64 * kWaves), lds, s,
                       ac, as, bc, bs, m, n, k, c, ldc);
    return hipGetLastError();
}

namespace {
int mfma_format(const mxq_qtensor *q)
{
    if (q->fmt == MXQ_FMT_E2M3)
        return kMfmaFP6;
    if (q->fmt == MXQ_FMT_FP4 && q->grid != MXQ_GRID_E1M2)
        return kMfmaFP4;   // E2M1 nibbles, capped or not
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
    if ((a->layout != MXQ_LAYOUT_ROWS && a->layout != MXQ_LAYOUT_MFMA) || a->layout != b->layout)
        return MXQ_ERR_UNSUPPORTED;
    if (a->layout == MXQ_LAYOUT_MFMA &&
        (reinterpret_cast<uintptr_t>(a->codes) % 16 || reinterpret_cast<uintptr_t>(b->codes) % 16 ||
         reinterpret_cast<uintptr_t>(a->scales) % 4 || reinterpret_cast<uintptr_t>(b->scales) % 4))
        return MXQ_ERR_ALIGN;
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
    const uint8_t *ac = static_cast<const uint8_t *>(a->codes);
    const uint8_t *bc = static_cast<const uint8_t *>(b->codes);
    if (a->layout == MXQ_LAYOUT_MFMA) {
        const int64_t tiles = ((m + kBM - 1) / kBM) * ((n + kBN - 1) / kBN);
        if (tiles > 0x7FFFFFFF)
            return MXQ_ERR_SHAPE;
        hipError_t e;
        if (fa == kMfmaFP4 && fb == kMfmaFP4)
            e = launch_tiled<kMfmaFP4, kMfmaFP4>(tiles, s, ac, a->scales, bc, b->scales, m, n, k, c, ldc);
        else if (fa == kMfmaFP6 && fb == kMfmaFP6)
            e = launch_tiled<kMfmaFP6, kMfmaFP6>(tiles, s, ac, a->scales, bc, b->scales, m, n, k, c, ldc);
        else if (fa == kMfmaFP4)
            e = launch_tiled<kMfmaFP4, kMfmaFP6>(tiles, s, ac, a->scales, bc, b->scales, m, n, k, c, ldc);
        else
            e = launch_tiled<kMfmaFP6, kMfmaFP4>(tiles, s, ac, a->scales, bc, b->scales, m, n, k, c, ldc);
        return e == hipSuccess ? MXQ_OK : MXQ_ERR_DEVICE;
    }
    const bool staged = k % 512 == 0 && reinterpret_cast<uintptr_t>(ac) % 16 == 0 &&
                        reinterpret_cast<uintptr_t>(bc) % 16 == 0 &&
                        reinterpret_cast<uintptr_t>(a->scales) % 16 == 0 &&
                        reinterpret_cast<uintptr_t>(b->scales) % 16 == 0;
    if (staged) {
        const int64_t tiles = ((m + kBM - 1) / kBM) * ((n + kBN - 1) / kBN);
        if (tiles > 0x7FFFFFFF)
            return MXQ_ERR_SHAPE;
        hipError_t e;
        if (fa == kMfmaFP4 && fb == kMfmaFP4)
            e = launch_staged<kMfmaFP4, kMfmaFP4>(tiles, s, ac, a->scales, bc, b->scales, m, n, k, c, ldc);
        else if (fa == kMfmaFP6 && fb == kMfmaFP6)
            e = launch_staged<kMfmaFP6, kMfmaFP6>(tiles, s, ac, a->scales, bc, b->scales, m, n, k, c, ldc);
        else if (fa == kMfmaFP4)
            e = launch_staged<kMfmaFP4, kMfmaFP6>(tiles, s, ac, a->scales, bc, b->scales, m, n, k, c, ldc);
        else
            e = launch_staged<kMfmaFP6, kMfmaFP4>(tiles, s, ac, a->scales, bc, b->scales, m, n, k, c, ldc);
        return e == hipSuccess ? MXQ_OK : MXQ_ERR_DEVICE;
    }
    // other K (multiples of 128) or alignments: direct loads, no LDS
    const dim3 grid((unsigned)((n + kTN - 1) / kTN), (unsigned)((m + kTM - 1) / kTM));
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

extern "C" mxq_status mxq_gemm_abt(const mxq_qtensor *a, const mxq_qtensor *b, int64_t m,
                                   int64_t n, int64_t k, float *c, int64_t ldc, void *stream)
{
    return mxq_wgrad_gemm(a, b, m, n, k, c, ldc, stream);
}
