// Grouped-query paged decode attention on the matrix cores (gfx950), bf16 or
// MXFP8 caches, head dim 128, 16-token blocks, up to 16 query heads per KV head.
//
// It computes what the VALU grouped kernel computes (exact softmax attention
// of one query token per sequence over its paged K/V, query head h reading
// KV head h / G: PagedAttention page table in "Cache KV, attention et
// optimisation de l'inference", GQA in CS336 lecture 10 notes; the online
// softmax of "Étape 2: softmax en carreaux"; FlashDecoding partitions merged
// by the same log-sum-exp reduce), and leaves the same partial results, so
// the same stream-K schedule and reduce kernel serve both.  What differs is
// where the arithmetic runs: the G heads of a group share each K/V block,
// which makes a block's work two small dense products,
//     S^T[token, head] = K[token, :] . Q^T[:, head]        (16 x 16 x 128)
//     O^T[dim, head]  += V^T[dim, token] . P^T[token, head] (128 x 16 x 16)
// and both go to v_mfma (16x16x32 and 16x16x16 bf16) with heads as the
// 16-wide N dimension (columns G..15 carry a zero query and are dropped).
// The VALU then has only the softmax of 4 scores per lane to do, instead of
// G dot products per token and the lane reductions behind them.
//
// gfx950 mapping, one wave64 per KV head of a stream share (4 per work-group,
// one per SIMD; a team of up to 4 waves streams neighbouring heads of one
// share):
//  * K and V tiles of a block (16 rows of 256 bytes each) stream HBM -> LDS
//    with global_load_lds_dwordx4 into a ring of NBUF slots, as in the VALU
//    kernel.  Chunk c (16 bytes) of row t is stored at chunk c ^ t: the
//    row-wise K reads of a 16-lane phase (16 rows, one chunk column) and the
//    transposed V reads (4 rows x 2 chunk columns per 16 lanes) then fall on
//    distinct banks.
//  * Lane (col = lane % 16, quad = lane / 16) holds, for the scores, row
//    `col` of K (the A operand: 8 dims per k-step) and head `col` of q (the
//    B operand, in registers for the whole segment); the product leaves it
//    the scores of tokens 4 quad .. 4 quad + 3 of head col.  That is exactly
//    the B-operand layout of the value product, so the probabilities go from
//    the softmax to the matrix core without leaving the lane; V^T comes from
//    LDS by ds_read_b64_tr_b16.
//  * Softmax per head (column): max over the lane's 4 scores and the 4 quads
//    (two row swaps, v_permlane16_swap and v_permlane32_swap); the running max moves only when a score passes it
//    by more than kSlack (log2 units), so the rescale of the 32 accumulators
//    is rare; probabilities are rounded to bf16 for the product and the
//    running sum adds the rounded values.
//
// MXFP8 caches (the blockwise-scaled fp8 of the CS336 lecture 10 notes,
// "常见陷阱"; E4M3 codes with one E8M0 scale per 32 values of a head row)
// run the same kernel with half the bytes per block.  Their tiles are
// contiguous per (block, KV head): K codes as 16 rows of 128 bytes, V codes
// transposed (128 dims x 16 tokens), and the two 64-byte scale tiles.
//  * Scores: a lane's K operand is 8 values of one 32-value block of one
//    token, so one v_cvt_scalef32_pk_bf16_fp8 per value pair turns codes into
//    bf16 with that block's scale applied (exact, as both are powers of two
//    times 3-bit mantissas; values below bf16's normal range, |v| < 2^-126,
//    come out as zero), and the four k-steps chain in one accumulator.
//  * Values: a V^T operand element is one token's value, each with its own
//    token's scale, so the codes convert unscaled and the scales go to P^T
//    instead: P'[t, h] = P[t, h] * 2^X(t, block), one copy of the B operand
//    per 32-dim block (two output tiles each).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "hip_util.h"
#include "launch.h"

namespace pa {
namespace {

constexpr int kMBS = 16;              // tokens per cache block
constexpr int kMD = 128;              // head dim (K and V)
constexpr int kMKSteps = kMD / 32;    // score k-steps
constexpr int kMDimTiles = kMD / 16;  // 16-dim tiles of the output
constexpr float kMSlack = 8.0f;       // lazy-rescale threshold, log2 units
constexpr float kMFloor = -3.0e38f;   // running max before any visible token (finite)
constexpr int kMGroupWaves = 4;

// Per-format tile geometry of one (block, KV head).
template <bool MX>
struct MTile;
template <>
struct MTile<false> {                    // bf16, the pages' [nb, bs, Hkv, d] layout
    static constexpr int kRowB = kMD * 2;        // 256-byte token rows
    static constexpr int kKB = kMBS * kRowB;     // 4 KB of K (and of V)
    static constexpr int kDma = kKB / 1024;      // 1 KB LDS-DMA loads per K (or V) tile
    static constexpr int kSlotB = 2 * kKB;       // K then V
    static constexpr int kPerBlock = 2 * kDma;   // loads per block
};
template <>
struct MTile<true> {                     // MXFP8
    static constexpr int kKB = kMBS * kMD;       // 2 KB of K codes (and of V codes)
    static constexpr int kDma = kKB / 1024;
    static constexpr int kScaleB = kMBS * (kMD / kMxBlock);  // 64-byte scale tile
    static constexpr int kScaleLds = kWave * 4;  // a dword LDS-DMA fills 256 bytes
    static constexpr int kSlotB = 2 * kKB + 2 * kScaleLds;  // K, V^T, K scales, V scales
    static constexpr int kPerBlock = 2 * kDma + 2;
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8_t lds_b128(uint32_t byte_addr) {
    return __builtin_bit_cast(
        bf16x8_t, *(const __attribute__((address_space(3))) u32x4_t *)(uintptr_t)byte_addr);
}
__device__ __forceinline__ u32x4_t lds_u128(uint32_t byte_addr) {
    return *(const __attribute__((address_space(3))) u32x4_t *)(uintptr_t)byte_addr;
}
__device__ __forceinline__ u32x2_t lds_u64(uint32_t byte_addr) {
    return *(const __attribute__((address_space(3))) u32x2_t *)(uintptr_t)byte_addr;
}
__device__ __forceinline__ uint32_t lds_u32(uint32_t byte_addr) {
    return *(const __attribute__((address_space(3))) uint32_t *)(uintptr_t)byte_addr;
}
__device__ __forceinline__ s16x4_t lds_tr_b64(uint32_t byte_addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t *)(uintptr_t)byte_addr);
}

// Two E4M3 codes (the low or high 16 bits of w) as a bf16 pair times scale.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_bf16(uint32_t w, float scale) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, HI));
}
// 2^(e - 127) for an E8M0 byte e < 255 (e = 0 is the subnormal 2^-127).
__device__ __forceinline__ float e8m0_f32(uint32_t e) {
    return as_f(e != 0 ? e << 23 : 0x00400000u);
}

// Wait until at most `later` blocks of PER loads are still in flight.
template <int PER, int NBUF>
__device__ __forceinline__ void wait_mblocks(int later) {
    if constexpr (NBUF >= 4) {
        if (later >= 3) { wait_vmem<3 * PER>(); return; }
        if (later == 2) { wait_vmem<2 * PER>(); return; }
    }
    if (later >= 1) { wait_vmem<PER>(); return; }
    wait_vmem<0>();
}

// Partition kernel: the stream-K schedule (teams of team_heads waves, one KV
// head each, sharing a share of the (sequence, head chunk, block) order) and
// partial-slot layout of the VALU grouped kernel (slot share + b * NC + ch,
// row (slot * team_heads + hw) * C + column, fp32 accumulator of D dims plus
// (max, sum) in log2 units).  MX selects MXFP8 caches (k_scale, v_scale
// used); otherwise the caches are bf16.
//
// Columns: with q_len new query tokens per sequence (causal among
// themselves, as in the masked attention of "Étape 2: Attention avec KV
// Cache": query i of the last q_len cached tokens sees tokens up to
// position L - q_len + i), the N dimension of the products holds C = G *
// q_len (query, head) pairs, column c = i * G + h, in NT tiles of 16.  One
// K/V fetch and one V^T read then serve all of them.  q is [B, q_len, Hq, D].
template <bool MX, int NBUF, int NT>
__global__ __launch_bounds__(kWave *kMGroupWaves) void gqa_mfma_partition_kernel(
    float *__restrict__ ws_acc, float2 *__restrict__ ws_ml, int32_t *__restrict__ ws_prefix,
    const uint16_t *__restrict__ q, const void *__restrict__ k_cache,
    const void *__restrict__ v_cache, const uint8_t *__restrict__ k_scale,
    const uint8_t *__restrict__ v_scale, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, float scale_log2, int num_seqs, int num_kv_heads,
    int group, int q_len, int max_blocks, int nshares, int team_heads, int window) {
    using TL = MTile<MX>;
    static_assert((NBUF & (NBUF - 1)) == 0 && NBUF >= 2 && NBUF <= 4, "ring depth 2 or 4");
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int sid = (blockIdx.x * kMGroupWaves + wave) / team_heads;  // this wave's team and share
    const int hw = wave % team_heads;                                  // its head within a chunk
    const int nchunks = num_kv_heads / team_heads;
    if (sid >= nshares) return;  // uniform over the team; waves never wait on each other
    const int col = lane & 15;
    const int quad = lane >> 4;
    const int num_q_heads = num_kv_heads * group;
    const int ncols = group * q_len;
    // this lane's columns (one per tile): query qi[ct], head hh[ct] of the group
    int qi[NT], hh[NT];
    bool live[NT];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
        const int c = 16 * ct + col;
        live[ct] = c < ncols;
        qi[ct] = live[ct] ? c / group : 0;
        hh[ct] = live[ct] ? c - qi[ct] * group : 0;
    }

    __shared__ __attribute__((aligned(16))) char s_ring_all[kMGroupWaves][NBUF * TL::kSlotB];
    __shared__ __attribute__((aligned(16))) int32_t s_ids_all[kMGroupWaves][2][kWave];
    int32_t(*s_ids)[kWave] = s_ids_all[wave];
    const uint32_t ring_lds = lds_offset(s_ring_all[wave]);
    const uint32_t ids_lds[2] = {lds_offset(&s_ids[0][0]), lds_offset(&s_ids[1][0])};

    ShareSpan sp;
    if (!find_share(sid, nshares, num_seqs, nchunks, kMBS, context_lens, ws_prefix, lane, sp,
                    window, hw == 0))
        return;
    const int x1 = sp.x1;
    int b = sp.b, nbb = sp.nbb, ch = sp.g, blk_start = sp.blk;

    const char *kbase = static_cast<const char *>(k_cache);
    const char *vbase = static_cast<const char *>(v_cache);

    // LDS byte offsets (inside a tile) this lane reads.
    uint32_t k_rd[kMKSteps];
    uint32_t v_rd[kMDimTiles];
    if constexpr (!MX) {
        //  K, score k-step j: row col, chunk (4 j + quad) ^ col.
        //  V^T, dim tile t: the transposed read's source row 4 quad + col / 4,
        //  dims 16 t + 4 (col % 4) .. + 3, i.e. chunk 2 t + (col % 4) / 2, half col % 2.
#pragma unroll
        for (int j = 0; j < kMKSteps; ++j)
            k_rd[j] = col * TL::kRowB + (((4 * j + quad) ^ col) << 4);
        const int vrow = 4 * quad + (col >> 2);
#pragma unroll
        for (int t = 0; t < kMDimTiles; ++t)
            v_rd[t] = vrow * TL::kRowB + (((2 * t + ((col & 3) >> 1)) ^ vrow) << 4) + 8 * (col & 1);
    } else {
        //  K codes, k-step j: 8 bytes of row col at dims 32 j + 8 quad, i.e. chunk
        //  2 j + quad / 2 (stored at chunk ^ ((row / 2) % 8)), half quad % 2.
        //  V^T codes, dim tile t: 4 bytes (tokens 4 quad ..) of row 16 t + col.
#pragma unroll
        for (int j = 0; j < kMKSteps; ++j)
            k_rd[j] = col * kMD + (((2 * j + (quad >> 1)) ^ ((col >> 1) & 7)) << 4) + 8 * (quad & 1);
#pragma unroll
        for (int t = 0; t < kMDimTiles; ++t) v_rd[t] = TL::kKB + (16 * t + col) * kMBS + 4 * quad;
    }

    // A segment's partial is kept in registers and written when the share
    // ends, or when more than kMPend wait (one with four column tiles, for
    // registers): vmcnt counts stores with the loads, in issue order, so a
    // load issued after a store (the next segment's block ids and q, then its
    // blocks) cannot be waited for before the store completes, which under
    // the read stream takes microseconds.
    struct MPart {
        f32x4_t acc[NT][kMDimTiles];
        float m[NT], l[NT];
        int64_t row;  // the segment's first partial row (uniform)
    };
    constexpr int kMPend = NT == 1 ? 2 : 1;
    MPart pend[kMPend];
    int npend = 0;  // (uniform)
    auto write_part = [&](const MPart &pp) {
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            if (live[ct]) {
                const int64_t row = pp.row + 16 * ct + col;
                // a column with no visible token in the segment reports max -inf
                if (quad == 0) ws_ml[row] = make_float2(pp.l[ct] > 0.f ? pp.m[ct] : kNegInf, pp.l[ct]);
                float *dst = ws_acc + row * kMD + 4 * quad;
#pragma unroll
                for (int t = 0; t < kMDimTiles; ++t)
                    *reinterpret_cast<f32x4_t *>(dst + 16 * t) = pp.acc[ct][t];
            }
        }
    };

    for (int x = sp.x0;;) {
        // ======== segment (b, ch), head g: blocks [blk_start, blk_start + nblk) ========
        const int g = ch * team_heads + hw;
        const int nblk = min(nbb - blk_start, x1 - x);
        const int ctx = context_lens[b];
        const int32_t *bt_row = block_tables + static_cast<int64_t>(b) * max_blocks;
        // the window's first token and block (0 and 0 without a window)
        const int wstart = window_start(ctx, window);
        const int wblk = blk_start + wstart / kMBS;  // table index of this segment's first block

        auto fetch_ids = [&](int m) {
            const int e = min(wblk + kWave * m + lane, max_blocks - 1);
            dma4(bt_row, static_cast<uint32_t>(e) * 4u, ids_lds[m & 1]);
        };
        fetch_ids(0);
        if (nblk > kWave) fetch_ids(1);

        // q^T as the score B operand: column (query qi, head g G + hh), dims
        // 32 j + 8 quad .. + 7; columns past G * q_len hold zeros.
        bf16x8_t qb[NT][kMKSteps];
        // tokens below lim[ct] are visible to this lane's column of tile ct
        int lim[NT];
        // Every q load is issued before any is settled (the empty asm makes the
        // compiler wait for a load there, so settling each one after its own
        // load would cost a memory round trip per load).
        u32x4_t qv[NT][kMKSteps];
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            const uint16_t *qr =
                q + ((static_cast<int64_t>(b) * q_len + qi[ct]) * num_q_heads + g * group + hh[ct]) *
                        kMD + 8 * quad;
#pragma unroll
            for (int j = 0; j < kMKSteps; ++j) qv[ct][j] = *reinterpret_cast<const u32x4_t *>(qr + 32 * j);
        }
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
#pragma unroll
            for (int j = 0; j < kMKSteps; ++j) {
                u32x4_t v = qv[ct][j];
                asm volatile("" : "+v"(v));
                if (!live[ct]) v = u32x4_t{0u, 0u, 0u, 0u};
                qb[ct][j] = __builtin_bit_cast(bf16x8_t, v);
            }
            lim[ct] = live[ct] ? ctx - q_len + 1 + qi[ct] : ctx;
        }
        // blocks from the window's start to this token are visible to every column
        const int all_visible = ctx - q_len + 1;
        // This lane's DMA sources inside one block's tile.
        uint32_t dma_off[TL::kDma];
        if constexpr (!MX) {
            // tile row 4 i + quad, chunk col ^ row, rows Hkv * 256 bytes apart
            const int64_t row_stride = static_cast<int64_t>(num_kv_heads) * TL::kRowB;
#pragma unroll
            for (int i = 0; i < TL::kDma; ++i) {
                const int t = 4 * i + quad;
                dma_off[i] = static_cast<uint32_t>(t * row_stride + g * TL::kRowB + ((col ^ t) << 4));
            }
        } else {
            // LDS chunk p = 64 i + lane is chunk p % 8 of row p / 8, holding that row's
            // chunk (p % 8) ^ ((row / 2) % 8)
#pragma unroll
            for (int i = 0; i < TL::kDma; ++i) {
                const int p = kWave * i + lane;
                const int t = p >> 3;
                dma_off[i] = static_cast<uint32_t>(t * kMD + (((p & 7) ^ ((t >> 1) & 7)) << 4));
            }
        }
        drain_vmem();  // q and the first ids have landed; the ring's accounting starts empty

        // running max of the lane's column (scaled, log2 units).  It starts at a
        // finite floor, not -inf: with several queries (or a window) a block can
        // be masked for some columns only, and the rescale branch below is taken
        // by the whole wave, so a column that has seen no visible token yet must
        // get alpha = 1 and weights 0 there, never exp2(-inf + inf).
        float m_run[NT];
        float l_run[NT];  // this lane's share of the column's running sum
        f32x4_t acc[NT][kMDimTiles];
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            m_run[ct] = kMFloor;
            l_run[ct] = 0.f;
#pragma unroll
            for (int t = 0; t < kMDimTiles; ++t) acc[ct][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }

        auto issue = [&](int n) {
            if ((n & (kWave - 1)) == 0 && n > 0 && n + kWave < nblk) fetch_ids((n >> 6) + 1);
            const int pb = __builtin_amdgcn_readfirstlane(s_ids[(n >> 6) & 1][n & (kWave - 1)]);
            const uint32_t slot = ring_lds + (n & (NBUF - 1)) * TL::kSlotB;
            if constexpr (!MX) {
                const int64_t blk_b = static_cast<int64_t>(kMBS) * num_kv_heads * TL::kRowB;
                const char *kb = kbase + static_cast<int64_t>(pb) * blk_b;
                const char *vb = vbase + static_cast<int64_t>(pb) * blk_b;
                sgpr_settle(kb);
#pragma unroll
                for (int i = 0; i < TL::kDma; ++i) dma16(kb, dma_off[i], slot + i * 1024);
#pragma unroll
                for (int i = 0; i < TL::kDma; ++i) dma16(vb, dma_off[i], slot + TL::kKB + i * 1024);
            } else {
                const int64_t tile = static_cast<int64_t>(pb) * num_kv_heads + g;
                const char *kb = kbase + tile * TL::kKB;
                const char *vb = vbase + tile * TL::kKB;
                sgpr_settle(kb);
#pragma unroll
                for (int i = 0; i < TL::kDma; ++i) dma16(kb, dma_off[i], slot + i * 1024);
#pragma unroll
                for (int i = 0; i < TL::kDma; ++i)
                    dma16(vb, static_cast<uint32_t>(kWave * i + lane) * 16u,
                          slot + TL::kKB + i * 1024);
                // the 64-byte scale tiles: lanes 16.. repeat lanes 0..15
                const uint32_t so = static_cast<uint32_t>(lane & 15) * 4u;
                dma4(k_scale + tile * TL::kScaleB, so, slot + 2 * TL::kKB);
                dma4(v_scale + tile * TL::kScaleB, so, slot + 2 * TL::kKB + TL::kScaleLds);
            }
        };

        auto compute_block = [&](int n) {
            const uint32_t kslot = ring_lds + (n & (NBUF - 1)) * TL::kSlotB;
            const int tok0 = (wblk + n) * kMBS;
            const int valid = ctx - tok0;  // tokens of this block in context

            // ---- scores S^T[token 4 quad + i, column 16 ct + col] ----
            f32x4_t s[NT];
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) s[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            u32x4_t vsc;  // MXFP8: V scales of tokens 4 quad + i (byte = 32-dim block)
            uint32_t vw[kMDimTiles];  // MXFP8: V^T codes, tokens 4 quad .. of dim 16 t + col
            if constexpr (!MX) {
                bf16x8_t ka[kMKSteps];
#pragma unroll
                for (int j = 0; j < kMKSteps; ++j) ka[j] = lds_b128(kslot + k_rd[j]);
#pragma unroll
                for (int j = 0; j < kMKSteps; ++j)
#pragma unroll
                    for (int ct = 0; ct < NT; ++ct)
                        s[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[j], qb[ct][j], s[ct], 0, 0, 0);
            } else {
                // every LDS read of the block first, so their latencies overlap
                u32x2_t kc[kMKSteps];
#pragma unroll
                for (int j = 0; j < kMKSteps; ++j) kc[j] = lds_u64(kslot + k_rd[j]);
                const uint32_t ksw = lds_u32(kslot + 2 * TL::kKB + 4 * col);  // token col's scales
                vsc = lds_u128(kslot + 2 * TL::kKB + TL::kScaleLds + 16 * quad);
#pragma unroll
                for (int t = 0; t < kMDimTiles; ++t) vw[t] = lds_u32(kslot + v_rd[t]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < kMKSteps; ++j) {
                    const float ksc = e8m0_f32((ksw >> (8 * j)) & 0xFFu);
                    const u32x4_t a = {fp8x2_bf16<false>(kc[j].x, ksc), fp8x2_bf16<true>(kc[j].x, ksc),
                                       fp8x2_bf16<false>(kc[j].y, ksc), fp8x2_bf16<true>(kc[j].y, ksc)};
#pragma unroll
                    for (int ct = 0; ct < NT; ++ct)
                        s[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, a), qb[ct][j], s[ct], 0, 0, 0);
                }
            }
            // V^T fragments, read while the scores are worked on
            s16x4_t va[kMDimTiles];
            if constexpr (!MX) {
#pragma unroll
                for (int t = 0; t < kMDimTiles; ++t) va[t] = lds_tr_b64(kslot + TL::kKB + v_rd[t]);
            } else {
#pragma unroll
                for (int t = 0; t < kMDimTiles; ++t)
                    va[t] = __builtin_bit_cast(s16x4_t, u32x2_t{fp8x2_bf16<false>(vw[t], 1.0f),
                                                                fp8x2_bf16<true>(vw[t], 1.0f)});
            }

            // ---- online softmax per column; probabilities rounded to bf16 ----
            // no column masks a token of this block
            const bool full = tok0 + kMBS <= all_visible && tok0 >= wstart;
            float p[NT][4];
            uint32_t p01[NT], p23[NT];
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
                float x[4];
                if (full) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) x[i] = s[ct][i] * scale_log2;
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        x[i] = (tok0 + 4 * quad + i < lim[ct] && tok0 + 4 * quad + i >= wstart)
                                   ? s[ct][i] * scale_log2
                                   : kNegInf;
                }
                float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
                bm = max_r32(max_r16(bm));
                if (__builtin_amdgcn_ballot_w64(bm > m_run[ct] + kMSlack) != 0) {
                    const float m_new = fmaxf(m_run[ct], bm);
                    const float alpha =
                        exp2_fast(m_run[ct] - m_new);
                    l_run[ct] *= alpha;
                    m_run[ct] = m_new;
#pragma unroll
                    for (int t = 0; t < kMDimTiles; ++t) acc[ct][t] *= alpha;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) p[ct][i] = exp2_fast(x[i] - m_run[ct]);
                p01[ct] = pack_bf16(p[ct][0], p[ct][1]);
                p23[ct] = pack_bf16(p[ct][2], p[ct][3]);
                l_run[ct] += (bf16_lo(p01[ct]) + bf16_hi(p01[ct])) + (bf16_lo(p23[ct]) + bf16_hi(p23[ct]));
            }

            // ---- O^T[16 t + 4 quad + i, head col] += V^T P^T ----
            if (valid < kMBS) {  // rows past the context contribute exactly zero, NaN or not
#pragma unroll
                for (int t = 0; t < kMDimTiles; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * quad + e >= valid) va[t][e] = 0;
            }
            if constexpr (!MX) {
#pragma unroll
                for (int ct = 0; ct < NT; ++ct) {
                    const s16x4_t pb = __builtin_bit_cast(s16x4_t, u32x2_t{p01[ct], p23[ct]});
#pragma unroll
                    for (int t = 0; t < kMDimTiles; ++t)
                        acc[ct][t] =
                            __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[t], pb, acc[ct][t], 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int jv = 0; jv < kMD / kMxBlock; ++jv) {
                    int e[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) e[i] = static_cast<int>((vsc[i] >> (8 * jv)) & 0xFFu) - 127;
#pragma unroll
                    for (int ct = 0; ct < NT; ++ct) {
                        float ps[4];  // ldexp keeps masked (zero) weights zero whatever their scale
#pragma unroll
                        for (int i = 0; i < 4; ++i) ps[i] = ldexpf(p[ct][i], e[i]);
                        const s16x4_t pb = __builtin_bit_cast(
                            s16x4_t, u32x2_t{pack_bf16(ps[0], ps[1]), pack_bf16(ps[2], ps[3])});
#pragma unroll
                        for (int t = 2 * jv; t < 2 * jv + 2; ++t)
                            acc[ct][t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[t], pb,
                                                                                  acc[ct][t], 0, 0, 0);
                    }
                }
            }
        };

#pragma unroll
        for (int n = 0; n < NBUF - 1; ++n)
            if (n < nblk) issue(n);
        for (int n = 0; n < nblk; ++n) {
            if (n + NBUF - 1 < nblk) {
                wait_lds();  // slot (n - 1) % NBUF and the ids in LDS are read
                issue(n + NBUF - 1);
            }
            wait_mblocks<TL::kPerBlock, NBUF>(min(NBUF - 1, nblk - 1 - n));
            compute_block(n);
        }

        // ---- this segment's partial: unnormalised acc, running max and sum ----
        {
            MPart cur;
            cur.row = ((static_cast<int64_t>(sid) + static_cast<int64_t>(b) * nchunks + ch) * team_heads +
                       hw) * ncols;
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
                cur.l[ct] = sum_r32(sum_r16(l_run[ct]));
                cur.m[ct] = m_run[ct];
#pragma unroll
                for (int t = 0; t < kMDimTiles; ++t) cur.acc[ct][t] = acc[ct][t];
            }
            if (npend == kMPend) {  // the oldest goes out now
                write_part(pend[0]);
#pragma unroll
                for (int i = 0; i + 1 < kMPend; ++i) pend[i] = pend[i + 1];
                pend[kMPend - 1] = cur;
            } else {
#pragma unroll
                for (int i = 0; i < kMPend; ++i)
                    if (i == npend) pend[i] = cur;
                ++npend;
            }
        }

        x += nblk;
        if (x >= x1) break;
        blk_start = 0;
        if (++ch == nchunks) {
            ch = 0;
            do {
                ++b;
                nbb = window_blocks(context_lens[b], window, kMBS);
            } while (nbb == 0);
        }
        wait_lds();  // every LDS read of this segment is done before the next one's DMA
    }
#pragma unroll
    for (int i = 0; i < kMPend; ++i)
        if (i < npend) write_part(pend[i]);
}

template <bool MX, int NBUF, int NT>
pa_status enqueue_gqa_mfma(const DecodeShape &s, const DecodeArgs &a, const DecodePlan &p,
                           float scale_log2, hipStream_t stream, std::string *why) {
    char *ws = static_cast<char *>(a.workspace);
    float *acc = reinterpret_cast<float *>(ws + p.acc_offset);
    float2 *ml = reinterpret_cast<float2 *>(ws + p.ml_offset);
    int32_t *prefix = reinterpret_cast<int32_t *>(ws + p.prefix_offset);
    const auto kernel = gqa_mfma_partition_kernel<MX, NBUF, NT>;
    // MXFP8: two work-groups (8 waves) per CU although LDS holds four: on the
    // 70B-shape batch 179 us against 189 us with 16 waves (and 1024 fewer
    // partial slots to merge), 187 against 199 us at 128K contexts.  bf16:
    // one work-group per CU, which a 4-deep ring fills; with the 2-deep ring
    // LDS would hold two, and that measures slower (c3 301.6 against 294.5 us).
    const int waves = stream_waves<gqa_mfma_partition_kernel<MX, NBUF, NT>>(
        kWave * kMGroupWaves, 1, kStreamWavesMax, kMGroupWaves, MX ? 2 : 1);
    const int th = team_heads(s.num_kv_heads, kMGroupWaves, p.group);
    const int nshares = waves / th > 0 ? waves / th : 1;
    const int groups = (nshares * th + kMGroupWaves - 1) / kMGroupWaves;
    hipLaunchKernelGGL(kernel, dim3(groups), dim3(kWave * kMGroupWaves), 0, stream, acc, ml,
                       prefix, static_cast<const uint16_t *>(a.q), a.k_cache, a.v_cache,
                       static_cast<const uint8_t *>(a.k_scale),
                       static_cast<const uint8_t *>(a.v_scale), a.block_tables, a.context_lens,
                       scale_log2, s.num_seqs, s.num_kv_heads, p.group, s.q_len,
                       s.max_blocks_per_seq, nshares, th, s.window);
    pa_status st = hip_status(hipGetLastError(), why, "partition launch");
    if (st != PA_OK) return st;
    return hip_status(enqueue_stream_reduce<uint16_t, kMD>(
                          static_cast<uint16_t *>(a.out), acc, ml, prefix, a.context_lens,
                          s.num_seqs, s.num_q_heads, s.num_kv_heads, p.group, kMBS, nshares, th,
                          stream, s.q_len, s.window, a.lse),
                      why, "reduce launch");
}

template <bool MX, int NT>
pa_status launch_mfma_nt(const DecodeShape &s, const DecodeArgs &a, const DecodePlan &p,
                         float scale_log2, hipStream_t stream, std::string *why) {
    if (p.ring_depth == 4) return enqueue_gqa_mfma<MX, 4, NT>(s, a, p, scale_log2, stream, why);
    return enqueue_gqa_mfma<MX, 2, NT>(s, a, p, scale_log2, stream, why);
}

template <bool MX>
pa_status launch_mfma(const DecodeShape &s, const DecodeArgs &a, const DecodePlan &p,
                      hipStream_t stream, std::string *why) {
    if (s.num_seqs == 0) return PA_OK;
    const float scale_log2 = static_cast<float>(static_cast<double>(a.scale) * 1.4426950408889634);
    const int cols = p.group * s.q_len;  // at most 16 * kMaxColTiles (plan_decode checks it)
    if (cols <= 16) return launch_mfma_nt<MX, 1>(s, a, p, scale_log2, stream, why);
    if (cols <= 32) return launch_mfma_nt<MX, 2>(s, a, p, scale_log2, stream, why);
    return launch_mfma_nt<MX, 4>(s, a, p, scale_log2, stream, why);
}

}  // namespace

pa_status launch_gqa_mfma_decode(const DecodeShape &s, const DecodeArgs &a, const DecodePlan &p,
                                 void *stream_arg, std::string *why) {
    const hipStream_t stream = static_cast<hipStream_t>(stream_arg);
    return launch_mfma<false>(s, a, p, stream, why);
}

pa_status launch_mxfp8_decode(const DecodeShape &s, const DecodeArgs &a, const DecodePlan &p,
                              void *stream_arg, std::string *why) {
    const hipStream_t stream = static_cast<hipStream_t>(stream_arg);
    return launch_mfma<true>(s, a, p, stream, why);
}

}  // namespace pa
