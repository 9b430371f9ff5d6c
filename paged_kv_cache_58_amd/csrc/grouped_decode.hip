// Grouped-query (and MHA) paged decode attention for gfx950.
//
// What is computed: for one query token per sequence, O = softmax(q K^T s) V
// over the sequence's cached tokens, K/V reached block by block through the
// block table (PagedAttention page table, "Cache KV, attention et
// optimisation de l'inference"), query head h reading KV head h / G (GQA,
// CS336 lecture 10 notes).  The softmax is taken online, block by block, with
// a running max and running sum that rescale what was accumulated so far
// (the tiled softmax of "Étape 2: softmax en carreaux" on the same page); the
// context is cut into partitions whose (accumulator, max, sum) a second
// kernel merges by log-sum-exp weights (FlashDecoding, named among vLLM's
// optimisations in the CS336 notes; exporting row max and sum from the
// attention kernel is the modification described in "Modification de
// l'Attention" of the KV-sparsity article).
//
// gfx950 mapping (one wave64 work-group per (partition, KV head, sequence)):
//  * A 16-token cache block of one KV head is 16 rows of D elements.  Lane
//    (tp = lane / 8, c = lane % 8) owns rows 2tp and 2tp+1, 16-byte chunks
//    c, c+8, ...: every load is 16 bytes wide and each group of 8 lanes reads
//    one 128-byte line.
//  * K and V travel HBM -> LDS with global_load_lds_dwordx4 (no VGPRs on the
//    way) into a ring of kRingDepth blocks, so several blocks are in flight
//    while the wave computes on an earlier one; explicit vmcnt waits retire
//    exactly one block per step.
//  * The block is fetched once for all G query heads of the group: each lane
//    holds its slice of q for all G heads and forms G partial dot products
//    per token with v_dot2_f32_bf16 (fp32 FMA for fp32 inputs).  The 8 lanes
//    of a token pair finish the dot products with three DPP adds
//    (quad_perm 1032, quad_perm 2301, row_half_mirror).
//  * Softmax: lane c owns head c.  The running max is raised only when a
//    score exceeds it by more than kSlack (log2 units), which keeps every
//    weight below 2^kSlack; otherwise no cross-lane max and no rescale run.
//    The result is the same exact softmax: any reference value works as
//    long as numerator and denominator share it.
//  * P.V: probabilities are rounded to bf16 pairs (tokens 2tp, 2tp+1); lane l
//    reads its output dims of both tokens from the V rows in LDS, pairs them
//    with v_perm_b32, and one v_dot2_f32_bf16 applies two tokens to one dim.
//    Lane l owns output dims {l * D/64 ...} of all G heads; the fp32
//    accumulators stay in registers until the partition ends.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdlib>

#include "launch.h"

namespace pa {
namespace {

constexpr int kWave = 64;
constexpr int kBS = 16;              // tokens per cache block on this path
constexpr float kSlack = 8.0f;       // lazy-rescale threshold, log2 units
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kMaxDevices = 64;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float as_f(uint32_t x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ uint32_t as_u(float x) { return __builtin_bit_cast(uint32_t, x); }

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                          __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    bf16x2_t v;
    v[0] = static_cast<__bf16>(lo);  // round to nearest even
    v[1] = static_cast<__bf16>(hi);
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return as_f(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return as_f(x & 0xffff0000u); }

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return as_f(static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(as_u(x)), CTRL, 0xF, 0xF, false)));
}

// Sum over the 8 lanes of a token pair (lane bits 0..2).
__device__ __forceinline__ float sum_over_c(float x) {
    x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
    x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
    x += dpp<0x141>(x);  // row_half_mirror: the other quad of the 8-lane half row
    return x;
}

// The 8 lanes of a token pair each hold partial dot products over their own
// dims for both tokens and all G heads.  Reduce-scatter them so that lane c
// ends with the full sums (both tokens) of head c / (8 / G): each step keeps
// half of the remaining heads (chosen by one lane bit) and adds the partner's
// partials of that half.  Partners: row_half_mirror (c <-> 7 - c) splits on
// bit 2, quad_perm 2301 (c ^ 2) on bit 1, quad_perm 1032 (c ^ 1) on bit 0; once
// one head is left the remaining steps are plain all-reduce adds.
template <int CTRL, int N>
__device__ __forceinline__ void halve(const float (&in)[2][2 * N], float (&out)[2][N], bool upper) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int k = 0; k < N; ++k) {
            const float keep = upper ? in[j][N + k] : in[j][k];
            const float send = upper ? in[j][k] : in[j][N + k];
            out[j][k] = keep + dpp<CTRL>(send);
        }
}

template <int G>
__device__ __forceinline__ void reduce_scatter_c(const float (&a)[2][G], int c, float (&x)[2]) {
    const bool b2 = (c >> 2) & 1, b1 = (c >> 1) & 1, b0 = c & 1;
    if constexpr (G == 8) {
        float r1[2][4], r2[2][2], r3[2][1];
        halve<0x141, 4>(a, r1, b2);
        halve<0x4E, 2>(r1, r2, b1);
        halve<0xB1, 1>(r2, r3, b0);
        x[0] = r3[0][0];
        x[1] = r3[1][0];
    } else if constexpr (G == 4) {
        float r1[2][2], r2[2][1];
        halve<0x141, 2>(a, r1, b2);
        halve<0x4E, 1>(r1, r2, b1);
        x[0] = r2[0][0] + dpp<0xB1>(r2[0][0]);
        x[1] = r2[1][0] + dpp<0xB1>(r2[1][0]);
    } else if constexpr (G == 2) {
        float r1[2][1];
        halve<0x141, 1>(a, r1, b2);
        x[0] = r1[0][0] + dpp<0x4E>(r1[0][0]);
        x[1] = r1[1][0] + dpp<0x4E>(r1[1][0]);
        x[0] += dpp<0xB1>(x[0]);
        x[1] += dpp<0xB1>(x[1]);
    } else {
        x[0] = sum_over_c(a[0][0]);
        x[1] = sum_over_c(a[1][0]);
    }
}

// Reductions over lane bits 3..5 (the 8 token pairs), used once per
// partition (sums) and on the rare rescale path (max).
__device__ __forceinline__ float max_over_tp(float x) {
    x = fmaxf(x, __shfl_xor(x, 8));
    x = fmaxf(x, __shfl_xor(x, 16));
    x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}
__device__ __forceinline__ float sum_over_tp(float x) {
    x += __shfl_xor(x, 8);
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T, int D, int G>
struct Cfg {
    static constexpr bool kBf16 = sizeof(T) == 2;
    static constexpr int kRowBytes = D * static_cast<int>(sizeof(T));
    static constexpr int kChunks = kRowBytes / 16;  // 16-byte chunks per row
    static constexpr int kCPL = kChunks / 8;        // chunks per lane per token
    static constexpr int kDPL = D / kWave;          // output dims per lane
    static constexpr int kPWords = kBf16 ? G * 8 : G * 16;
    static_assert(kCPL >= 1 && kChunks % 8 == 0, "row must be a multiple of 128 bytes");
    static_assert(kDPL >= 1, "head dim must be a multiple of 64");
};

// LDS address of a __shared__ object (what M0 takes for an LDS-DMA load).
__device__ __forceinline__ uint32_t lds_offset(const void *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (const __attribute__((address_space(3))) char *)(p)));
}

// One global_load_lds_dwordx4: every lane reads 16 bytes at sbase + voff and
// the wave's 64 x 16 bytes land in LDS at m0 + 16 * lane, without passing
// through VGPRs.  The nt bit marks the stream as read-once.  Issued from asm
// so that the compiler does not serialise the ring with vmcnt(0) before every
// LDS read; the kernel places the exact vmcnt waits itself (wait_vmem).
__device__ __forceinline__ void dma16(const void *sbase, uint32_t voff, uint32_t lds) {
    asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "{m0}"(lds)
                 : "memory");
}

// Wait until at most N vector-memory operations of this wave are in flight
// (they retire in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most `later` blocks of PER loads each are still in flight.
template <int PER, int NBUF>
__device__ __forceinline__ void wait_blocks(int later) {
    if constexpr (NBUF >= 4) {
        if (later >= 3) { wait_vmem<3 * PER>(); return; }
        if (later == 2) { wait_vmem<2 * PER>(); return; }
    }
    if constexpr (NBUF >= 2) {
        if (later >= 1) { wait_vmem<PER>(); return; }
    }
    wait_vmem<0>();
}

__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// One global_load_lds_dword: lane l's 4 bytes at sbase + voff land in LDS at
// m0 + 4 * l (used for the block ids of a segment).
__device__ __forceinline__ void dma4(const void *sbase, uint32_t voff, uint32_t lds) {
    asm volatile("global_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}

// s_waitcnt the compiler itself understands (it then knows its own loads,
// issued before, are complete): vmcnt(0), no wait on the other counters.
__device__ __forceinline__ void drain_vmem() {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    asm volatile("" ::: "memory");  // and no LDS read may be hoisted above it
}

// Inclusive prefix sum across the wave.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int t = __shfl_up(v, d);
        if (lane >= d) v += t;
    }
    return v;
}

// Blocks each work-group of the stream takes: an equal share of all
// (sequence, KV head, block) work, and at least kMinShare so that tiny
// batches do not split into fragments that cost more to merge than to run.
constexpr int kMinShare = 16;
__host__ __device__ __forceinline__ int stream_share(int total, int waves) {
    const int r = (total + waves - 1) / waves;
    return r > kMinShare ? r : kMinShare;
}

// ---------------------------------------------------------------------------
// Split-context partition kernel, stream-K schedule.
//
// All (sequence b, KV head g, cache block) work items are laid out in one
// global order (b, then g, then block) and cut into gridDim.x equal shares;
// work-group w streams share w, which may cross from one (b, g) "segment" to
// the next.  For each segment it touches it leaves (acc, max, sum) of the G
// query heads in partial slot w + (b * Hkv + g); the slots of one segment are
// therefore consecutive, from w0 + k to w1 + k where w0 and w1 are the first
// and last shares that overlap it.  Every work-group finds its share from
// the context lengths alone; work-group 0 also stores the per-sequence block
// prefix sums for the reduce.  Launched with one work-group per resident
// wave slot, so every wave streams for the whole kernel.
// ---------------------------------------------------------------------------
template <typename T, int D, int G, int NBUF>
__global__ __launch_bounds__(kWave) void grouped_partition_kernel(
    float *__restrict__ ws_acc, float2 *__restrict__ ws_ml, int32_t *__restrict__ ws_prefix,
    const T *__restrict__ q, const T *__restrict__ k_cache, const T *__restrict__ v_cache,
    const int32_t *__restrict__ block_tables, const int32_t *__restrict__ context_lens,
    float scale_log2, int num_seqs, int num_kv_heads, int max_blocks) {
    using C = Cfg<T, D, G>;
    constexpr int CPL = C::kCPL;
    constexpr int DPL = C::kDPL;
    constexpr int KV_INSTR = 2 * CPL;        // 16-byte loads per lane for K (and for V)
    constexpr int PER_BLOCK = 2 * KV_INSTR;  // LDS-DMA loads per block
    constexpr int SLOT_U4 = PER_BLOCK * kWave;
    static_assert((NBUF & (NBUF - 1)) == 0 && NBUF >= 2 && NBUF <= 4, "ring depth 2 or 4");

    const int lane = threadIdx.x;
    const int tp = lane >> 3;
    const int c = lane & 7;
    constexpr int LPH = 8 / G;                // lanes of a token pair per head
    const int hc = c / LPH;                   // the head whose softmax this lane carries
    const bool head_writer = (c % LPH) == 0;  // one lane per (token pair, head) publishes
    const int num_q_heads = num_kv_heads * G;

    // Ring of NBUF blocks.  Slot layout: K then V, each KV_INSTR rows of 64
    // lanes x 16 bytes; row (j * CPL + i), lane (tp, c) = token 2 tp + j,
    // 16-byte chunk c + 8 i of the row.
    __shared__ __attribute__((aligned(16))) uint4 s_ring[NBUF * SLOT_U4];
    __shared__ __attribute__((aligned(16))) uint32_t s_p[C::kPWords];
    __shared__ __attribute__((aligned(16))) int32_t s_ids[2][kWave];
    __shared__ float s_alpha[8];

    // ---- this work-group's share of the global block order ----------------
    int seq_blocks_total = 0;
    for (int base = 0; base < num_seqs; base += kWave) {
        const int bb = base + lane;
        const int nb = bb < num_seqs ? (context_lens[bb] + kBS - 1) / kBS : 0;
        const int incl = wave_incl_scan(nb, lane);
        if (blockIdx.x == 0 && bb < num_seqs) ws_prefix[bb] = seq_blocks_total + incl - nb;
        seq_blocks_total += __builtin_amdgcn_readlane(incl, kWave - 1);
    }
    if (blockIdx.x == 0 && lane == 0) ws_prefix[num_seqs] = seq_blocks_total;
    const int total = num_kv_heads * seq_blocks_total;
    const int share = stream_share(total, static_cast<int>(gridDim.x));
    const int64_t x0l = static_cast<int64_t>(blockIdx.x) * share;
    if (x0l >= total) return;
    const int x0 = static_cast<int>(x0l);
    const int x1 = min(x0 + share, total);

    // The sequence holding global block x0: first b whose blocks end past it.
    int b = 0, nbb = 0, cb = 0;
    for (int base = 0, carry = 0;; base += kWave) {
        const int bb = base + lane;
        const int nb = bb < num_seqs ? (context_lens[bb] + kBS - 1) / kBS : 0;
        const int incl = wave_incl_scan(nb, lane);
        const bool past = bb < num_seqs &&
                          static_cast<int64_t>(num_kv_heads) * (carry + incl) > x0;
        const uint64_t hit = __builtin_amdgcn_ballot_w64(past);
        if (hit != 0) {
            const int f = __builtin_ctzll(hit);
            b = base + f;
            nbb = __builtin_amdgcn_readlane(nb, f);
            cb = carry + __builtin_amdgcn_readlane(incl, f) - nbb;
            break;
        }
        carry += __builtin_amdgcn_readlane(incl, kWave - 1);
    }
    int g = (x0 - num_kv_heads * cb) / nbb;
    int blk_start = (x0 - num_kv_heads * cb) - g * nbb;

    const int64_t row_stride = static_cast<int64_t>(num_kv_heads) * C::kRowBytes;
    const int64_t blk_stride = kBS * row_stride;
    const uint32_t ring_lds = lds_offset(s_ring);
    const uint32_t ids_lds[2] = {lds_offset(&s_ids[0][0]), lds_offset(&s_ids[1][0])};

    // Where, in a slot's V rows, this lane finds the dword holding its first
    // output dim for token 2 tp' (row j = 0) and 2 tp' + 1 (row j = 1).
    constexpr int kEB = static_cast<int>(sizeof(T));
    const int pv_byte = lane * DPL * kEB;
    const int pv_chunk = pv_byte >> 4;
    const int pv_word = ((pv_chunk >> 3) * kWave + (pv_chunk & 7)) * 4 + ((pv_byte & 15) >> 2);
    // bf16 with one dim per lane: which half of the dword holds it
    const uint32_t pv_sel = (kEB == 2 && DPL == 1 && (lane & 1)) ? 0x07060302u : 0x05040100u;

    for (int x = x0;;) {
        // ======== segment (b, g): blocks [blk_start, blk_start + nblk) ========
        const int nblk = min(nbb - blk_start, x1 - x);
        const int ctx = context_lens[b];
        const int32_t *bt_row = block_tables + static_cast<int64_t>(b) * max_blocks;

        // block ids, 64 per LDS buffer; chunk m holds entries blk_start + 64 m + lane
        auto fetch_ids = [&](int m) {
            const int e = min(blk_start + kWave * m + lane, max_blocks - 1);
            dma4(bt_row, static_cast<uint32_t>(e) * 4u, ids_lds[m & 1]);
        };
        fetch_ids(0);
        if (nblk > kWave) fetch_ids(1);

        // q slices: chunk (c + 8 i) of each of the G heads of this group.
        uint4 qv[G][CPL];
        {
            const char *qb = reinterpret_cast<const char *>(q) +
                             (static_cast<int64_t>(b) * num_q_heads + g * G) * C::kRowBytes;
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int i = 0; i < CPL; ++i)
                    qv[h][i] = *reinterpret_cast<const uint4 *>(qb + h * C::kRowBytes +
                                                                (c + 8 * i) * 16);
        }
        // Byte offsets, inside one physical block, of this lane's two rows.
        uint32_t off[2][CPL];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < CPL; ++i)
                off[j][i] = static_cast<uint32_t>((2 * tp + j) * row_stride + g * C::kRowBytes +
                                                  (c + 8 * i) * 16);
        // Segment start: the ring is empty; q and the first ids must land
        // before the ring's vmcnt accounting starts.
        drain_vmem();

        const char *kbase = reinterpret_cast<const char *>(k_cache);
        const char *vbase = reinterpret_cast<const char *>(v_cache);

        float m_run = kNegInf;  // running max of head hc (scaled, log2 units)
        float l_run = 0.f;      // this lane's share of the running sum of head hc
        float acc[G][DPL];
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int d = 0; d < DPL; ++d) acc[h][d] = 0.f;

        // Start block n's K and V streaming into ring slot n % NBUF.  Entering
        // id chunk m (block 64 m) also starts the ids of chunk m + 1, which
        // are needed 64 blocks later.
        auto issue = [&](int n) {
            if ((n & (kWave - 1)) == 0 && n > 0 && n + kWave < nblk) fetch_ids((n >> 6) + 1);
            const int pb = __builtin_amdgcn_readfirstlane(s_ids[(n >> 6) & 1][n & (kWave - 1)]);
            const char *kb = kbase + static_cast<int64_t>(pb) * blk_stride;
            const char *vb = vbase + static_cast<int64_t>(pb) * blk_stride;
            const uint32_t slot = ring_lds + (n & (NBUF - 1)) * (SLOT_U4 * 16);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < CPL; ++i)
                    dma16(kb, off[j][i], slot + (j * CPL + i) * (kWave * 16));
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < CPL; ++i)
                    dma16(vb, off[j][i], slot + (KV_INSTR + j * CPL + i) * (kWave * 16));
        };

        auto compute_block = [&](int n) {
            const uint4 *slot = s_ring + (n & (NBUF - 1)) * SLOT_U4;
            const int tok0 = (blk_start + n) * kBS;
            const bool partial = tok0 + kBS > ctx;  // only the sequence's last block
            bool valid[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) valid[j] = !partial || (tok0 + 2 * tp + j < ctx);

            // ---- scores for the G heads of both tokens ---------------------
            uint4 kr[2][CPL];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < CPL; ++i) kr[j][i] = slot[(j * CPL + i) * kWave + lane];
            float part_dot[2][G];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    float a = 0.f;
#pragma unroll
                    for (int i = 0; i < CPL; ++i) {
                        if constexpr (C::kBf16) {
                            a = dot2_bf16(qv[h][i].x, kr[j][i].x, a);
                            a = dot2_bf16(qv[h][i].y, kr[j][i].y, a);
                            a = dot2_bf16(qv[h][i].z, kr[j][i].z, a);
                            a = dot2_bf16(qv[h][i].w, kr[j][i].w, a);
                        } else {
                            a = fmaf(as_f(qv[h][i].x), as_f(kr[j][i].x), a);
                            a = fmaf(as_f(qv[h][i].y), as_f(kr[j][i].y), a);
                            a = fmaf(as_f(qv[h][i].z), as_f(kr[j][i].z), a);
                            a = fmaf(as_f(qv[h][i].w), as_f(kr[j][i].w), a);
                        }
                    }
                    part_dot[j][h] = a;
                }

            // ---- online softmax for head hc --------------------------------
            float x2[2];
            reduce_scatter_c<G>(part_dot, c, x2);
#pragma unroll
            for (int j = 0; j < 2; ++j) x2[j] = valid[j] ? x2[j] * scale_log2 : kNegInf;
            const float xmax = fmaxf(x2[0], x2[1]);
            if (__builtin_amdgcn_ballot_w64(xmax > m_run + kSlack) != 0) {
                const float bmax = max_over_tp(xmax);
                const float m_new = fmaxf(m_run, bmax);
                const float alpha = exp2_fast(m_run - m_new);
                l_run *= alpha;
                m_run = m_new;
                if (tp == 0 && head_writer) s_alpha[hc] = alpha;
                __syncthreads();
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float a = s_alpha[h];
#pragma unroll
                    for (int d = 0; d < DPL; ++d) acc[h][d] *= a;
                }
            }
            const float p0 = exp2_fast(x2[0] - m_run);
            const float p1 = exp2_fast(x2[1] - m_run);

            __syncthreads();  // the previous block's reads of s_p are done
            if constexpr (C::kBf16) {
                const uint32_t pk = pack_bf16(p0, p1);
                l_run += bf16_lo(pk) + bf16_hi(pk);
                if (head_writer) s_p[hc * 8 + tp] = pk;
            } else {
                l_run += p0 + p1;
                if (head_writer)
                    *reinterpret_cast<float2 *>(&s_p[hc * 16 + 2 * tp]) = make_float2(p0, p1);
            }
            __syncthreads();

            // ---- P.V for all G heads of this lane's dims -------------------
            const uint32_t *vw =
                reinterpret_cast<const uint32_t *>(slot + KV_INSTR * kWave) + pv_word;
            constexpr int kRowW = CPL * kWave * 4;  // dwords between the j = 0 and j = 1 rows
            if constexpr (C::kBf16) {
#pragma unroll
                for (int quad = 0; quad < 2; ++quad) {
                    uint4 pq[G];
#pragma unroll
                    for (int h = 0; h < G; ++h)
                        pq[h] = *reinterpret_cast<const uint4 *>(&s_p[h * 8 + quad * 4]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int tq = quad * 4 + e;  // token pair 2 tq, 2 tq + 1
                        uint32_t a = vw[tq * 32];
                        uint32_t bb = vw[kRowW + tq * 32];
                        if (partial) {  // masked rows contribute exactly zero, NaN or not
                            if (tok0 + 2 * tq >= ctx) a = 0;
                            if (tok0 + 2 * tq + 1 >= ctx) bb = 0;
                        }
                        uint32_t vp[DPL];
                        if constexpr (DPL == 2) {
                            vp[0] = __builtin_amdgcn_perm(bb, a, 0x05040100u);
                            vp[1] = __builtin_amdgcn_perm(bb, a, 0x07060302u);
                        } else {
                            vp[0] = __builtin_amdgcn_perm(bb, a, pv_sel);
                        }
#pragma unroll
                        for (int h = 0; h < G; ++h) {
                            const uint32_t ph = e == 0 ? pq[h].x : e == 1 ? pq[h].y
                                              : e == 2 ? pq[h].z : pq[h].w;
#pragma unroll
                            for (int d = 0; d < DPL; ++d)
                                acc[h][d] = dot2_bf16(ph, vp[d], acc[h][d]);
                        }
                    }
                }
            } else {
#pragma unroll
                for (int t = 0; t < kBS; ++t) {
                    const uint32_t *row = vw + (t & 1) * kRowW + (t >> 1) * 32;
                    float vv[DPL];
#pragma unroll
                    for (int d = 0; d < DPL; ++d)
                        vv[d] = (partial && tok0 + t >= ctx) ? 0.f : as_f(row[d]);
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        const float ph = as_f(s_p[h * 16 + t]);
#pragma unroll
                        for (int d = 0; d < DPL; ++d) acc[h][d] = fmaf(ph, vv[d], acc[h][d]);
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
            wait_blocks<PER_BLOCK, NBUF>(min(NBUF - 1, nblk - 1 - n));
            compute_block(n);
        }

        // ---- this segment's partial: unnormalised acc, running max and sum ----
        const float l_tot = sum_over_tp(l_run);
        const int64_t slot_row =
            (static_cast<int64_t>(blockIdx.x) + static_cast<int64_t>(b) * num_kv_heads + g) * G;
        if (tp == 0 && head_writer) ws_ml[slot_row + hc] = make_float2(m_run, l_tot);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float *dst = ws_acc + (slot_row + h) * D + lane * DPL;
            if constexpr (DPL == 2)
                *reinterpret_cast<float2 *>(dst) = make_float2(acc[h][0], acc[h][1]);
            else
                dst[0] = acc[h][0];
        }

        x += nblk;
        if (x >= x1) break;
        // next segment in the global order; sequences with no blocks hold none
        blk_start = 0;
        if (++g == num_kv_heads) {
            g = 0;
            do {
                ++b;
                nbb = (context_lens[b] + kBS - 1) / kBS;
            } while (nbb == 0);
        }
        wait_lds();  // every LDS read of this segment is done before the next one's DMA
    }
}

// ---------------------------------------------------------------------------
// Reduce over the stream-K partial slots of each (sequence, query head):
// O = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s, M = max_s m_s.
// One work-group of W waves per (query head, sequence); wave w takes slots
// w, w + W, ... of the segment.
// ---------------------------------------------------------------------------
template <typename T, int D, int G, int W>
__global__ __launch_bounds__(kWave *W) void stream_reduce_kernel(
    T *__restrict__ out, const float *__restrict__ ws_acc, const float2 *__restrict__ ws_ml,
    const int32_t *__restrict__ ws_prefix, const int32_t *__restrict__ context_lens,
    int num_seqs, int num_kv_heads, int waves) {
    constexpr int DPL = D / kWave;
    const int h = blockIdx.x;
    const int b = blockIdx.y;
    const int g = h / G;
    const int hh = h - g * G;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int num_q_heads = num_kv_heads * G;
    const int nb = (context_lens[b] + kBS - 1) / kBS;
    T *o = out + (static_cast<int64_t>(b) * num_q_heads + h) * D + lane * DPL;

    __shared__ float s_max[W];
    __shared__ float s_num[W][D];
    __shared__ float s_den[W];

    if (nb <= 0) {  // empty context: O = 0
        if (wave == 0)
#pragma unroll
            for (int d = 0; d < DPL; ++d) o[d] = static_cast<T>(0.f);
        return;
    }
    const int total = num_kv_heads * ws_prefix[num_seqs];
    const int share = stream_share(total, waves);
    const int k = b * num_kv_heads + g;
    const int seg_lo = num_kv_heads * ws_prefix[b] + g * nb;
    const int w0 = seg_lo / share;
    const int n = (seg_lo + nb - 1) / share - w0 + 1;  // partial slots of this segment
    const int64_t first = (static_cast<int64_t>(w0) + k) * G + hh;  // row of slot w0 + k

    float M = kNegInf;
    for (int p = tid; p < n; p += kWave * W) M = fmaxf(M, ws_ml[first + static_cast<int64_t>(p) * G].x);
    for (int sh = 32; sh >= 1; sh >>= 1) M = fmaxf(M, __shfl_xor(M, sh));
    if constexpr (W > 1) {
        if (lane == 0) s_max[wave] = M;
        __syncthreads();
        M = s_max[0];
#pragma unroll
        for (int w = 1; w < W; ++w) M = fmaxf(M, s_max[w]);
    }

    float num[DPL];
#pragma unroll
    for (int d = 0; d < DPL; ++d) num[d] = 0.f;
    float den = 0.f;
    for (int p = wave; p < n; p += W) {
        const int64_t r = first + static_cast<int64_t>(p) * G;
        const float2 mp = ws_ml[r];
        const float wgt = exp2_fast(mp.x - M);
        den = fmaf(wgt, mp.y, den);
        const float *a = ws_acc + r * D + lane * DPL;
        if constexpr (DPL % 2 == 0) {
#pragma unroll
            for (int d = 0; d < DPL; d += 2) {
                const float2 v = *reinterpret_cast<const float2 *>(a + d);
                num[d] = fmaf(wgt, v.x, num[d]);
                num[d + 1] = fmaf(wgt, v.y, num[d + 1]);
            }
        } else {
            num[0] = fmaf(wgt, a[0], num[0]);
        }
    }
    if constexpr (W > 1) {
#pragma unroll
        for (int d = 0; d < DPL; ++d) s_num[wave][lane * DPL + d] = num[d];
        if (lane == 0) s_den[wave] = den;
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int w = 1; w < W; ++w) {
            den += s_den[w];
#pragma unroll
            for (int d = 0; d < DPL; ++d) num[d] += s_num[w][lane * DPL + d];
        }
    }
    if constexpr (sizeof(T) == 2) {
        if constexpr (DPL % 2 == 0) {
#pragma unroll
            for (int d = 0; d < DPL; d += 2)
                *reinterpret_cast<uint32_t *>(o + d) = pack_bf16(num[d] / den, num[d + 1] / den);
        } else {
            const __bf16 r = static_cast<__bf16>(num[0] / den);
            o[0] = __builtin_bit_cast(T, r);
        }
    } else {
#pragma unroll
        for (int d = 0; d < DPL; ++d) o[d] = num[d] / den;
    }
}

// ---------------------------------------------------------------------------
// Log-sum-exp reduce: O = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,
// M = max_p m_p, over the partitions that hold tokens of the sequence.
// One work-group per (query head, sequence); wave w takes partitions w, w+W..
// ---------------------------------------------------------------------------
template <typename T, int D, int W>
__global__ __launch_bounds__(kWave *W) void lse_reduce_kernel(
    T *__restrict__ out, const float *__restrict__ ws_acc, const float2 *__restrict__ ws_ml,
    const int32_t *__restrict__ context_lens, int num_q_heads, int num_parts, int part_tokens) {
    constexpr int DPL = D / kWave;
    const int h = blockIdx.x;
    const int b = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int ctx = context_lens[b];
    const int n = ctx > 0 ? (ctx + part_tokens - 1) / part_tokens : 0;
    const int64_t row = static_cast<int64_t>(b) * num_q_heads + h;
    T *o = out + row * D + lane * DPL;

    __shared__ float s_max[W];
    __shared__ float s_num[W][D];
    __shared__ float s_den[W];

    if (n == 0) {  // empty context: O = 0
        if (wave == 0)
#pragma unroll
            for (int d = 0; d < DPL; ++d) o[d] = static_cast<T>(0.f);
        return;
    }
    const float2 *ml = ws_ml + row * num_parts;
    float M = kNegInf;
    for (int p = tid; p < n; p += kWave * W) M = fmaxf(M, ml[p].x);
    for (int sh = 32; sh >= 1; sh >>= 1) M = fmaxf(M, __shfl_xor(M, sh));
    if constexpr (W > 1) {
        if (lane == 0) s_max[wave] = M;
        __syncthreads();
        M = s_max[0];
#pragma unroll
        for (int w = 1; w < W; ++w) M = fmaxf(M, s_max[w]);
    }

    float num[DPL];
#pragma unroll
    for (int d = 0; d < DPL; ++d) num[d] = 0.f;
    float den = 0.f;
    for (int p = wave; p < n; p += W) {
        const float2 mp = ml[p];
        const float w = exp2_fast(mp.x - M);
        den = fmaf(w, mp.y, den);
        const float *a = ws_acc + (row * num_parts + p) * D + lane * DPL;
        if constexpr (DPL % 2 == 0) {
#pragma unroll
            for (int d = 0; d < DPL; d += 2) {
                const float2 v = *reinterpret_cast<const float2 *>(a + d);
                num[d] = fmaf(w, v.x, num[d]);
                num[d + 1] = fmaf(w, v.y, num[d + 1]);
            }
        } else {
            num[0] = fmaf(w, a[0], num[0]);
        }
    }
    if constexpr (W > 1) {
#pragma unroll
        for (int d = 0; d < DPL; ++d) s_num[wave][lane * DPL + d] = num[d];
        if (lane == 0) s_den[wave] = den;
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int w = 1; w < W; ++w) {
            den += s_den[w];
#pragma unroll
            for (int d = 0; d < DPL; ++d) num[d] += s_num[w][lane * DPL + d];
        }
    }
    if constexpr (sizeof(T) == 2) {
        if constexpr (DPL % 2 == 0) {
#pragma unroll
            for (int d = 0; d < DPL; d += 2)
                *reinterpret_cast<uint32_t *>(o + d) = pack_bf16(num[d] / den, num[d + 1] / den);
        } else {
            const __bf16 r = static_cast<__bf16>(num[0] / den);
            o[0] = __builtin_bit_cast(T, r);
        }
    } else {
#pragma unroll
        for (int d = 0; d < DPL; ++d) o[d] = num[d] / den;
    }
}

// Work-groups of the stream: one per wave slot the partition kernel keeps
// resident on the current device, so that every wave streams from start to
// end.  Slots per CU = the smaller of the register limit (occupancy query)
// and the LDS limit (CU LDS / the kernel's static LDS), rounded down to a
// multiple of the 4 SIMDs so that every SIMD carries the same number of
// equal shares; capped by the workspace's slot count.
template <typename K>
int stream_waves(K kernel) {
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
    int w = cache[dev].load(std::memory_order_relaxed);
    if (w == 0) {
        int cus = 0, per_cu = 0, lds_cu = 0;
        hipFuncAttributes attr{};
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kWave, 0) != hipSuccess)
            per_cu = 0;
        if (hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                                  dev) == hipSuccess &&
            hipFuncGetAttributes(&attr, reinterpret_cast<const void *>(kernel)) == hipSuccess &&
            attr.sharedSizeBytes > 0) {
            const int by_lds = lds_cu / static_cast<int>(attr.sharedSizeBytes);
            if (by_lds < per_cu) per_cu = by_lds;
        }
        if (per_cu >= 4) per_cu -= per_cu % 4;
        w = cus * per_cu;
        if (w <= 0) w = 2048;  // 256 CUs x 2 waves per SIMD
        if (w > kStreamWavesMax) w = kStreamWavesMax;
        cache[dev].store(w, std::memory_order_relaxed);
    }
    if (const char *env = std::getenv("PA_STREAM_WAVES")) {  // tuning / tests
        const int v = std::atoi(env);
        if (v >= 1 && v <= kStreamWavesMax) w = v;
    }
    return w;
}

template <typename T, int D, int G, int NBUF>
pa_status enqueue_grouped(const DecodeShape &s, const DecodeArgs &a, const DecodePlan &p,
                          float scale_log2, hipStream_t stream, std::string *why) {
    char *ws = static_cast<char *>(a.workspace);
    float *acc = reinterpret_cast<float *>(ws + p.acc_offset);
    float2 *ml = reinterpret_cast<float2 *>(ws + p.ml_offset);
    int32_t *prefix = reinterpret_cast<int32_t *>(ws + p.prefix_offset);
    const auto kernel = grouped_partition_kernel<T, D, G, NBUF>;
    const int waves = stream_waves(kernel);
    hipLaunchKernelGGL(kernel, dim3(waves), dim3(kWave), 0, stream, acc, ml, prefix,
                       static_cast<const T *>(a.q), static_cast<const T *>(a.k_cache),
                       static_cast<const T *>(a.v_cache), a.block_tables, a.context_lens,
                       scale_log2, s.num_seqs, s.num_kv_heads, s.max_blocks_per_seq);
    pa_status st = hip_status(hipGetLastError(), why, "partition launch");
    if (st != PA_OK) return st;
    const dim3 grid(s.num_q_heads, s.num_seqs);
    hipLaunchKernelGGL((stream_reduce_kernel<T, D, G, 4>), grid, dim3(kWave * 4), 0, stream,
                       static_cast<T *>(a.out), acc, ml, prefix, a.context_lens, s.num_seqs,
                       s.num_kv_heads, waves);
    return hip_status(hipGetLastError(), why, "reduce launch");
}

template <typename T, int D>
pa_status enqueue_grouped_g(const DecodeShape &s, const DecodeArgs &a, const DecodePlan &p,
                            float scale_log2, hipStream_t stream, std::string *why) {
    if (p.ring_depth == 4) {
        switch (p.group) {
            case 1: return enqueue_grouped<T, D, 1, 4>(s, a, p, scale_log2, stream, why);
            case 2: return enqueue_grouped<T, D, 2, 4>(s, a, p, scale_log2, stream, why);
            case 4: return enqueue_grouped<T, D, 4, 4>(s, a, p, scale_log2, stream, why);
            default: return enqueue_grouped<T, D, 8, 4>(s, a, p, scale_log2, stream, why);
        }
    }
    switch (p.group) {
        case 1: return enqueue_grouped<T, D, 1, 2>(s, a, p, scale_log2, stream, why);
        case 2: return enqueue_grouped<T, D, 2, 2>(s, a, p, scale_log2, stream, why);
        case 4: return enqueue_grouped<T, D, 4, 2>(s, a, p, scale_log2, stream, why);
        default: return enqueue_grouped<T, D, 8, 2>(s, a, p, scale_log2, stream, why);
    }
}

template <typename T, int D>
void enqueue_reduce(const DecodeShape &s, const DecodeArgs &a, const DecodePlan &p,
                    int part_tokens, hipStream_t stream) {
    const char *ws = static_cast<const char *>(a.workspace);
    const float *acc = reinterpret_cast<const float *>(ws + p.acc_offset);
    const float2 *ml = reinterpret_cast<const float2 *>(ws + p.ml_offset);
    const dim3 grid(s.num_q_heads, s.num_seqs);
    if (p.num_parts > 8)
        hipLaunchKernelGGL((lse_reduce_kernel<T, D, 4>), grid, dim3(kWave * 4), 0, stream,
                           static_cast<T *>(a.out), acc, ml, a.context_lens, s.num_q_heads,
                           p.num_parts, part_tokens);
    else
        hipLaunchKernelGGL((lse_reduce_kernel<T, D, 1>), grid, dim3(kWave), 0, stream,
                           static_cast<T *>(a.out), acc, ml, a.context_lens, s.num_q_heads,
                           p.num_parts, part_tokens);
}

}  // namespace

pa_status launch_lse_reduce(const DecodeShape &s, const DecodeArgs &a, const DecodePlan &p,
                            int part_tokens, hipStream_t stream, std::string *why) {
    if (s.dtype == PA_BF16) {
        if (s.head_dim_v == 64) enqueue_reduce<uint16_t, 64>(s, a, p, part_tokens, stream);
        else if (s.head_dim_v == 128) enqueue_reduce<uint16_t, 128>(s, a, p, part_tokens, stream);
        else enqueue_reduce<uint16_t, 512>(s, a, p, part_tokens, stream);
    } else {
        if (s.head_dim_v == 64) enqueue_reduce<float, 64>(s, a, p, part_tokens, stream);
        else enqueue_reduce<float, 128>(s, a, p, part_tokens, stream);
    }
    return hip_status(hipGetLastError(), why, "reduce launch");
}

pa_status launch_grouped_decode(const DecodeShape &s, const DecodeArgs &a, const DecodePlan &p,
                                hipStream_t stream, std::string *why) {
    if (s.num_seqs == 0) return PA_OK;
    const float scale_log2 = static_cast<float>(static_cast<double>(a.scale) * 1.4426950408889634);
    if (s.dtype == PA_BF16) {
        if (s.head_dim_k == 64)
            return enqueue_grouped_g<uint16_t, 64>(s, a, p, scale_log2, stream, why);
        return enqueue_grouped_g<uint16_t, 128>(s, a, p, scale_log2, stream, why);
    }
    if (s.head_dim_k == 64) return enqueue_grouped_g<float, 64>(s, a, p, scale_log2, stream, why);
    return enqueue_grouped_g<float, 128>(s, a, p, scale_log2, stream, why);
}

}  // namespace pa
