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
// gfx950 mapping (each wave64 streams one KV head of a share of the blocks;
// a work-group holds kGroupWaves such waves, which the hardware places one
// per SIMD, and the waves of a team stream neighbouring heads of the same
// share without synchronising):
//  * A 16-token cache block of one KV head is 16 rows of D elements.  Lane
//    (tp = lane / 8, c = lane % 8) owns rows 2tp and 2tp+1, 16-byte chunks
//    c, c+8, ...: every load is 16 bytes wide and each group of 8 lanes reads
//    one 128-byte line.
//  * K and V travel HBM -> LDS with global_load_lds_dwordx4 (no VGPRs on the
//    way) into a ring of NBUF blocks, so several blocks are in flight while
//    the wave computes on an earlier one; explicit vmcnt waits retire exactly
//    one block per step, and the ring runs on across a share's segments (the
//    next segment's block ids and q are fetched ahead, see "segments").
//  * The block is fetched once for all G query heads of the group: each lane
//    holds its slice of q for all G heads and forms G partial dot products
//    per token with v_dot2_f32_bf16 (fp32 FMA for fp32 inputs).  The 8 lanes
//    of a token pair finish the dot products with three DPP adds
//    (quad_perm 1032, quad_perm 2301, row_half_mirror).
//  * Softmax: lane c carries head c / (8 / G).  The running max is raised only when a
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

#include <cstdint>

#include "device_common.h"
#include "hip_util.h"
#include "launch.h"

namespace pa {
namespace {

constexpr int kBS = 16;              // tokens per cache block on this path
constexpr float kSlack = 8.0f;       // lazy-rescale threshold, log2 units

// Sum over the 8 lanes of a token pair (lane bits 0..2).
__device__ __forceinline__ float sum_over_c(float x) {
    x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
    x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
    x += dpp<0x141>(x);  // row_half_mirror: the other quad of the 8-lane half row
    return x;
}

// The 8 lanes of a token pair each hold partial dot products over their own
// dims for both tokens and all G heads.  Reduce-scatter them so that lane c
// ends with the full sums (both tokens) of its head hc = c / (8 / G).  Each
// lane stores its partials in a lane-dependent order: slot i holds head
// i ^ hc (q is loaded in that order).  A step with partner c ^ m (m = 7:
// row_half_mirror, m = 2: quad_perm 2301, m = 1: quad_perm 1032) keeps the
// lower half of the slots, whose heads share the lane's bit of hc, and adds
// the partner's slot i ^ (m >> s) (s = log2(8 / G)), which holds the same
// head there; the slot index is the same on every lane, so no select is
// needed.  Once one head is left the remaining steps are plain all-reduce adds.
template <int G>
__device__ __forceinline__ void reduce_scatter_c(const float (&a)[2][G], float (&x)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        if constexpr (G == 8) {
            float r1[4], r2[2];
#pragma unroll
            for (int i = 0; i < 4; ++i) r1[i] = a[j][i] + dpp<0x141>(a[j][i ^ 7]);
#pragma unroll
            for (int i = 0; i < 2; ++i) r2[i] = r1[i] + dpp<0x4E>(r1[i ^ 2]);
            x[j] = r2[0] + dpp<0xB1>(r2[1]);
        } else if constexpr (G == 4) {
            float r1[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) r1[i] = a[j][i] + dpp<0x141>(a[j][i ^ 3]);
            const float r2 = r1[0] + dpp<0x4E>(r1[1]);
            x[j] = r2 + dpp<0xB1>(r2);
        } else if constexpr (G == 2) {
            float r1 = a[j][0] + dpp<0x141>(a[j][1]);
            r1 += dpp<0x4E>(r1);
            x[j] = r1 + dpp<0xB1>(r1);
        } else {
            x[j] = sum_over_c(a[j][0]);
        }
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

template <typename T, int D, int G>
struct Cfg {
    static constexpr bool kBf16 = sizeof(T) == 2;
    static constexpr int kRowBytes = D * static_cast<int>(sizeof(T));
    static constexpr int kChunks = kRowBytes / 16;  // 16-byte chunks per row
    static constexpr int kCPL = kChunks / 8;        // chunks per lane per token
    static constexpr int kDPL = D / kWave;          // output dims per lane
    static constexpr int kPWords = kBf16 ? G * 8 : G * 16;
    // A segment's q rows (G heads) reach LDS in kQDma 1 KB LDS-DMA loads.
    static constexpr int kQBytes = G * kRowBytes;
    static constexpr int kQDma = (kQBytes + 1023) / 1024;
    static_assert(kCPL >= 1 && kChunks % 8 == 0, "row must be a multiple of 128 bytes");
    static_assert(kDPL >= 1, "head dim must be a multiple of 64");
};

// Independent streaming waves per work-group: 4 (one per SIMD) when their
// LDS fits in a CU's 160 KB, else 2, else 1.
template <typename T, int D, int G, int NBUF>
constexpr int group_waves() {
    using C = Cfg<T, D, G>;
    constexpr int per_wave = NBUF * 2 * 2 * C::kCPL * kWave * 16 + C::kPWords * 4 + 2 * kWave * 4 +
                             8 * 4 + 2 * C::kQDma * 1024;
    return 4 * per_wave <= 160 * 1024 ? 4 : 2 * per_wave <= 160 * 1024 ? 2 : 1;
}

// ---------------------------------------------------------------------------
// Split-context partition kernel, stream-K schedule.
//
// The waves of a work-group form teams of TH (team_heads) waves; the KV
// heads of a sequence form NC = Hkv / TH chunks of TH heads.  All (sequence
// b, chunk ch, cache block) work items are laid out in one global order (b,
// then ch, then block) and cut into nshares equal shares; team s streams
// share s, which may cross from one (b, ch) "segment" to the next, wave hw of
// the team taking KV head g = ch TH + hw of every block.  The team's waves do
// not synchronise: they start together and do the same work, so they read
// neighbouring head slices of the same token rows at about the same time.
// For each segment a share touches, each wave leaves (acc, max, sum) of its G
// query heads in partial slot s + (b NC + ch), row (slot TH + hw) G + head;
// the slots of one segment are therefore consecutive, from w0 + k to w1 + k
// (k = b NC + ch) where w0 and w1 are the first and last shares that overlap
// it.  Every team finds its share from the context lengths alone; team 0
// also stores the per-sequence block prefix sums for the reduce.  Launched
// with one work-group per resident slot, so every wave streams for the
// whole kernel.  TH = 1 is one share per wave.
// ---------------------------------------------------------------------------
template <typename T, int D, int G, int NBUF, int kGroupWaves = group_waves<T, D, G, NBUF>()>
__global__ __launch_bounds__(kWave *kGroupWaves) void grouped_partition_kernel(
    float *__restrict__ ws_acc, float2 *__restrict__ ws_ml, int32_t *__restrict__ ws_prefix,
    const T *__restrict__ q, const T *__restrict__ k_cache, const T *__restrict__ v_cache,
    const int32_t *__restrict__ block_tables, const int32_t *__restrict__ context_lens,
    float scale_log2, int num_seqs, int num_kv_heads, int max_blocks, int nshares, int team_heads,
    int window) {
    using C = Cfg<T, D, G>;
    constexpr int CPL = C::kCPL;
    constexpr int DPL = C::kDPL;
    constexpr int KV_INSTR = 2 * CPL;        // 16-byte loads per lane for K (and for V)
    constexpr int PER_BLOCK = 2 * KV_INSTR;  // LDS-DMA loads per block
    constexpr int SLOT_U4 = PER_BLOCK * kWave;
    static_assert((NBUF & (NBUF - 1)) == 0 && NBUF >= 2 && NBUF <= 4, "ring depth 2 or 4");

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int sid = (blockIdx.x * kGroupWaves + wave) / team_heads;  // this wave's team and share
    const int hw = wave % team_heads;                                 // its head within a chunk
    const int nchunks = num_kv_heads / team_heads;
    if (sid >= nshares) return;  // uniform over the team; waves never wait on each other
    const int tp = lane >> 3;
    const int c = lane & 7;
    constexpr int LPH = 8 / G;                // lanes of a token pair per head
    const int hc = c / LPH;                   // the head whose softmax this lane carries
    const bool head_writer = (c % LPH) == 0;  // one lane per (token pair, head) publishes
    const int num_q_heads = num_kv_heads * G;

    // Ring of NBUF blocks.  Slot layout: K then V, each KV_INSTR rows of 64
    // lanes x 16 bytes; row (j * CPL + i), lane (tp, c) = token 2 tp + j,
    // 16-byte chunk c + 8 i of the row.
    // (every wave of the work-group has its own)
    __shared__ __attribute__((aligned(16))) uint4 s_ring_all[kGroupWaves][NBUF * SLOT_U4];
    __shared__ __attribute__((aligned(16))) uint32_t s_p_all[kGroupWaves][C::kPWords];
    __shared__ __attribute__((aligned(16))) int32_t s_ids_all[kGroupWaves][2][kWave];
    __shared__ float s_alpha_all[kGroupWaves][8];
    // q rows of the segment being started, for segments k & 1
    __shared__ __attribute__((aligned(16))) uint4 s_q_all[kGroupWaves][2][C::kQDma * kWave];
    uint4 *s_ring = s_ring_all[wave];
    uint32_t *s_p = s_p_all[wave];
    int32_t(*s_ids)[kWave] = s_ids_all[wave];
    float *s_alpha = s_alpha_all[wave];

    // ---- this team's share of the global block order -------------------------
    ShareSpan sp;
    if (!find_share(sid, nshares, num_seqs, nchunks, kBS, context_lens, ws_prefix, lane, sp,
                    window, hw == 0))
        return;
    const int P = sp.x1 - sp.x0;  // blocks of the share, over every segment it touches

    const int64_t row_stride = static_cast<int64_t>(num_kv_heads) * C::kRowBytes;
    // bytes per physical block: below 2^32 (at most 65535 KV heads of 512-byte rows), so a
    // block's offset is one 32 x 32 -> 64-bit product
    const uint32_t blk_stride = static_cast<uint32_t>(kBS * row_stride);
    const uint32_t ring_lds = lds_offset(s_ring);
    const uint32_t ids_lds[2] = {lds_offset(&s_ids[0][0]), lds_offset(&s_ids[1][0])};
    const uint32_t q_lds[2] = {lds_offset(&s_q_all[wave][0][0]), lds_offset(&s_q_all[wave][1][0])};

    // Where, in a slot's V rows, this lane finds the dword holding its first
    // output dim for token 2 tp' (row j = 0) and 2 tp' + 1 (row j = 1).
    constexpr int kEB = static_cast<int>(sizeof(T));
    const int pv_byte = lane * DPL * kEB;
    const int pv_chunk = pv_byte >> 4;
    const int pv_word = ((pv_chunk >> 3) * kWave + (pv_chunk & 7)) * 4 + ((pv_byte & 15) >> 2);
    // bf16 with one dim per lane: which half of the dword holds it
    const uint32_t pv_sel = (kEB == 2 && DPL == 1 && (lane & 1)) ? 0x07060302u : 0x05040100u;

    // Byte offsets, inside one physical block and KV head, of this lane's two
    // rows (the head's offset goes into the scalar base).
    uint32_t off[2][CPL];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < CPL; ++i)
            off[j][i] = static_cast<uint32_t>((2 * tp + j) * row_stride + (c + 8 * i) * 16);
    const char *kbase = reinterpret_cast<const char *>(k_cache);
    const char *vbase = reinterpret_cast<const char *>(v_cache);

    // ---- segments ---------------------------------------------------------------
    // The share is one stream of P blocks over consecutive (sequence, chunk)
    // segments.  Segment k of the share: sequence b, head chunk ch (this wave's
    // KV head g = ch TH + hw), its blocks from window block blk0 on, nblk of
    // them in this share.  Two cursors walk the stream: the issue side starts
    // each block's K/V loads NBUF - 1 blocks ahead of the compute side, and
    // crosses into the next segment as soon as the current one is issued, so a
    // segment switch costs the compute side no memory round trip.  The next
    // segment's block ids and q rows are fetched into LDS when the issue side
    // enters the current segment's last chunk of 64 blocks; the issue side
    // never runs more than one segment ahead of the compute side, which
    // bounds the q buffers to two.
    struct Seg {
        int b, ch, blk0, nblk, ctx, tbl0;  // tbl0: block-table index of the first block
    };
    auto make_seg = [&](int b, int ch, int blk0, int s0) {
        Seg sg;
        sg.b = b;
        sg.ch = ch;
        sg.blk0 = blk0;
        sg.ctx = context_lens[b];
        sg.nblk = min(window_blocks(sg.ctx, window, kBS) - blk0, P - s0);
        sg.tbl0 = blk0 + window_first_block(sg.ctx, window, kBS);
        return sg;
    };
    // the segment after sg in the global order (there is one: the share goes on)
    auto successor = [&](const Seg &sg, int s0) {
        int b = sg.b, ch = sg.ch + 1;
        if (ch == nchunks) {
            ch = 0;
            do {
                ++b;
            } while (window_blocks(context_lens[b], window, kBS) == 0);
        }
        return make_seg(b, ch, 0, s0);
    };
    // block ids: chunk m of segment sg (entries tbl0 + 64 m + lane) into buffer buf
    auto fetch_ids = [&](const Seg &sg, int m, int buf) {
        const int32_t *bt_row = block_tables + static_cast<int64_t>(sg.b) * max_blocks;
        const int e = min(sg.tbl0 + kWave * m + lane, max_blocks - 1);
        dma4(bt_row, static_cast<uint32_t>(e) * 4u, ids_lds[buf]);
    };
    // q rows of segment sg's G heads into q buffer buf (kQDma loads; lanes past
    // the rows reread the last 16 bytes into the buffer's unused tail)
    auto fetch_q = [&](const Seg &sg, int buf) {
        const char *qb = reinterpret_cast<const char *>(q) +
                         (static_cast<int64_t>(sg.b) * num_q_heads + (sg.ch * team_heads + hw) * G) *
                             C::kRowBytes;
        sgpr_settle(qb);
#pragma unroll
        for (int i = 0; i < C::kQDma; ++i)
            dma16(qb, static_cast<uint32_t>(min(1024 * i + 16 * lane, C::kQBytes - 16)),
                  q_lds[buf] + 1024 * i);
    };

    // ---- issue side -------------------------------------------------------------
    Seg is = make_seg(sp.b, sp.g, sp.blk, 0);
    int is_k = 0, is_s0 = 0, in = 0, ipar = 0;  // ids chunk m of `is` sits in buffer (ipar + m) & 1
    // this wave's KV head inside the pools, for segment `is`
    auto head_base = [&](const char *pool, const Seg &sg) {
        return pool + static_cast<int64_t>(sg.ch * team_heads + hw) * C::kRowBytes;
    };
    const char *k_seg = head_base(kbase, is);
    const char *v_seg = head_base(vbase, is);
    // The id of block `in`, read from LDS one issue ahead (valid when id_ready):
    // the LDS round trip then overlaps the compute instead of the issue.
    int id_next = 0;
    bool id_ready = false;
    Seg nx = is;
    int nx_ipar = 0;
    bool nx_ready = false;
    int gi = 0;  // blocks issued
    int cs_k = 0;  // the compute side's segment (the issue side stays within one of it)

    // Wait until the successor's id and q fetches have landed, `tail` blocks
    // (kQDma + tail * PER_BLOCK loads) having been issued after the id fetch.
    auto wait_since_fetch = [&](int tail) {
        if constexpr (NBUF >= 4) {
            if (tail >= 3) { wait_vmem<C::kQDma + 3 * PER_BLOCK>(); return; }
            if (tail == 2) { wait_vmem<C::kQDma + 2 * PER_BLOCK>(); return; }
        }
        wait_vmem<C::kQDma + PER_BLOCK>();
    };

    // Issues the next block of the stream; false when it must wait for the
    // compute side to reach the current issue segment first.
    auto issue_next = [&]() -> bool {
        if (in == is.nblk) {
            if (is_k > cs_k) return false;
            // The successor's first ids were fetched, then its q, then the
            // loads of the `tail` blocks of the last chunk: with fewer than
            // NBUF of them the compute side has not waited for the fetch yet,
            // so wait here for everything issued before those loads.
            const int tail = is.nblk - ((is.nblk - 1) & ~(kWave - 1));
            if (tail < NBUF) wait_since_fetch(tail);
            is_s0 += is.nblk;
            is = nx;
            ipar = nx_ipar;
            ++is_k;
            in = 0;
            nx_ready = false;
            id_ready = false;
            k_seg = head_base(kbase, is);
            v_seg = head_base(vbase, is);
        }
        if ((in & (kWave - 1)) == 0) {  // entering chunk m: fetch what comes 64 blocks later
            const int m = in >> 6;
            if (in + kWave < is.nblk) {
                fetch_ids(is, m + 1, (ipar + m + 1) & 1);
            } else if (is_s0 + is.nblk < P && !nx_ready) {
                nx = successor(is, is_s0 + is.nblk);
                nx_ipar = (ipar + m + 1) & 1;
                fetch_ids(nx, 0, nx_ipar);
                fetch_q(nx, (is_k + 1) & 1);
                nx_ready = true;
            }
        }
        int pb;
        if (id_ready)
            pb = __builtin_amdgcn_readfirstlane(id_next);
        else
            pb = __builtin_amdgcn_readfirstlane(s_ids[(ipar + (in >> 6)) & 1][in & (kWave - 1)]);
        const uint64_t blk_off = static_cast<uint64_t>(static_cast<uint32_t>(pb)) * blk_stride;
        const char *kb = k_seg + blk_off;
        const char *vb = v_seg + blk_off;
        const uint32_t slot = ring_lds + (gi & (NBUF - 1)) * (SLOT_U4 * 16);
        sgpr_settle(kb);
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
        ++in;
        ++gi;
        // Read the next id of this segment now.  Its chunk was fetched 64
        // blocks before its first block (the compute side has waited for
        // everything issued before that), and the next fetch writes the other
        // buffer.  A successor segment's first id is read at the switch, after
        // the wait for its fetch.
        id_ready = in < is.nblk;
        if (id_ready) id_next = s_ids[(ipar + (in >> 6)) & 1][in & (kWave - 1)];
        return true;
    };

    // ---- compute side -----------------------------------------------------------
    Seg cs = is;
    float m_run = kNegInf;  // running max of head hc (scaled, log2 units)
    float l_run = 0.f;      // this lane's share of the running sum of head hc
    float acc[G][DPL];
    // q slices: chunk (c + 8 i) of each of the G heads of the segment's group;
    // slot h holds head h ^ hc (the order reduce_scatter_c works in)
    uint4 qv[G][CPL];
    auto load_q = [&](int buf) {
        const uint4 *qs = reinterpret_cast<const uint4 *>(buf ? &s_q_all[wave][1][0] : &s_q_all[wave][0][0]);
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int i = 0; i < CPL; ++i)
                qv[h][i] = qs[((h ^ hc) * C::kRowBytes + (c + 8 * i) * 16) >> 4];
    };
    auto reset = [&]() {
        m_run = kNegInf;
        l_run = 0.f;
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int d = 0; d < DPL; ++d) acc[h][d] = 0.f;
    };

    auto compute_block = [&](int n, int g_slot) {
        const uint4 *slot = s_ring + (g_slot & (NBUF - 1)) * SLOT_U4;
        const int ctx = cs.ctx;
        const int wstart = window_start(ctx, window);
        const int tok0 = (cs.tbl0 + n) * kBS;
        // only the sequence's last block, and the window's first, hold tokens
        // outside [wstart, ctx); V rows below wstart are real data and get
        // weight 0, rows at or past ctx are zeroed below
        const bool partial = tok0 + kBS > ctx || tok0 < wstart;
        bool valid[2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
            valid[j] = !partial || (tok0 + 2 * tp + j < ctx && tok0 + 2 * tp + j >= wstart);

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
                        a = i == 0 ? dot2_bf16_0(qv[h][i].x, kr[j][i].x)
                                   : dot2_bf16(qv[h][i].x, kr[j][i].x, a);
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
        reduce_scatter_c<G>(part_dot, x2);
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
            wait_lds();  // the wave's own LDS writes are complete
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float a = s_alpha[h];
#pragma unroll
                for (int d = 0; d < DPL; ++d) acc[h][d] *= a;
            }
        }
        const float p0 = exp2_fast(x2[0] - m_run);
        const float p1 = exp2_fast(x2[1] - m_run);

        wait_lds();  // the previous block's reads of s_p are done
        if constexpr (C::kBf16) {
            const uint32_t pk = pack_bf16(p0, p1);
            l_run += bf16_lo(pk) + bf16_hi(pk);
            if (head_writer) s_p[hc * 8 + tp] = pk;
        } else {
            l_run += p0 + p1;
            if (head_writer)
                *reinterpret_cast<float2 *>(&s_p[hc * 16 + 2 * tp]) = make_float2(p0, p1);
        }
        wait_lds();  // this wave's probabilities are in LDS

        // ---- P.V for all G heads of this lane's dims -------------------
        const uint32_t *vw =
            reinterpret_cast<const uint32_t *>(slot + KV_INSTR * kWave) + pv_word;
        constexpr int kRowW = CPL * kWave * 4;  // dwords between the j = 0 and j = 1 rows
        if constexpr (C::kBf16) {
            // Every LDS read of the product first (probabilities of both
            // halves, the V words of all 8 token pairs), then the arithmetic:
            // a lone wave on its SIMD hides the reads' latency only behind its
            // own later instructions.
            uint4 pq[2][G];
            uint32_t va[8], vb[8];
#pragma unroll
            for (int quad = 0; quad < 2; ++quad)
#pragma unroll
                for (int h = 0; h < G; ++h)
                    pq[quad][h] = *reinterpret_cast<const uint4 *>(&s_p[h * 8 + quad * 4]);
#pragma unroll
            for (int tq = 0; tq < 8; ++tq) {
                va[tq] = vw[tq * 32];
                vb[tq] = vw[kRowW + tq * 32];
            }
            __builtin_amdgcn_sched_barrier(0);
            // Rows at or past the context contribute exactly zero, NaN or
            // not.  Only a partial block compares tokens with the context
            // length, in place on the loaded words, so that one copy of the
            // arithmetic serves every block.
            if (partial) {
#pragma unroll
                for (int tq = 0; tq < 8; ++tq) {
                    if (tok0 + 2 * tq >= ctx) va[tq] = 0;
                    if (tok0 + 2 * tq + 1 >= ctx) vb[tq] = 0;
                }
            }
#pragma unroll
            for (int tq = 0; tq < 8; ++tq) {  // token pair 2 tq, 2 tq + 1
                uint32_t vp[DPL];
                if constexpr (DPL == 2) {
                    vp[0] = __builtin_amdgcn_perm(vb[tq], va[tq], 0x05040100u);
                    vp[1] = __builtin_amdgcn_perm(vb[tq], va[tq], 0x07060302u);
                } else {
                    vp[0] = __builtin_amdgcn_perm(vb[tq], va[tq], pv_sel);
                }
                const int e = tq & 3;
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const uint4 &pw = pq[tq >> 2][h];
                    const uint32_t ph = e == 0 ? pw.x : e == 1 ? pw.y : e == 2 ? pw.z : pw.w;
#pragma unroll
                    for (int d = 0; d < DPL; ++d)
                        acc[h][d] = dot2_bf16(ph, vp[d], acc[h][d]);
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

    // A segment's partial (unnormalised acc, running max and sum) is kept in
    // registers and written when the share ends, or when more than kPend
    // wait: vmcnt counts stores with the loads, in issue order, so a block
    // loaded after a store cannot be waited for before the store completes,
    // and under the read stream that takes longer than the ring's slack (on
    // c3 the stores at every segment switch cost about 10 us of 315).
    struct Part {
        float acc[G][DPL];
        float m, l;
        int64_t row;  // first row of the segment's slot (uniform)
    };
    constexpr int kPend = 2;
    Part pend[kPend];
    int npend = 0;  // (uniform)
    auto write_part = [&](const Part &pp) {
        if (tp == 0 && head_writer) ws_ml[pp.row + hc] = make_float2(pp.m, pp.l);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float *dst = ws_acc + (pp.row + h) * D + lane * DPL;
            if constexpr (DPL == 2)
                *reinterpret_cast<float2 *>(dst) = make_float2(pp.acc[h][0], pp.acc[h][1]);
            else
                dst[0] = pp.acc[h][0];
        }
    };
    auto finish_segment = [&]() {
        Part cur;
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int d = 0; d < DPL; ++d) cur.acc[h][d] = acc[h][d];
        cur.m = m_run;
        cur.l = sum_over_tp(l_run);
        cur.row = ((static_cast<int64_t>(sid) + static_cast<int64_t>(cs.b) * nchunks + cs.ch) * team_heads +
                   hw) * G;
        if (npend == kPend) {  // the oldest goes out now
            write_part(pend[0]);
#pragma unroll
            for (int i = 0; i + 1 < kPend; ++i) pend[i] = pend[i + 1];
            pend[kPend - 1] = cur;
        } else {
#pragma unroll
            for (int i = 0; i < kPend; ++i)
                if (i == npend) pend[i] = cur;
            ++npend;
        }
    };

    // ---- prologue: the first segment's ids and q, then the ring -------------------
    fetch_ids(is, 0, 0);
    fetch_q(is, 0);
    drain_vmem();  // (the compiler's own loads too: nothing of it is pending in the loop)
    load_q(0);
    reset();
    for (int n = 0; n < NBUF - 1 && gi < P; ++n) issue_next();

    // Segments of the share, then their blocks (block gcb of the share is
    // block n of segment cs).
    int gcb = 0;
    for (;;) {
        for (int n = 0; n < cs.nblk; ++n, ++gcb) {
            while (gi < P && gi <= gcb + NBUF - 1) {
                wait_lds();  // slot gi % NBUF, the ids and the q buffers in LDS are read
                if (!issue_next()) break;
            }
            wait_blocks<PER_BLOCK, NBUF>(min(NBUF - 1, gi - 1 - gcb));
            compute_block(n, gcb);
        }
        finish_segment();
        if (gcb == P) break;
        // The issue side is in the next segment already (it issued the
        // segment's first block before this segment's last was computed).
        cs = is;
        ++cs_k;
        // That first block has landed, and the segment's q rows (loaded
        // before it) with it.  They go to registers before the issue side
        // may refill that q buffer for the segment after next.
        wait_blocks<PER_BLOCK, NBUF>(min(NBUF - 1, gi - 1 - gcb));
        load_q(cs_k & 1);
        reset();
    }
#pragma unroll
    for (int i = 0; i < kPend; ++i)
        if (i < npend) write_part(pend[i]);
}

template <typename T, int D, int G, int NBUF>
pa_status enqueue_grouped(const DecodeShape &s, const DecodeArgs &a, const DecodePlan &p,
                          float scale_log2, hipStream_t stream, std::string *why) {
    char *ws = static_cast<char *>(a.workspace);
    float *acc = reinterpret_cast<float *>(ws + p.acc_offset);
    float2 *ml = reinterpret_cast<float2 *>(ws + p.ml_offset);
    int32_t *prefix = reinterpret_cast<int32_t *>(ws + p.prefix_offset);
    const auto kernel = grouped_partition_kernel<T, D, G, NBUF>;
    constexpr int kGroupWaves = group_waves<T, D, G, NBUF>();
    // One work-group per CU (a wave per SIMD): where LDS would hold two (MHA
    // at the 2-deep ring), the second measures slower (c2 191.8 against
    // 187.7 us with one).
    const int waves = stream_waves<grouped_partition_kernel<T, D, G, NBUF>>(
        kWave * kGroupWaves, 1, kStreamWavesMax, kGroupWaves, 1);
    const int th = team_heads(s.num_kv_heads, kGroupWaves, G);
    const int nshares = waves / th > 0 ? waves / th : 1;
    const int groups = (nshares * th + kGroupWaves - 1) / kGroupWaves;
    hipLaunchKernelGGL(kernel, dim3(groups), dim3(kWave * kGroupWaves), 0, stream, acc, ml, prefix,
                       static_cast<const T *>(a.q), static_cast<const T *>(a.k_cache),
                       static_cast<const T *>(a.v_cache), a.block_tables, a.context_lens,
                       scale_log2, s.num_seqs, s.num_kv_heads, s.max_blocks_per_seq, nshares, th,
                       s.window);
    pa_status st = hip_status(hipGetLastError(), why, "partition launch");
    if (st != PA_OK) return st;
    return hip_status(enqueue_stream_reduce<T, D>(static_cast<T *>(a.out), acc, ml, prefix,
                                                  a.context_lens, s.num_seqs, s.num_q_heads,
                                                  s.num_kv_heads, G, kBS, nshares, th, stream,
                                                  1, s.window, a.lse),
                      why, "reduce launch");
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

}  // namespace

pa_status launch_grouped_decode(const DecodeShape &s, const DecodeArgs &a, const DecodePlan &p,
                                void *stream_arg, std::string *why) {
    const hipStream_t stream = static_cast<hipStream_t>(stream_arg);
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
