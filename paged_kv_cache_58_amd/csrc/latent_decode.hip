// Latent-mode (MLA-style) paged decode attention for gfx950, on MFMA.
//
// What is computed: every query head attends over one shared cached latent
// per token, 576 values (512 latent + 64 RoPE dims, the MLA bullet of the
// CS336 lecture 10 notes, "核心概念与定义"); the whole row is the key and its
// first 512 values are the value:
//   s_t = scale * q_h . c_t,   O_h = sum_t softmax(s)_t c_t[0:512]
// with the latent reached block by block through the block table (the page
// table of "Cache KV, attention et optimisation de l'inference").  As on the
// grouped path the softmax runs online with a running max and sum, the
// block order is cut into stream-K shares, and a log-sum-exp reduce merges
// the partials (FlashDecoding).
//
// Here all query heads share one K/V row, so each block is a dense
// contraction and runs on the matrix cores (v_mfma_f32_32x32x16_bf16).
//  * A work-group has four waves, one per SIMD, and covers every query head
//    (padded to 32, 64 or 128).  Each sequence is cut into parts of
//    near-equal size, one work-group per part, so a work-group streams one
//    stretch of one sequence (split-KV partitions; the log-sum-exp reduce
//    merges a sequence's parts).  The latent is streamed in units of 32
//    tokens (half a 64-token block, 36 KB) by global_load_lds_dwordx4 into
//    an LDS ring of four main regions (dims 0..511) and three RoPE regions
//    (dims 512..575): while unit u is being consumed, units u + 2 and u + 3
//    are in flight.
//  * Scores: wave w computes S^T[token, head] = L[token, :] . Q^T for heads
//    32w..32w+31; the latent rows are the A operand (16 contiguous bytes per
//    lane) and q sits in registers as the B operand for the whole segment.
//    A lane's S^T accumulator holds 16 of the unit's 32 tokens for one head
//    (the other 16 sit in lane ^ 32, one v_permlane32_swap away), so the
//    running max is an in-lane max and one lane exchange, and the
//    probabilities, rounded to bf16, come out in the B-operand layout of
//    O^T[dim, head] += V^T[dim, token] . P^T[token, head].  They go to LDS
//    (8 KB per unit, two buffers), with the rescale factors of heads whose
//    running max moved.
//  * Values: wave w accumulates O^T for dims 512 w / NW .. + 512 / NW - 1 of
//    every head, as (16 / NW) x NW register-blocked 32 x 32 tiles held in the
//    accumulation registers (256 per lane).  Each V^T fragment (transposed
//    reads, ds_read_b64_tr_b16) feeds NW products and each P^T fragment
//    16 / NW, so the LDS traffic per product stays well under what the
//    matrix core consumes (a wave reading every dim itself would issue four
//    times the transposed reads, which run at about a quarter of the rate of
//    16-byte reads).
//  * Software pipeline, one barrier per unit: the score products of unit
//    u + 1 run as one chain with the unit's DMA rows and bookkeeping between
//    them, then the value products of unit u one at a time, each after an
//    even share of the softmax of unit u + 1.  A wave overlaps its own
//    matrix-core and vector work only when other instructions follow a
//    product: a product issued right after another stalls the wave until the
//    first one leaves the matrix core.
//  * LDS layout of a unit: the first 64 16-byte chunks of every row (dims
//    0..511) in a 32 KB region of 1 KB rows, the 8 RoPE chunks in a 4 KB
//    region of 128-byte rows.  Chunk c of main row t sits at c ^ swm(t),
//    RoPE chunk c of row t at c ^ swr(t); both keep every phase of the
//    row-wise and transposed reads on distinct banks.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "device_common.h"
#include "hip_util.h"
#include "launch.h"

namespace pa {
namespace {

constexpr int kLBS = 64;                      // tokens per cache block
constexpr int kDK = 576;                      // latent width (key)
constexpr int kDV = 512;                      // value width (leading part of the row)
constexpr int kRowB = kDK * 2;                // bytes per token row in HBM
constexpr int kMainChunks = kDV * 2 / 16;     // 64 chunks: dims 0..511
constexpr int kMainRowB = kMainChunks * 16;   // 1 KB main row in LDS
constexpr int kRopeRowB = kRowB - kMainRowB;  // 128-byte RoPE row in LDS
constexpr int kBlockB = kLBS * kRowB;         // 72 KB per block in HBM
constexpr int kUnitTok = 32;                  // tokens per ring slot (half a block)
constexpr int kUnitMainB = kUnitTok * kMainRowB;  // 32 KB main region
constexpr int kUnitB = kUnitTok * kRowB;      // 36 KB per slot
constexpr int kSlots = 4;                     // ring slots (a power of two keeps the
                                              // slot arithmetic in shifts and immediates)
constexpr int kDmaPerUnit = kUnitB / 1024;    // 36: 32 main rows + 4 groups of 8 RoPE rows
constexpr int kHeads = 32;                    // heads per score tile
constexpr int kLatentNW = 4;                  // waves of a partition work-group, one per SIMD
constexpr int kKSteps = kDK / 16;             // 36 k-steps of q . L
constexpr int kMainKSteps = kDV / 16;         // the first 32 of them read the main region
constexpr int kDimTiles = kDV / 32;           // 16 tiles of the output
constexpr float kLSlack = 8.0f;               // lazy-rescale threshold, log2 units

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Main-region swizzle: over any 16 consecutive rows swm takes 16 distinct
// values (a 16-lane phase of a row-wise read of one chunk column hits 16
// different bank groups); over 4 rows 4a..4a+3 its bits 2..3 take 4
// distinct values and bits 0..1 stay fixed, so a 32-lane phase of the
// transposed reads (4 rows x chunks 4m..4m+3) hits 16 different groups.
__host__ __device__ constexpr int swm(int t) { return ((t & 3) << 2) | ((t >> 2) & 3); }
// RoPE-region swizzle: 128-byte rows put even and odd rows in opposite
// halves of the banks; (t >> 1) & 7 spreads 8 same-parity rows over the half.
__host__ __device__ constexpr int swr(int t) { return (t >> 1) & 7; }

__device__ __forceinline__ s16x4_t ds_read_tr(uint32_t byte_addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t *)(uintptr_t)byte_addr);
}

__device__ __forceinline__ bf16x8_t ds_read_b128(uint32_t byte_addr) {
    return __builtin_bit_cast(
        bf16x8_t, *(const __attribute__((address_space(3))) u32x4_t *)(uintptr_t)byte_addr);
}

// The products are issued from inline assembly so that the 256 output
// accumulators can be pinned to the accumulation registers ("a") while the
// scores stay in VGPRs ("v"); the compiler would otherwise give every MFMA
// the same register file.  Hazards the compiler cannot see are handled here
// (and the compiled code is checked for them by the test suite):
//  * operands: the A and B operands come straight from LDS reads or from q,
//    which only vector loads write; a score chain starts from the constant 0
//    as C, and the rare rescale of the accumulators ends with s_nop 2;
//  * a chain of products into one accumulator needs no wait states between
//    links (the matrix core forwards its own result as C);
//  * results: before anything but the next product reads or writes an
//    accumulator, a fence waits 32 cycles, more than the pass count of one
//    product plus its write-back.
// The "memory" clobber pins each statement between the LDS reads around it,
// which keeps the read-ahead distance written in the source.
__device__ __forceinline__ void mfma_v0(f32x16_t &c, bf16x8_t a, bf16x8_t b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b) : "memory");
}
__device__ __forceinline__ void mfma_v(f32x16_t &c, bf16x8_t a, bf16x8_t b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b) : "memory");
}
// The last product of a score chain, then the fence.
__device__ __forceinline__ void mfma_v_fence(f32x16_t &c, bf16x8_t a, bf16x8_t b) {
    asm volatile(
        "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
        "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
        : "+v"(c) : "v"(a), "v"(b) : "memory");
}
__device__ __forceinline__ void mfma_a(f32x16_t &c, bf16x8_t a, bf16x8_t b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b) : "memory");
}
// A tile of the output accumulators read into VGPRs element by element by
// inline asm that takes each value from the accumulation registers: code
// after the unit loop reads the tiles only through this, so the compiler
// keeps them where the loop left them instead of copying all 256 into VGPRs
// at the loop's exit (which spills).  Only after acc_fence.
__device__ __forceinline__ f32x16_t acc_tile(const f32x16_t &a) {
    f32x16_t x;
#pragma unroll
    for (int e = 0; e < 16; ++e) asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(x[e]) : "a"(a[e]));
    return x;
}
// Fence over the output tiles (before the rescale and the final store).
template <int N>
__device__ __forceinline__ void acc_fence(f32x16_t (&acc)[N]) {
    static_assert(N == 4 || N == 8 || N == 16, "4, 8 or 16 output tiles");
    if constexpr (N == 16) {
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]), "+a"(acc[4]),
                       "+a"(acc[5]), "+a"(acc[6]), "+a"(acc[7]), "+a"(acc[8]), "+a"(acc[9]),
                       "+a"(acc[10]), "+a"(acc[11]), "+a"(acc[12]), "+a"(acc[13]), "+a"(acc[14]),
                       "+a"(acc[15])
                     :: "memory");
    } else if constexpr (N == 8) {
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]), "+a"(acc[4]),
                       "+a"(acc[5]), "+a"(acc[6]), "+a"(acc[7])
                     :: "memory");
    } else {
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3])
                     :: "memory");
    }
}

template <int HT>
__global__ __launch_bounds__(kLatentNW *kWave) __attribute__((amdgpu_waves_per_eu(1, 1)))
void latent_partition_kernel(uint16_t *__restrict__ out, float *__restrict__ ws_acc,
                             float2 *__restrict__ ws_ml,
                             int32_t *__restrict__ ws_prefix, const uint16_t *__restrict__ q,
                             const uint16_t *__restrict__ latent,
                             const int32_t *__restrict__ block_tables,
                             const int32_t *__restrict__ context_lens, float scale_log2,
                             int num_seqs, int num_heads, int max_blocks) {
    // HT head tiles (of 32) in the work-group; its four waves (one per SIMD)
    // split each tile's score contraction KS ways: wave w scores head tile
    // w % HT over k-split w / HT, and accumulates every head tile's outputs
    // for its DT output dim tiles.
    constexpr int NW = kLatentNW;
    constexpr int KS = NW / HT;
    constexpr int DT = kDimTiles / NW;  // output dim tiles per wave
    static_assert(NW % HT == 0, "head tiles divide the waves");
    constexpr int kMainPer = kMainKSteps / KS;              // main k-steps of a split (multiple of 8)
    constexpr int kRopePer = (kKSteps - kMainKSteps) / KS;  // RoPE k-steps of a split
    constexpr int kKW = kMainPer + kRopePer;                // k-steps of a split
    static_assert(kMainPer % 8 == 0 && kRopePer * KS == kKSteps - kMainKSteps, "k-step split");
    constexpr int NA = DT * HT;         // output tiles per wave
    constexpr int kVR = 3;              // V^T operands read ahead
    constexpr int kRA = 3;              // score A operands read ahead
    constexpr int kNV = 2 * DT;         // value steps (of HT products) per unit
    constexpr int kVP = kNV * HT;       // value products per unit

    // Ring: main regions (dims 0..511 of 32 rows) for units u % 4, RoPE
    // regions (dims 512..575) for units u % 3: while step u runs, unit u's
    // main region (values), unit u + 1's main and RoPE regions (scores) and
    // units u + 2 and u + 3 (streaming in) are live, and unit u's RoPE rows
    // are not needed any more.  That leaves room for two probability buffers.
    __shared__ __attribute__((aligned(16))) uint4 s_main[kSlots][kUnitMainB / 16];
    __shared__ __attribute__((aligned(16))) uint4 s_rope[3][(kUnitB - kUnitMainB) / 16];
    __shared__ __attribute__((aligned(16))) u32x4_t s_p[2][HT][2][kWave];  // P^T fragments of unit u in [u & 1]
    __shared__ float s_alpha[2][HT * kHeads];  // rescale factor of each head, unit u in [u & 1]
    __shared__ __attribute__((aligned(4))) uint8_t s_flag[2][4];  // byte ht: head tile ht rescaled in unit u
    __shared__ __attribute__((aligned(16))) int32_t s_ids[2][kWave];
    __shared__ __attribute__((aligned(16))) uint4 s_sink[kWave];  // target of padding loads
    __shared__ float s_l[HT * kHeads];  // each head's running sum, for the partial
    // partial scores of the waves with k-split > 0, read by their tile's first wave
    __shared__ __attribute__((aligned(16))) u32x4_t s_spart[KS > 1 ? (KS - 1) * HT * 4 * kWave : 1];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    __builtin_assume(wave >= 0 && wave < NW);
    const int l31 = lane & 31;    // MFMA row (A) / column (B, C) of this lane
    const int hk = lane >> 5;     // which 8 of a 16-wide k-step this lane holds
    const int ht_w = wave % HT;            // this wave's head tile in the scores
    const int ksplit = wave / HT;          // and its share of their contraction
    const int head = ht_w * kHeads + l31;  // this lane's head in the scores
    const bool head_ok = head < num_heads;

    // ---- this work-group's part: a sequence-aligned split ------------------
    // Sequence b (nu_b = ceil(ctx_b / 32) units of 32 tokens) is cut into
    // k_b = ceil(nu_b / P) parts of near-equal size, P the smallest part size
    // for which every part gets a work-group (sum of k_b <= gridDim.x; the
    // host launches at least one work-group per sequence).  Work-group j
    // takes part j - K_b of the sequence b with K_b <= j < K_b + k_b, K_b the
    // number of parts of the sequences before b, so each work-group streams
    // one stretch of one sequence: a change of segment inside a work-group
    // (partial store, q reload, refilling the ring) costs about as much as a
    // dozen units, and units rather than 64-token blocks keep the parts
    // within one unit of each other.  The work-group of part index j (below)
    // stores its partial in slot j, and the one of index 0 stores K_b
    // (num_seqs + 1 entries) for the reduce; a sequence of one part writes
    // its output itself.  The unit counts of
    // the first 256 sequences stay in registers for the search.
    auto seq_units = [&](int bb) {
        return bb < num_seqs ? (context_lens[bb] + kUnitTok - 1) / kUnitTok : 0;
    };
    constexpr int kCached = 4;
    int nu_c[kCached];
    {
        // every load first (clamped in bounds, num_seqs >= 1), so that they
        // share one memory round trip, then the counts
        int ctx_c[kCached];
#pragma unroll
        for (int r = 0; r < kCached; ++r) ctx_c[r] = context_lens[min(r * kWave + lane, num_seqs - 1)];
#pragma unroll
        for (int r = 0; r < kCached; ++r)
            nu_c[r] = r * kWave + lane < num_seqs ? (ctx_c[r] + kUnitTok - 1) / kUnitTok : 0;
    }
    // f(first sequence of the chunk, this lane's unit count) for every chunk of 64 sequences
    auto each_chunk = [&](auto &&f) {
#pragma unroll
        for (int r = 0; r < kCached; ++r)
            if (r * kWave < num_seqs) f(r * kWave, nu_c[r]);
        for (int base = kCached * kWave; base < num_seqs; base += kWave) f(base, seq_units(base + lane));
    };
    auto wave_sum = [&](int v) { return __builtin_amdgcn_readlane(wave_incl_scan(v, lane), kWave - 1); };
    int total = 0, most = 0;  // units of all sequences; of the longest
    each_chunk([&](int, int nu) {
        total += wave_sum(nu);
        int m = nu;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) m = max(m, __shfl_xor(m, d));
        most = max(most, m);
    });
    if (total == 0) return;  // every context empty: the reduce writes zeros
    const int grid = static_cast<int>(gridDim.x);
    // Part index j runs over the work-groups so that the parts of a sequence
    // sit on one XCD (work-groups are dealt to the 8 XCDs in turn, so j takes
    // every 8th one; they then share that XCD's L2 for q and the block table).
    const int j = grid % 8 == 0 ? static_cast<int>(blockIdx.x % 8u) * (grid / 8) +
                                      static_cast<int>(blockIdx.x / 8u)
                                : static_cast<int>(blockIdx.x);
    auto parts = [&](int P) {  // sum over the sequences of ceil(nu_b / P)
        int k_all = 0;
        each_chunk([&](int, int nu) { k_all += wave_sum((nu + P - 1) / P); });
        return k_all;
    };
    // parts(P) only falls as P grows; parts(most) <= num_seqs <= grid, and
    // parts(P) <= total / P + num_seqs, so P = ceil(total / (grid - num_seqs))
    // fits too when grid > num_seqs
    int lo = max(1, (total + grid - 1) / grid), hi = most;
    if (grid > num_seqs) hi = min(hi, (total + grid - num_seqs - 1) / (grid - num_seqs));
    hi = max(hi, lo);
    while (lo < hi) {
        const int mid = (lo + hi) / 2;
        if (parts(mid) <= grid) hi = mid;
        else lo = mid + 1;
    }
    const int P = lo;
    int b = -1, part = 0, k_b = 1, nu_b = 0, carry = 0;
    each_chunk([&](int base, int nu) {
        const int bb = base + lane;
        const int k = (nu + P - 1) / P;
        const int incl = wave_incl_scan(k, lane);
        if (j == 0 && wave == 0 && bb < num_seqs) ws_prefix[bb] = carry + incl - k;
        const uint64_t hit =
            __builtin_amdgcn_ballot_w64(bb < num_seqs && carry + incl > j);
        if (b < 0 && hit != 0) {
            const int f = __builtin_ctzll(hit);
            b = base + f;
            k_b = __builtin_amdgcn_readlane(k, f);
            nu_b = __builtin_amdgcn_readlane(nu, f);
            part = j - (carry + __builtin_amdgcn_readlane(incl, f) - k_b);
        }
        carry += __builtin_amdgcn_readlane(incl, kWave - 1);
    });
    if (j == 0 && tid == 0) ws_prefix[num_seqs] = carry;
    if (b < 0) return;  // a work-group past the last part (uniform)
    // this part: units [seg_u0, seg_u1) of sequence b; unit u of the segment
    // is half (h0 + u) & 1 of block blk_start + ((h0 + u) >> 1)
    const int seg_u0 = part * nu_b / k_b;
    const int seg_u1 = (part + 1) * nu_b / k_b;
    const int blk_start = seg_u0 >> 1;
    const int h0 = seg_u0 & 1;
    const int seg_blocks = ((seg_u1 - 1) >> 1) - blk_start + 1;

    // the main regions start zeroed (rows past a context are never fetched)
    for (int i = tid; i < kSlots * kUnitMainB / 16; i += NW * kWave)
        (&s_main[0][0])[i] = make_uint4(0u, 0u, 0u, 0u);
    const uint32_t main_lds = lds_offset(s_main);
    const uint32_t rope_lds = lds_offset(s_rope);
    const uint32_t ids_lds[2] = {lds_offset(&s_ids[0][0]), lds_offset(&s_ids[1][0])};
    auto main_slot = [&](int u) { return main_lds + (u % kSlots) * kUnitMainB; };
    auto rope_slot = [&](int u) { return rope_lds + (u % 3) * (kUnitB - kUnitMainB); };

    // ---- per-lane LDS addresses (bytes, relative to a region) -------------
    // S^T A operand: unit row l31, chunk 2 ks + hk.  swm of that row is
    // swm(lane & 15) and the xor touches the low 4 chunk bits only, so the
    // byte offset in a main row is 256 (ks >> 3) + (32 (ks & 7) ^ qx) with
    // qx = 16 (hk ^ swm).  RoPE rows likewise: offset 32 (ks - 32) ^ rx.
    const uint32_t qrow = l31 * kMainRowB;
    const uint32_t qx = 16u * static_cast<uint32_t>(hk ^ swm(lane & 15));
    const uint32_t rrow = l31 * kRopeRowB;
    const uint32_t rx = 16u * static_cast<uint32_t>(hk ^ swr(l31));
    // V^T A operand by transposed reads.  16-lane group g = lane >> 4 reads
    // rows tb + (i >> 2), i = lane & 15, dims 32 dt + 16 (g & 1) + 4 (i & 3),
    // with tb = 16 s + 8 qq + 4 hk; lane i then receives the 4 tokens
    // tb .. tb + 3 of dim 32 dt + (lane & 31).  The row's swm depends on
    // (qq, hk, i >> 2) only; the chunk is 16 (dt >> 2) + 4 (dt & 3) + c0 with
    // c0 = 2 (g & 1) + ((i & 3) >> 1) < 4, so the offset in a row is
    // 256 (dt >> 2) + (64 (dt & 3) ^ vy[qq]) with vy = 16 (c0 ^ swm(row)).
    // With DT = 4 dim tiles per wave, dt = dg & 3 and dg >> 2 = wave, so the
    // lane's part of the address of (qq, dt) is one of 8 values, formed once:
    // vofs[qq][dt] = row offset + ((64 dt) ^ vy[qq]); a read then adds the
    // unit's slot and 256 wave (uniform) and takes 16 s rows as an immediate.
    static_assert(kDimTiles / kLatentNW == 4, "four dim tiles per wave");
    uint32_t vofs[2][4];
    {
        const int i = lane & 15;
        const int c0 = 2 * ((lane >> 4) & 1) + ((i & 3) >> 1);
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
            const int trow = 8 * qq + 4 * hk + (i >> 2);
            const uint32_t vrow = trow * kMainRowB + 8 * (i & 1);
            const uint32_t vy = 16u * static_cast<uint32_t>(c0 ^ swm(trow));
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) vofs[qq][dt] = vrow + ((64u * dt) ^ vy);
        }
    }
    // P^T fragment (buffer, head tile ht, k-step s) of this lane: 16 bytes
    const uint32_t p_lds = lds_offset(&s_p[0][0][0][0]) + 16 * lane;
    constexpr uint32_t kPBuf = HT * 2 * kWave * 16;

    {
        // ======== the segment: sequence b, units [seg_u0, seg_u1) ========
        const int nblk = seg_blocks;
        const int ctx = context_lens[b];
        const int32_t *bt_row = block_tables + static_cast<int64_t>(b) * max_blocks;
        auto fetch_ids = [&](int m) {
            const int en = min(blk_start + kWave * m + lane, max_blocks - 1);
            dma4(bt_row, static_cast<uint32_t>(en) * 4u, ids_lds[m & 1]);
        };
        if (wave == 0) {
            fetch_ids(0);
            if (nblk > kWave) fetch_ids(1);
        }
        // q^T B-operand fragments of this lane's head: dims 16 kg + 8 hk .. + 7
        // for the k-steps kg of this wave's split (zero for padding heads past
        // num_heads): local step k < kMainPer is main step ksplit kMainPer + k,
        // the others RoPE steps 32 + ksplit kRopePer + (k - kMainPer).
        bf16x8_t qf[kKW];
        if (head_ok) {
            const uint4 *qr = reinterpret_cast<const uint4 *>(
                q + (static_cast<int64_t>(b) * num_heads + head) * kDK + 8 * hk);
#pragma unroll
            for (int k = 0; k < kKW; ++k) {
                const int kg = k < kMainPer ? ksplit * kMainPer + k
                                            : kMainKSteps + ksplit * kRopePer + (k - kMainPer);
                qf[k] = __builtin_bit_cast(bf16x8_t, qr[2 * kg]);
            }
#pragma unroll
            for (int k = 0; k < kKW; ++k) settle(qf[k]);
        } else {
#pragma unroll
            for (int k = 0; k < kKW; ++k) qf[k] = bf16x8_t{};
        }
        drain_vmem();
        __syncthreads();  // ids landed for every wave; the previous segment is done
        // The scale goes into each exponential (one fused multiply-add per
        // score) and the running max is taken over the raw q . c, which needs
        // a positive scale: a negative one negates q instead, and zero becomes
        // the smallest normal float (every weight then rounds to 1, as at 0).
        if (scale_log2 < 0.f) {  // (uniform)
#pragma unroll
            for (int k = 0; k < kKW; ++k)
                qf[k] = __builtin_bit_cast(bf16x8_t, __builtin_bit_cast(u32x4_t, qf[k]) ^ 0x80008000u);
        }
        const float sc = fmaxf(fabsf(scale_log2), 1.17549435e-38f);

        float m_run = kNegInf;  // running max of this lane's head (log2 units)
        float l_run = 0.f;      // this lane's share of its running sum
        // O^T tile (dt, ht) = acc[dt * HT + ht]: dims 32 (DT wave + dt) +
        // 8 (j >> 2) + 4 hk + (j & 3) of head 32 ht + l31
        f32x16_t acc[NA];
#pragma unroll
        for (int t = 0; t < NA; ++t) acc[t] = f32x16_t{};

        // Units of this segment: 32-token halves of blocks, each holding at
        // least one context token (unit u is half (h0 + u) & 1 of block
        // blk_start + ((h0 + u) >> 1)).  Tokens at or past seg_lim belong to
        // no unit of the segment.
        const int seg_tok0 = seg_u0 * kUnitTok;
        const int seg_lim = min(ctx, seg_u1 * kUnitTok);
        const int nunits = seg_u1 - seg_u0;

        // DMA of unit u: this wave's rows i = wave + NW k, k < kPer, of the
        // unit's 36 (32 main rows, 4 groups of 8 RoPE rows).  A main row at or
        // past the context goes into s_sink instead of the slot: only the
        // destination is selected (not branched, so every wave has exactly
        // kPer loads per unit in flight and the vmcnt waits below stay exact),
        // and the source row still lies inside the unit's block.  The slot
        // keeps what it held, which is finite: the main regions start zeroed
        // and later hold only fetched rows of the context.  The probabilities
        // of those tokens are exactly 0, so they contribute exactly 0 (a NaN
        // there would not).  RoPE rows only feed scores, which are masked.
        // A unit past the segment's last (not live) loads the same rows of the
        // pool's first block into s_sink, so every step has kPer loads.
        // Since wave < NW and NW k is a multiple of NW, swm(i) = (wave << 2) ^
        // swm(NW k): one lane term serves every row of the wave, and the
        // wave's row offset goes into the unit's source and destination.
        constexpr int kPer = (kDmaPerUnit + NW - 1) / NW;
        // rows issued beside the score chain, one before every third product
        // from the third; the rest (with a short chain) right after it
        constexpr int kChainRows = kKW / 3 < kPer ? kKW / 3 : kPer;
        const uint32_t ln_w = static_cast<uint32_t>(lane) ^ (static_cast<uint32_t>(wave) << 2);
        struct UnitDma {
            const char *src;  // the unit's first row + wave rows
            uint32_t dst;     // the unit's main slot + wave rows
            int nfetch;       // rows of the unit in the context, minus wave (uniform)
            bool live;
        };
        const char *pool = reinterpret_cast<const char *>(latent);
        auto unit_dma = [&](int u, bool live, int pb) {
            UnitDma d;
            // (operands are selected rather than results, which keeps this
            // free of branches)
            const int pbl = live ? pb : 0;
            const int half = live ? ((h0 + u) & 1) : 0;
            d.src = pool + static_cast<int64_t>(pbl) * kBlockB + half * (kUnitTok * kRowB) + wave * kRowB;
            d.dst = main_slot(u) + wave * kMainRowB;
            const int rows = min(kUnitTok, ctx - (seg_tok0 + u * kUnitTok));
            d.nfetch = (live ? rows : 0) - wave;
            d.live = live;
            return d;
        };
        auto issue_row = [&](int u, const UnitDma &d, int k) {
            if (NW * k >= kDmaPerUnit) return;  // (wave < NW: then i >= 36 too)
            if (NW * k < kUnitTok) {            // main region: row i, lane = swizzled chunk
                const uint32_t off =
                    ((ln_w ^ static_cast<uint32_t>(swm(NW * k))) << 4) + NW * k * kRowB;
                dma16(d.src, off, NW * k < d.nfetch ? d.dst + NW * k * kMainRowB : lds_offset(s_sink));
            } else {                            // RoPE region: 8 rows x 8 chunks
                const int r = wave + NW * k - kUnitTok;
                const int t = 8 * r + (lane >> 3);
                const uint32_t off = (t - wave) * kRowB + (kMainChunks + ((lane & 7) ^ swr(t))) * 16;
                dma16(d.src, off, d.live ? rope_slot(u) + r * 1024 : lds_offset(s_sink));
            }
        };
        // Block ids come in chunks of 64 through s_ids; wave 0 fetches chunk
        // c + 1 when the first unit of chunk c is issued.
        auto refill_ids = [&](int u) {
            // unit u is the first half of block n = (h0 + u) / 2, n a positive
            // multiple of 64 with a further chunk after this one
            const int hu = h0 + u;
            if (wave == 0 && (hu & (2 * kWave - 1)) == 0 && hu > 0 && (hu >> 1) + kWave < nblk)
                fetch_ids((hu >> 7) + 1);
        };
        auto unit_id = [&](int u) {
            const int n = (h0 + u) >> 1;  // block of unit u, from blk_start
            return s_ids[(n >> 6) & 1][n & (kWave - 1)];
        };

        // A operand of score k-step ks of unit u (the lane's 12 row offsets
        // stay live, as do the 8 of the V^T reads below)
        // (local step k of this wave's split; its main steps start at a
        // multiple of 8, so their chunk term stays a constant)
        // The 8 main and kRopePer RoPE lane addresses of a unit are formed once
        // (qk_bases); each read then adds only an immediate offset.
        const uint32_t qmain = static_cast<uint32_t>(ksplit * kMainPer / 8) * 256u;
        constexpr int kQB = kMainPer < 8 ? kMainPer : 8;
        uint32_t qb_main[kQB], qb_rope[kRopePer];
        auto qk_bases = [&](int u) {
#pragma unroll
            for (int j = 0; j < kQB; ++j) qb_main[j] = (main_slot(u) + qmain + qrow) + ((32u * j) ^ qx);
#pragma unroll
            for (int j = 0; j < kRopePer; ++j)
                qb_rope[j] = (rope_slot(u) + rrow) +
                             ((32u * static_cast<uint32_t>(ksplit * kRopePer + j)) ^ rx);
        };
        auto qk_read = [&](int k) {
            return ds_read_b128(k < kMainPer ? qb_main[k & 7] + 256 * (k >> 3) : qb_rope[k - kMainPer]);
        };
        // V^T operand (k-step s, this wave's dim tile dt, half qq) of unit u
        uint32_t vbase[2][4];  // this unit's V^T read bases (set by value_prefetch)
        auto pv_read = [&](int u, int s, int dt, int qq) {
            (void)u;
            return ds_read_tr(vbase[qq][dt] + (16 * s) * kMainRowB);
        };

        // The score chain over k-steps [k0, k1) into s, of the unit whose
        // addresses score_prefetch formed (A operands read kRA steps ahead);
        // before each product f(ks) runs, pinned there by the products'
        // memory clobber.
        bf16x8_t xa[kRA];
        auto score_steps = [&](f32x16_t &s, int k0, int k1, auto &&f) {
#pragma unroll
            for (int ks = k0; ks < k1; ++ks) {
                f(ks);
                const int r = ks % kRA;
                if (ks == 0) mfma_v0(s, xa[r], qf[ks]);
                else if (ks + 1 < kKW) mfma_v(s, xa[r], qf[ks]);
                else mfma_v_fence(s, xa[r], qf[ks]);
                if (ks + kRA < kKW) xa[r] = qk_read(ks + kRA);
            }
        };
        auto score_prefetch = [&](int u) {
            qk_bases(u);
#pragma unroll
            for (int ks = 0; ks < kRA; ++ks) xa[ks] = qk_read(ks);
        };

        // Softmax of unit u from its raw scores s, in kSub pieces so that it
        // spreads evenly between the value products: the running max and sum
        // of this lane's head and the P^T fragments of this wave's head tile
        // into buffer u & 1, with the rescale factor when the max moved.
        // Register j of s: token 8 (j >> 2) + 4 hk + (j & 3) of the unit;
        // tokens at or past seg_lim are masked, so the score chain that runs
        // past a segment's last unit changes nothing here.  Pieces: 0..3
        // empty (they keep the pieces' spacing among the value products); 4
        // masks (only a unit that reaches the segment's limit, its last or one
        // past it, holds tokens to mask); 5..8 the max of the raw scores over
        // registers 4(k - 5) .. + 3; 9 the other 16 tokens of the head, in
        // lane ^ 32; 10 the scaled block max, the running max and the rescale
        // decision; 11..26 one probability 2^(sc s - m) each (register k - 11),
        // the second of a pair packing the pair, adding both rounded values to
        // the running sum and, every fourth pair, writing a P^T fragment.
        constexpr int kSub = 27;
        bool moved = false;
        float bmax = kNegInf;
        float pe = 0.f;  // the first probability of a pair
        uint32_t w4[4];
        auto softmax_sub = [&](f32x16_t &s, int u, int k) {
            const int tok0 = seg_tok0 + u * kUnitTok;
            if (k < 4) {
                // (nothing: the scale is applied inside the exponentials)
            } else if (k == 4) {
                if (__builtin_expect(tok0 + kUnitTok > seg_lim, 0)) {  // (uniform)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int tk = tok0 + 8 * (j >> 2) + 4 * hk + (j & 3);
                        s[j] = tk < seg_lim ? s[j] : kNegInf;
                    }
                }
            } else if (k < 9) {
                const int b = k - 5;
                float lmax = b == 0 ? kNegInf : bmax;
#pragma unroll
                for (int j = 4 * b; j < 4 * b + 4; ++j) lmax = fmaxf(lmax, s[j]);
                bmax = lmax;
            } else if (k == 9) {
                const auto r = __builtin_amdgcn_permlane32_swap(as_u(bmax), as_u(bmax), false, false);
                bmax = fmaxf(as_f(r[0]), as_f(r[1]));
            } else if (k == 10) {
                const float bs = bmax * sc;  // the block max, scaled
                moved = __builtin_amdgcn_ballot_w64(bs > m_run + kLSlack) != 0;
                if (moved) {
                    const float m_new = fmaxf(m_run, bs);
                    const float alpha = exp2_fast(m_run - m_new);
                    l_run *= alpha;
                    m_run = m_new;
                    if (hk == 0) s_alpha[u & 1][head] = alpha;
                }
                if (lane == 0) s_flag[u & 1][ht_w] = (moved && u > 0) ? 1 : 0;  // u = 0: nothing to rescale
            } else {
                const int jj = k - 11, v = jj >> 1, sv = v >> 2, e = v & 3;
                if ((jj & 1) == 0) {
                    pe = exp2_fast(fmaf(s[jj], sc, -m_run));
                } else {
                    w4[e] = pack_bf16(pe, exp2_fast(fmaf(s[jj], sc, -m_run)));
                    l_run = dot2_bf16(w4[e], 0x3F803F80u, l_run);  // + both rounded values (bf16 1, 1)
                    if (e == 3)
                        *(__attribute__((address_space(3))) u32x4_t *)(uintptr_t)(
                            p_lds + (u & 1) * kPBuf + (ht_w * 2 + sv) * kWave * 16) =
                            u32x4_t{w4[0], w4[1], w4[2], w4[3]};
                }
            }
        };

        // O^T += V^T P^T for this wave's dims, every head, unit u: 2 DT value
        // steps i (k-step i / DT, dim tile i % DT) of HT products each, issued
        // one at a time.  value_begin(u, i) takes step i's V^T operand (read
        // kVR steps ahead into slot i % kVR) and issues the reads of step
        // i + kVR; value_product(i, ht) is the product of head tile ht.  The
        // P^T fragments of k-step 0 are read during the score chain (p_read),
        // each of k-step 1 right after its k-step 0 fragment's last product.
        s16x4_t vlo[kVR], vhi[kVR];
        bf16x8_t pb[HT];
        bf16x8_t va;
        auto value_prefetch = [&](int u) {
#pragma unroll
            for (int qq = 0; qq < 2; ++qq)
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) vbase[qq][dt] = main_slot(u) + 256 * wave + vofs[qq][dt];
#pragma unroll
            for (int i = 0; i < kVR; ++i) {
                vlo[i] = pv_read(u, i / DT, i % DT, 0);
                vhi[i] = pv_read(u, i / DT, i % DT, 1);
            }
        };
        auto p_read = [&](int u, int s, int ht) {
            pb[ht] = ds_read_b128(p_lds + (u & 1) * kPBuf + (ht * 2 + s) * kWave * 16);
        };
        auto value_begin = [&](int u, int i) {
            const int r = i % kVR;
            va = __builtin_bit_cast(bf16x8_t,
                                    __builtin_shufflevector(vlo[r], vhi[r], 0, 1, 2, 3, 4, 5, 6, 7));
            if (i + kVR < kNV) {
                vlo[r] = pv_read(u, (i + kVR) / DT, (i + kVR) % DT, 0);
                vhi[r] = pv_read(u, (i + kVR) / DT, (i + kVR) % DT, 1);
            }
        };
        auto value_product = [&](int u, int i, int ht) {
            mfma_a(acc[(i % DT) * HT + ht], va, pb[ht]);
            if (i == DT - 1) p_read(u, 1, ht);
        };
        // rescale of the accumulators for unit u when a running max moved (rare);
        // tile by tile through VGPRs so that at most one tile is out of the
        // accumulation registers at a time
        // The flags of unit u (byte ht for head tile ht) are read right after
        // the step's barrier and applied after the score chain, so that their
        // LDS round trip is not waited for.
        auto read_flags = [&](int u) {
            return *(const __attribute__((address_space(3))) uint32_t *)(uintptr_t)lds_offset(
                &s_flag[u & 1][0]);
        };
        auto rescale = [&](int u, uint32_t flw) {
            uint32_t any = flw;
            if constexpr (HT < 4) any &= (1u << (8 * HT)) - 1u;  // (bytes past HT are never written)
            if (__builtin_expect(any != 0, 0)) {
                float alpha[HT];
#pragma unroll
                for (int ht = 0; ht < HT; ++ht)
                    alpha[ht] = ((flw >> (8 * ht)) & 0xFFu) != 0 ? s_alpha[u & 1][ht * kHeads + l31] : 1.0f;
                acc_fence(acc);
#pragma unroll
                for (int t = 0; t < NA; ++t) {
                    f32x16_t xv = acc[t];
                    asm volatile("" : "+v"(xv));
                    xv *= alpha[t % HT];
                    asm volatile("" : "+v"(xv));
                    acc[t] = xv;
                    asm volatile("" : "+a"(acc[t]));
                }
                asm volatile("s_nop 2" ::: "memory");
            }
        };

        // The waves of a head tile with k-split > 0 hand their partial scores
        // to the tile's first wave (k-split 0), which adds them in k-split
        // order and alone runs the softmax; one barrier between the two.
        auto exchange = [&](f32x16_t &s) {
            if constexpr (KS > 1) {
                if (ksplit > 0) {
                    u32x4_t *dst = &s_spart[((ksplit - 1) * HT + ht_w) * 4 * kWave + lane];
#pragma unroll
                    for (int qd = 0; qd < 4; ++qd)
                        dst[qd * kWave] = u32x4_t{as_u(s[4 * qd]), as_u(s[4 * qd + 1]),
                                                  as_u(s[4 * qd + 2]), as_u(s[4 * qd + 3])};
                }
                __syncthreads();
                if (ksplit == 0) {
#pragma unroll
                    for (int j = 1; j < KS; ++j) {
                        const u32x4_t *src = &s_spart[((j - 1) * HT + ht_w) * 4 * kWave + lane];
#pragma unroll
                        for (int qd = 0; qd < 4; ++qd) {
                            const u32x4_t v = src[qd * kWave];
#pragma unroll
                            for (int i = 0; i < 4; ++i) s[4 * qd + i] += as_f(v[i]);
                        }
                    }
                }
            }
        };

        // ---- the software pipeline --------------------------------------------
        // Step u: the score products of unit u + 1 (one dependent chain, with
        // this wave's DMA rows of unit u + 3 and the bookkeeping between its
        // products), then the value products of unit u one at a time, each
        // after an even share of the softmax of unit u + 1.  Unit u + 3
        // streams into the regions units u - 1 (main) and u (RoPE) used.  One
        // barrier per step: every wave's rows of unit u + 1 have landed, every
        // wave's probabilities of unit u are in buffer u & 1, and every wave is
        // done with step u - 1.  Past the segment's last unit the score chain
        // runs over stale LDS and its tokens are all masked (one code path for
        // every step keeps the register allocation in budget).
        for (int u = 0; u < 3; ++u) {
            const bool live = u < nunits;
            if (live) refill_ids(u);
            const UnitDma d = unit_dma(u, live, live ? __builtin_amdgcn_readfirstlane(unit_id(u)) : 0);
            for (int k = 0; k < kPer; ++k) issue_row(u, d, k);
        }
        {  // unit 0's scores and softmax, alone
            // units 1 and 2 (loads issued after unit 0's; vmcnt holds at most
            // 63, and waiting for fewer outstanding loads is safe)
            wait_vmem<(2 * kPer < 63 ? 2 * kPer : 63)>();
            __syncthreads();
            f32x16_t s;
            score_prefetch(0);
            score_steps(s, 0, kKW, [](int) {});
            exchange(s);
            if (ksplit == 0) {
#pragma unroll
                for (int k = 0; k < kSub; ++k) softmax_sub(s, 0, k);
            }
        }

        for (int u = 0; u < nunits; ++u) {
            const int u1 = u + 1, u3 = u + 3;
            const bool has_u3 = u3 < nunits;
            wait_vmem<kPer>();  // this wave's rows of unit u + 1 have landed (unit u + 2's may not)
            const int id3 = has_u3 ? unit_id(u3) : 0;
            __syncthreads();
            // the step's LDS reads first, so that their latency passes under
            // the bookkeeping
            const uint32_t flw = read_flags(u);
            score_prefetch(u1);
            value_prefetch(u);
            UnitDma d3;
            f32x16_t s;
            score_steps(s, 0, kKW, [&](int ks) {
                if (ks == 1) {
                    if (has_u3) refill_ids(u3);
                    d3 = unit_dma(u3, has_u3, __builtin_amdgcn_readfirstlane(id3));
                }
                if (ks >= 2 && (ks - 2) % 3 == 0 && (ks - 2) / 3 < kChainRows) issue_row(u3, d3, (ks - 2) / 3);
                if (ks == kKW - 4) {  // unit u's P^T fragments of k-step 0
#pragma unroll
                    for (int ht = 0; ht < HT; ++ht) p_read(u, 0, ht);
                }
            });
#pragma unroll
            for (int k = kChainRows; k < kPer; ++k) issue_row(u3, d3, k);
            rescale(u, flw);
            exchange(s);
            // kVP value products, one per slot t; before product t the softmax
            // pieces k with k kVP / kSub in [t, t + 1).  A scheduling fence
            // after each product keeps the products apart: back to back, a
            // product waits for the one before it to leave the matrix core and
            // the wave issues nothing else meanwhile.
#pragma unroll
            for (int t = 0; t < kVP; ++t) {
                const int i = t / HT, ht = t % HT;
                if (ksplit == 0) {
#pragma unroll
                    for (int k = (t * kSub + kVP - 1) / kVP; k < ((t + 1) * kSub + kVP - 1) / kVP; ++k)
                        softmax_sub(s, u1, k);
                }
                if (ht == 0) value_begin(u, i);
                value_product(u, i, ht);
                __builtin_amdgcn_sched_barrier(0);
            }
            // This unit's value products drain before the step ends: the
            // compiler may move the accumulators between registers on the
            // loop's edges (its exit, say), ahead of any statement after them.
            acc_fence(acc);
        }

        // ---- this part's result ----------------------------------------------
        // A sequence of one part writes its output, acc / l in bf16.  Otherwise
        // slot j gets (max, sum) per head in fp32 from the score waves, and
        // the part's output normalised by its own sum, acc / l, in fp32; the
        // tiles of a wave go out in register order, so every store writes
        // 1 KB of consecutive bytes.
        const float l_tot = l_run + __shfl_xor(l_run, 32);
        if (ksplit == 0 && hk == 0) s_l[head] = l_tot;
        __syncthreads();  // every head's sum is in s_l
        float inv[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const float l = s_l[ht * kHeads + l31];
            inv[ht] = l > 0.f ? 1.0f / l : 0.f;
        }
        if (k_b == 1) {
            // out[b, h, dims 32 (DT wave + dt) + 8 qd + 4 hk .. + 3] of tile
            // t = dt HT + ht (h = 32 ht + lane % 32)
#pragma unroll
            for (int t = 0; t < NA; ++t) {
                const int dt = t / HT, h = (t % HT) * kHeads + l31;
                if (h >= num_heads) continue;
                const f32x16_t x = acc_tile(acc[t]);
                const float r = inv[t % HT];
                uint16_t *o = out + (static_cast<int64_t>(b) * num_heads + h) * kDV +
                              32 * (DT * wave + dt) + 4 * hk;
#pragma unroll
                for (int qd = 0; qd < 4; ++qd)
                    *reinterpret_cast<uint2 *>(o + 8 * qd) =
                        make_uint2(pack_bf16(x[4 * qd] * r, x[4 * qd + 1] * r),
                                   pack_bf16(x[4 * qd + 2] * r, x[4 * qd + 3] * r));
            }
        } else {
            const int64_t slot = j;
            if (ksplit == 0 && hk == 0) ws_ml[slot * (HT * kHeads) + head] = make_float2(m_run, l_tot);
            f32x4_t *dst = reinterpret_cast<f32x4_t *>(ws_acc) + slot * (kDimTiles * HT * 4 * kWave) +
                           (DT * wave) * (HT * 4 * kWave) + lane;
#pragma unroll
            for (int t = 0; t < NA; ++t) {
                const f32x16_t x = acc_tile(acc[t]);
                const float r = inv[t % HT];
#pragma unroll
                for (int qd = 0; qd < 4; ++qd)
                    dst[(t * 4 + qd) * kWave] =
                        f32x4_t{x[4 * qd] * r, x[4 * qd + 1] * r, x[4 * qd + 2] * r, x[4 * qd + 3] * r};
            }
        }
    }
}

// Log-sum-exp merge of a sequence's parts, O = sum_p 2^(m_p - M) l_p O_p /
// sum_p 2^(m_p - M) l_p (the merge rule of the grouped path, with each part's
// output already divided by its l_p), reading the register-ordered fp32
// tiles: work-group (dim tile dg, b) writes dims 32 dg .. + 31 of every head;
// thread t = 64 ht + lane always sees head 32 ht + (lane & 31), and 16-byte
// piece qd of its tile holds dims 32 dg + 8 qd + 4 (lane >> 5) .. + 3.  The
// kernel is a few memory round trips long, so every load of a batch of
// kBatch parts is issued before any is used, and batches merge by the
// running max.
template <int HT>
__global__ __launch_bounds__(HT *kWave) void latent_reduce_kernel(
    uint16_t *__restrict__ out, const float *__restrict__ ws_acc, const float2 *__restrict__ ws_ml,
    const int32_t *__restrict__ ws_prefix, const int32_t *__restrict__ context_lens,
    int num_seqs, int num_heads) {
    constexpr int kBatch = 8;
    const int dg = blockIdx.x;
    const int b = blockIdx.y;
    const int t = threadIdx.x;
    const int ht = t / kWave, lane = t & (kWave - 1);
    const int head = ht * kHeads + (lane & 31);
    if (head >= num_heads) return;
    // the sequence's parts are slots ws_prefix[b] .. ws_prefix[b + 1] - 1; the
    // prefix is read together with the length (it is in bounds, and written
    // by the partition whenever some context is non-empty)
    const int ctx = context_lens[b];
    const int first = ws_prefix[b];
    const int n = ws_prefix[b + 1] - first;
    asm volatile("" ::"s"(ctx), "s"(first), "s"(n));  // one round trip for the three
    uint16_t *o = out + (static_cast<int64_t>(b) * num_heads + head) * kDV + 32 * dg +
                  4 * (lane >> 5);
    if (ctx <= 0) {  // empty context: O = 0
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) *reinterpret_cast<uint2 *>(o + 8 * qd) = make_uint2(0, 0);
        return;
    }
    if (n == 1) return;  // a sequence of one part: the partition wrote its output

    // part p holds its normalised output O_p (fp32) and (m_p, l_p): the merge
    // weight is 2^(m_p - M) l_p
    float M = kNegInf, den = 0.f;
    f32x4_t num[4] = {};
    for (int p0 = 0; p0 < n; p0 += kBatch) {
        float2 mp[kBatch];
        f32x4_t v[kBatch][4];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if (p0 + j >= n) break;  // (uniform)
            const int64_t slot = first + p0 + j;
            mp[j] = ws_ml[slot * (HT * kHeads) + head];
            const f32x4_t *a = reinterpret_cast<const f32x4_t *>(ws_acc) +
                               slot * (kDimTiles * HT * 4 * kWave) + ((dg * HT + ht) * 4) * kWave +
                               lane;
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) v[j][qd] = a[qd * kWave];
        }
        float bm = kNegInf;
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
            if (p0 + j < n) bm = fmaxf(bm, mp[j].x);
        if (bm > M) {  // the first batch, or a larger max: rescale what is merged
            const float c = exp2_fast(M - bm);
            den *= c;
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) num[qd] *= c;
            M = bm;
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if (p0 + j >= n) break;  // (uniform; those entries were not loaded)
            const float wgt = mp[j].y > 0.f ? exp2_fast(mp[j].x - M) * mp[j].y : 0.f;
            den += wgt;
#pragma unroll
            for (int qd = 0; qd < 4; ++qd)
#pragma unroll
                for (int i = 0; i < 4; ++i) num[qd][i] = fmaf(wgt, v[j][qd][i], num[qd][i]);
        }
    }
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
        const uint32_t lo = pack_bf16(num[qd][0] / den, num[qd][1] / den);
        const uint32_t hi = pack_bf16(num[qd][2] / den, num[qd][3] / den);
        *reinterpret_cast<uint2 *>(o + 8 * qd) = make_uint2(lo, hi);
    }
}

template <int HT>
pa_status enqueue_latent(const DecodeShape &s, const DecodeArgs &a, const DecodePlan &p,
                         float scale_log2, hipStream_t stream, std::string *why) {
    char *ws = static_cast<char *>(a.workspace);
    float *acc = reinterpret_cast<float *>(ws + p.acc_offset);
    float2 *ml = reinterpret_cast<float2 *>(ws + p.ml_offset);
    int32_t *prefix = reinterpret_cast<int32_t *>(ws + p.prefix_offset);
    const auto kernel = latent_partition_kernel<HT>;
    // one work-group per resident slot, and at least one per sequence (each
    // work-group streams a part of one sequence)
    const int waves = std::max(
        stream_waves<latent_partition_kernel<HT>>(kLatentNW * kWave, 1, kLatentWavesMax), s.num_seqs);
    hipLaunchKernelGGL(kernel, dim3(waves), dim3(kLatentNW * kWave), 0, stream,
                       static_cast<uint16_t *>(a.out), acc, ml, prefix,
                       static_cast<const uint16_t *>(a.q), static_cast<const uint16_t *>(a.k_cache),
                       a.block_tables, a.context_lens, scale_log2, s.num_seqs, s.num_q_heads,
                       s.max_blocks_per_seq);
    pa_status st = hip_status(hipGetLastError(), why, "latent partition launch");
    if (st != PA_OK) return st;
    hipLaunchKernelGGL(latent_reduce_kernel<HT>, dim3(kDimTiles, s.num_seqs), dim3(HT * kWave), 0,
                       stream, static_cast<uint16_t *>(a.out), acc, ml, prefix, a.context_lens,
                       s.num_seqs, s.num_q_heads);
    return hip_status(hipGetLastError(), why, "latent reduce launch");
}

}  // namespace

pa_status launch_latent_decode(const DecodeShape &s, const DecodeArgs &a, const DecodePlan &p,
                               void *stream_arg, std::string *why) {
    const hipStream_t stream = static_cast<hipStream_t>(stream_arg);
    if (s.num_seqs == 0) return PA_OK;
    const float scale_log2 = static_cast<float>(static_cast<double>(a.scale) * 1.4426950408889634);
    switch (latent_head_tiles(s.num_q_heads)) {
        case 1: return enqueue_latent<1>(s, a, p, scale_log2, stream, why);
        case 2: return enqueue_latent<2>(s, a, p, scale_log2, stream, why);
        default: return enqueue_latent<4>(s, a, p, scale_log2, stream, why);
    }
}

}  // namespace pa
