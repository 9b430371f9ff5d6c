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
//  * A work-group has NW = 1, 2 or 4 waves, one per SIMD, and covers 32 NW
//    heads (the query heads, padded).  The latent is streamed in units of 32
//    tokens (half a 64-token block, 36 KB) by global_load_lds_dwordx4 into a
//    four-slot LDS ring: two units are in flight while one is read, by
//    every wave, from LDS (deeper read-ahead only stalled the in-order waves
//    at issue).  Rows past the context are zero-filled instead of fetched.
//  * Scores: wave w computes S^T[token, head] = L[token, :] . Q^T for heads
//    32w..32w+31; the latent rows are the A operand (16 contiguous bytes per
//    lane) and q sits in registers as the B operand for the whole segment.
//    A lane's S^T accumulator holds 16 of the unit's 32 tokens for one head
//    (the other 16 sit in lane ^ 32), so the running max is an in-lane max
//    and one lane exchange, and the probabilities, rounded to bf16, come out
//    in the B-operand layout of O^T[dim, head] += V^T[dim, token] .
//    P^T[token, head].  They go to LDS (8 KB per unit), with the rescale
//    factors of heads whose running max moved.
//  * Values: wave w accumulates O^T for dims 512 w / NW .. + 512 / NW - 1 of
//    every head, as (16 / NW) x NW register-blocked 32 x 32 tiles held in the
//    accumulation registers (256 per lane).  Each V^T fragment (transposed
//    reads, ds_read_b64_tr_b16) feeds NW products and each P^T fragment
//    16 / NW, so the LDS traffic per product stays well under what the
//    matrix core consumes.
//  * LDS layout of a unit: the first 64 16-byte chunks of every row (dims
//    0..511) in a 32 KB region of 1 KB rows, the 8 RoPE chunks in a 4 KB
//    region of 128-byte rows.  Chunk c of main row t sits at c ^ swm(t),
//    RoPE chunk c of row t at c ^ swr(t); both keep every phase of the
//    row-wise and transposed reads on distinct banks.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
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
constexpr int kAhead = 2;                     // units in flight while one is computed
constexpr int kSlots = 4;                     // ring slots (a power of two keeps the
                                              // slot arithmetic in shifts and immediates)
constexpr int kDmaPerUnit = kUnitB / 1024;    // 36: 32 main rows + 4 groups of 8 RoPE rows
constexpr int kHeads = 32;                    // heads per wave in the scores (one tile)
constexpr int kKSteps = kDK / 16;             // 36 k-steps of q . L
constexpr int kMainKSteps = kDV / 16;         // the first 32 of them read the main region
constexpr int kDimTiles = kDV / 32;           // 16 tiles of the output
constexpr float kLSlack = 8.0f;               // lazy-rescale threshold, log2 units
constexpr int kQD = 6;                        // S^T k-steps of A operands read ahead

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
// The last product of each of the two score chains, then the fence.
__device__ __forceinline__ void mfma_v_last(f32x16_t &c0, f32x16_t &c1, bf16x8_t a0, bf16x8_t a1,
                                            bf16x8_t b0, bf16x8_t b1) {
    asm volatile(
        "v_mfma_f32_32x32x16_bf16 %0, %2, %4, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %1, %3, %5, %1\n\t"
        "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
        : "+v"(c0), "+v"(c1) : "v"(a0), "v"(a1), "v"(b0), "v"(b1) : "memory");
}
__device__ __forceinline__ void mfma_a(f32x16_t &c, bf16x8_t a, bf16x8_t b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b) : "memory");
}
// Fence over the 16 output tiles (before the rescale and the final store).
__device__ __forceinline__ void acc_fence(f32x16_t (&acc)[16]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]), "+a"(acc[4]),
                   "+a"(acc[5]), "+a"(acc[6]), "+a"(acc[7]), "+a"(acc[8]), "+a"(acc[9]),
                   "+a"(acc[10]), "+a"(acc[11]), "+a"(acc[12]), "+a"(acc[13]), "+a"(acc[14]),
                   "+a"(acc[15])
                 :: "memory");
}

template <int NW>
__global__ __launch_bounds__(NW *kWave) __attribute__((amdgpu_waves_per_eu(1, 1)))
void latent_partition_kernel(float *__restrict__ ws_acc, float2 *__restrict__ ws_ml,
                             int32_t *__restrict__ ws_prefix, const uint16_t *__restrict__ q,
                             const uint16_t *__restrict__ latent,
                             const int32_t *__restrict__ block_tables,
                             const int32_t *__restrict__ context_lens, float scale_log2,
                             int num_seqs, int num_heads, int max_blocks) {
    constexpr int HT = NW;              // head tiles (of 32) in the work-group
    constexpr int DT = kDimTiles / NW;  // output dim tiles per wave
    static_assert(DT * HT == 16, "16 accumulator tiles per wave");
    constexpr int kVR = 4;              // V^T operands read ahead

    __shared__ __attribute__((aligned(16))) uint4 s_ring[kSlots][kUnitB / 16];
    __shared__ __attribute__((aligned(16))) u32x4_t s_p[HT][2][kWave];  // P^T fragments
    __shared__ float s_alpha[HT * kHeads];  // rescale factor of each head this unit
    __shared__ __attribute__((aligned(16))) int32_t s_flag[4];  // head tile ht rescaled
    __shared__ __attribute__((aligned(16))) int32_t s_ids[2][kWave];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    __builtin_assume(wave >= 0 && wave < NW);
    const int l31 = lane & 31;    // MFMA row (A) / column (B, C) of this lane
    const int hk = lane >> 5;     // which 8 of a 16-wide k-step this lane holds
    const int head = wave * kHeads + l31;  // this lane's head in the scores
    const bool head_ok = head < num_heads;

    // ---- this work-group's share of the global block order (b, block) ----
    int seq_blocks_total = 0;
    for (int base = 0; base < num_seqs; base += kWave) {
        const int bb = base + lane;
        const int nb = bb < num_seqs ? (context_lens[bb] + kLBS - 1) / kLBS : 0;
        const int incl = wave_incl_scan(nb, lane);
        if (blockIdx.x == 0 && wave == 0 && bb < num_seqs)
            ws_prefix[bb] = seq_blocks_total + incl - nb;
        seq_blocks_total += __builtin_amdgcn_readlane(incl, kWave - 1);
    }
    if (blockIdx.x == 0 && tid == 0) ws_prefix[num_seqs] = seq_blocks_total;
    const int total = seq_blocks_total;
    const int share = stream_share(total, static_cast<int>(gridDim.x));
    const int64_t x0l = static_cast<int64_t>(blockIdx.x) * share;
    if (x0l >= total) return;  // uniform over the work-group
    const int x0 = static_cast<int>(x0l);
    const int x1 = min(x0 + share, total);

    int b = 0, nbb = 0, cb = 0;
    for (int base = 0, carry = 0;; base += kWave) {
        const int bb = base + lane;
        const int nb = bb < num_seqs ? (context_lens[bb] + kLBS - 1) / kLBS : 0;
        const int incl = wave_incl_scan(nb, lane);
        const uint64_t hit = __builtin_amdgcn_ballot_w64(bb < num_seqs && carry + incl > x0);
        if (hit != 0) {
            const int f = __builtin_ctzll(hit);
            b = base + f;
            nbb = __builtin_amdgcn_readlane(nb, f);
            cb = carry + __builtin_amdgcn_readlane(incl, f) - nbb;
            break;
        }
        carry += __builtin_amdgcn_readlane(incl, kWave - 1);
    }
    int blk_start = x0 - cb;

    const uint32_t ring_lds = lds_offset(s_ring);
    const uint32_t ids_lds[2] = {lds_offset(&s_ids[0][0]), lds_offset(&s_ids[1][0])};

    // ---- per-lane LDS addresses (bytes, relative to a ring slot) ----------
    // S^T A operand: unit row l31, chunk 2 ks + hk.  swm of that row is
    // swm(lane & 15) and the xor touches the low 4 chunk bits only, so the
    // byte offset in a row is 256 (ks >> 3) + (32 (ks & 7) ^ qx) with
    // qx = 16 (hk ^ swm).  RoPE rows likewise: offset 32 (ks - 32) ^ rx.
    const uint32_t qrow = l31 * kMainRowB;
    const uint32_t qx = 16u * static_cast<uint32_t>(hk ^ swm(lane & 15));
    const uint32_t rrow = kUnitMainB + l31 * kRopeRowB;
    const uint32_t rx = 16u * static_cast<uint32_t>(hk ^ swr(l31));
    // V^T A operand by transposed reads.  16-lane group g = lane >> 4 reads
    // rows tb + (i >> 2), i = lane & 15, dims 32 dt + 16 (g & 1) + 4 (i & 3),
    // with tb = 16 s + 8 qq + 4 hk; lane i then receives the 4 tokens
    // tb .. tb + 3 of dim 32 dt + (lane & 31).  The row's swm depends on
    // (qq, hk, i >> 2) only; the chunk is 16 (dt >> 2) + 4 (dt & 3) + c0 with
    // c0 = 2 (g & 1) + ((i & 3) >> 1) < 4, so the offset in a row is
    // 256 (dt >> 2) + (64 (dt & 3) ^ vy[qq]) with vy = 16 (c0 ^ swm(row)).
    uint32_t vrow[2], vy[2];
    {
        const int i = lane & 15;
        const int c0 = 2 * ((lane >> 4) & 1) + ((i & 3) >> 1);
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
            const int trow = 8 * qq + 4 * hk + (i >> 2);
            vrow[qq] = trow * kMainRowB + 8 * (i & 1);
            vy[qq] = 16u * static_cast<uint32_t>(c0 ^ swm(trow));
        }
    }
    // P^T fragment (head tile ht, k-step s) of this lane: 16 bytes
    const uint32_t p_lds = lds_offset(&s_p[0][0][0]) + 16 * lane;

    for (int x = x0;;) {
        // ======== segment: sequence b, blocks [blk_start, blk_start + nblk) ========
        const int nblk = min(nbb - blk_start, x1 - x);
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
        // q^T B-operand fragments of this lane's head: dims 16 ks + 8 hk .. + 7
        // for every k-step (zero for padding heads past num_heads).
        bf16x8_t qf[kKSteps];
        if (head_ok) {
            const uint4 *qr = reinterpret_cast<const uint4 *>(
                q + (static_cast<int64_t>(b) * num_heads + head) * kDK + 8 * hk);
#pragma unroll
            for (int ks = 0; ks < kKSteps; ++ks) qf[ks] = __builtin_bit_cast(bf16x8_t, qr[2 * ks]);
#pragma unroll
            for (int ks = 0; ks < kKSteps; ++ks) settle(qf[ks]);
        } else {
#pragma unroll
            for (int ks = 0; ks < kKSteps; ++ks) qf[ks] = bf16x8_t{};
        }
        drain_vmem();
        __syncthreads();  // ids landed for every wave; the previous segment is done

        float m_run = kNegInf;  // running max of this lane's head (log2 units)
        float l_run = 0.f;      // this lane's share of its running sum
        // O^T tile (dt, ht) = acc[dt * HT + ht]: dims 32 (DT wave + dt) +
        // 8 (j >> 2) + 4 hk + (j & 3) of head 32 ht + l31
        f32x16_t acc[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) acc[t] = f32x16_t{};

        // Units of this segment: 32-token halves of its blocks that hold at
        // least one context token (only a sequence's last block can end
        // early, so unit u is half u & 1 of block u >> 1).
        const int seg_tok0 = blk_start * kLBS;
        const int nunits =
            (min(ctx, (blk_start + nblk) * kLBS) - seg_tok0 + kUnitTok - 1) / kUnitTok;

        // DMA of unit u into ring slot u % 4: this wave's rows i = wave + NW k,
        // k < kPer, of the unit's 36 (32 main rows, 4 groups of 8 RoPE rows).
        // Main rows at or past the context are zero-filled instead (NaN in the
        // V operand would survive a zero probability); RoPE rows only feed
        // scores, which are masked.
        constexpr int kPer = (kDmaPerUnit + NW - 1) / NW;
        auto unit_src = [&](int u, int pb) {
            return reinterpret_cast<const char *>(latent) + static_cast<int64_t>(pb) * kBlockB +
                   (u & 1) * kUnitTok * kRowB;
        };
        auto issue_row = [&](int u, const char *src, int k) {
            const int i = wave + NW * k;
            if (i >= kDmaPerUnit) return;
            const uint32_t slot = ring_lds + (u % kSlots) * kUnitB;
            // recomputed per row rather than kept live across the loop
            int ln = lane;
            asm volatile("" : "+v"(ln));
            if (i < kUnitTok) {  // main region: row i, lane = swizzled chunk
                if (i < ctx - (seg_tok0 + u * kUnitTok)) {
                    dma16(src, i * kRowB + ((ln ^ swm(i)) * 16), slot + i * kMainRowB);
                } else {
                    *(__attribute__((address_space(3))) u32x4_t *)(uintptr_t)(
                        slot + i * kMainRowB + ln * 16) = u32x4_t{0, 0, 0, 0};
                }
            } else {             // RoPE region: 8 rows x 8 chunks
                const int t = 8 * (i - kUnitTok) + (ln >> 3);
                dma16(src, t * kRowB + (kMainChunks + ((ln & 7) ^ swr(t))) * 16,
                      slot + kUnitMainB + (i - kUnitTok) * 1024);
            }
        };
        // Block ids come in chunks of 64 through s_ids; wave 0 fetches chunk
        // c + 1 when the first unit of chunk c is issued.
        auto refill_ids = [&](int u) {
            const int n = u >> 1;
            if (wave == 0 && (u & 1) == 0 && (n & (kWave - 1)) == 0 && n > 0 && n + kWave < nblk)
                fetch_ids((n >> 6) + 1);
        };
        auto unit_id = [&](int u) { return s_ids[((u >> 1) >> 6) & 1][(u >> 1) & (kWave - 1)]; };

        // V^T operand (k-step s, this wave's dim tile dt, half qq) of unit u
        auto pv_read = [&](int u, int s, int dt, int qq) {
            const int dg = DT * wave + dt;  // global dim tile
            return ds_read_tr(ring_lds + (u % kSlots) * kUnitB + (16 * s) * kMainRowB +
                              256 * (dg >> 2) + vrow[qq] + ((64u * (dg & 3)) ^ vy[qq]));
        };

        // ---- scores and probabilities of unit u for this wave's 32 heads ----
        auto scores = [&](int u, int un, const char *srcn) {
            const uint32_t slot = ring_lds + (u % kSlots) * kUnitB;
            const int tok0 = seg_tok0 + u * kUnitTok;
            // S^T = L . Q^T: 32 tokens x 32 heads, in two accumulator chains
            // (even and odd k-steps)
            auto qk_read = [&](int ks) {
                const uint32_t addr =
                    ks < kMainKSteps
                        ? slot + qrow + 256 * (ks >> 3) + ((32u * (ks & 7)) ^ qx)
                        : slot + rrow + ((32u * (ks - kMainKSteps)) ^ rx);
                return ds_read_b128(addr);
            };
            bf16x8_t xa[kQD];
#pragma unroll
            for (int ks = 0; ks < kQD; ++ks) xa[ks] = qk_read(ks);
            f32x16_t sa, sb;
#pragma unroll
            for (int ks = 0; ks < kKSteps; ++ks) {
                const int r = ks % kQD;
                if (ks < 2) {
                    mfma_v0(ks ? sb : sa, xa[r], qf[ks]);
                } else if (ks + 2 < kKSteps) {
                    mfma_v(ks & 1 ? sb : sa, xa[r], qf[ks]);
                } else if (ks + 1 == kKSteps) {
                    mfma_v_last(sa, sb, xa[(ks - 1) % kQD], xa[r], qf[ks - 1], qf[ks]);
                }
                if (ks + kQD < kKSteps && ks + 2 < kKSteps) xa[r] = qk_read(ks + kQD);
                // this wave's DMA rows of unit un, spread over 9 points of the
                // chain so that each issues in the shadow of the products
                if ((ks & 3) == 3 && un >= 0) {
                    constexpr int kStep = (kPer + 8) / 9;
#pragma unroll
                    for (int k = (ks >> 2) * kStep; k < ((ks >> 2) + 1) * kStep && k < kPer; ++k)
                        issue_row(un, srcn, k);
                }
            }
            // online softmax: reg j holds token 8 (j >> 2) + 4 hk + (j & 3) of
            // the unit for this lane's head
            float lmax = kNegInf;
            if (tok0 + kUnitTok <= ctx) {  // every unit but a sequence's last
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    sa[j] = (sa[j] + sb[j]) * scale_log2;
                    lmax = fmaxf(lmax, sa[j]);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int tk = tok0 + 8 * (j >> 2) + 4 * hk + (j & 3);
                    sa[j] = tk < ctx ? (sa[j] + sb[j]) * scale_log2 : kNegInf;
                    lmax = fmaxf(lmax, sa[j]);
                }
            }
            const float bmax = fmaxf(lmax, __shfl_xor(lmax, 32));
            const bool moved = __builtin_amdgcn_ballot_w64(bmax > m_run + kLSlack) != 0;
            if (moved) {
                const float m_new = fmaxf(m_run, bmax);
                const float alpha = exp2_fast(m_run - m_new);
                l_run *= alpha;
                m_run = m_new;
                if (hk == 0) s_alpha[head] = alpha;
            }
            if (lane == 0) s_flag[wave] = moved && u > 0;  // u = 0: the accumulators are zero
            // P^T B-operand fragment of k-step s (tokens 16 s ..): k = 8 hk + jj
            // is S^T reg 8 s + jj
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                uint32_t w4[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    w4[v] = pack_bf16(exp2_fast(sa[8 * s + 2 * v] - m_run),
                                      exp2_fast(sa[8 * s + 2 * v + 1] - m_run));
                    l_run += bf16_lo(w4[v]) + bf16_hi(w4[v]);
                }
                s_p[wave][s][lane] = u32x4_t{w4[0], w4[1], w4[2], w4[3]};
            }
        };

        // ---- O^T += V^T . P^T for this wave's dims, every head, unit u ------
        // V^T operand i = DT s + dt (k-step s, dim tile dt) sits in ring slot
        // i % kVR of vlo / vhi; the first kVR are read before the barrier.
        auto values = [&](int u, s16x4_t (&vlo)[kVR], s16x4_t (&vhi)[kVR]) {
            // rescale the heads whose running max moved (rare); tile by tile
            // through VGPRs so that at most one tile is out of the
            // accumulation registers at a time
            const u32x4_t fl = *(const __attribute__((address_space(3))) u32x4_t *)(
                uintptr_t)lds_offset(s_flag);
            if (__builtin_expect((fl[0] | fl[1] | fl[2] | fl[3]) != 0, 0)) {
                float alpha[HT];
#pragma unroll
                for (int ht = 0; ht < HT; ++ht)
                    alpha[ht] = fl[ht] != 0 ? s_alpha[ht * kHeads + l31] : 1.0f;
                acc_fence(acc);
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    f32x16_t x = acc[t];
                    asm volatile("" : "+v"(x));
                    x *= alpha[t % HT];
                    asm volatile("" : "+v"(x));
                    acc[t] = x;
                    asm volatile("" : "+a"(acc[t]));
                }
                asm volatile("s_nop 2" ::: "memory");
            }
            bf16x8_t pb[HT];
#pragma unroll
            for (int i = 0; i < 2 * DT; ++i) {
                const int s = i / DT, dt = i % DT;
                if (dt == 0) {
#pragma unroll
                    for (int ht = 0; ht < HT; ++ht)
                        pb[ht] = ds_read_b128(p_lds + (ht * 2 + s) * kWave * 16);
                }
                const int r = i % kVR;
                const bf16x8_t va = __builtin_bit_cast(
                    bf16x8_t, __builtin_shufflevector(vlo[r], vhi[r], 0, 1, 2, 3, 4, 5, 6, 7));
                if (i + kVR < 2 * DT) {
                    vlo[r] = pv_read(u, (i + kVR) / DT, (i + kVR) % DT, 0);
                    vhi[r] = pv_read(u, (i + kVR) / DT, (i + kVR) % DT, 1);
                }
#pragma unroll
                for (int ht = 0; ht < HT; ++ht) mfma_a(acc[dt * HT + ht], va, pb[ht]);
            }
        };

        for (int u = 0; u < nunits && u < kAhead; ++u) {
            refill_ids(u);
            const char *src = unit_src(u, __builtin_amdgcn_readfirstlane(unit_id(u)));
            for (int k = 0; k < kPer; ++k) issue_row(u, src, k);
        }
        for (int u = 0; u < nunits; ++u) {
            // unit un streams in during this step; its block id is read before
            // the barrier, whose LDS wait covers the read
            const int un = u + kAhead < nunits ? u + kAhead : -1;
            const int idn = un >= 0 ? unit_id(un) : 0;
            // this wave's rows of unit u have landed once at most the units
            // issued after it are outstanding
            const int later = min(nunits - 1 - u, kAhead - 1);
            if (later >= 2 && 2 * kPer <= 63) wait_vmem<(2 * kPer <= 63 ? 2 * kPer : 0)>();
            else if (later >= 1 && kPer <= 63) wait_vmem<(kPer <= 63 ? kPer : 0)>();
            else wait_vmem<0>();
            __syncthreads();  // every wave's rows landed; unit u - 1 is no longer read
            if (un >= 0) refill_ids(un);
            scores(u, un, un >= 0 ? unit_src(un, __builtin_amdgcn_readfirstlane(idn)) : nullptr);
            // the first V^T operands go out before the barrier
            s16x4_t vlo[kVR], vhi[kVR];
#pragma unroll
            for (int i = 0; i < kVR; ++i) {
                vlo[i] = pv_read(u, i / DT, i % DT, 0);
                vhi[i] = pv_read(u, i / DT, i % DT, 1);
            }
            __syncthreads();  // every wave's probabilities and rescale flags are in LDS
            values(u, vlo, vhi);
        }

        // ---- this segment's partial -----------------------------------------
        // Slot blockIdx.x + b: (max, sum) per head from the score waves; the
        // accumulator tiles of this wave in register order, so every store
        // writes 1 KB of consecutive bytes.
        const float l_tot = l_run + __shfl_xor(l_run, 32);
        acc_fence(acc);
        {
            const int64_t slot = static_cast<int64_t>(blockIdx.x) + b;
            if (hk == 0) ws_ml[slot * (HT * kHeads) + head] = make_float2(m_run, l_tot);
            f32x4_t *dst = reinterpret_cast<f32x4_t *>(ws_acc) + slot * (16 * HT * 4 * kWave) +
                           (DT * wave) * (HT * 4 * kWave) + lane;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int ht = 0; ht < HT; ++ht)
#pragma unroll
                    for (int qd = 0; qd < 4; ++qd) {
                        const f32x16_t &t = acc[dt * HT + ht];
                        dst[((dt * HT + ht) * 4 + qd) * kWave] =
                            f32x4_t{t[4 * qd], t[4 * qd + 1], t[4 * qd + 2], t[4 * qd + 3]};
                    }
        }

        x += nblk;
        if (x >= x1) break;
        blk_start = 0;
        do {
            ++b;
            nbb = (context_lens[b] + kLBS - 1) / kLBS;
        } while (nbb == 0);
        wait_lds();
        __syncthreads();  // every wave is done with this segment's LDS and ids
    }
}

// Log-sum-exp merge of a sequence's partial slots (the same merge rule as the
// grouped path), reading the register-ordered tiles: work-group (dim tile
// dg, b) writes dims 32 dg .. + 31 of every head; thread t = 64 ht + lane
// always sees head 32 ht + (lane & 31), and float4 qd of its tile holds dims
// 32 dg + 8 qd + 4 (lane >> 5) .. + 3.
template <int NW>
__global__ __launch_bounds__(NW *kWave) void latent_reduce_kernel(
    uint16_t *__restrict__ out, const float *__restrict__ ws_acc, const float2 *__restrict__ ws_ml,
    const int32_t *__restrict__ ws_prefix, const int32_t *__restrict__ context_lens,
    int num_seqs, int num_heads, int waves) {
    constexpr int HT = NW;
    const int dg = blockIdx.x;
    const int b = blockIdx.y;
    const int t = threadIdx.x;
    const int ht = t / kWave, lane = t & (kWave - 1);
    const int head = ht * kHeads + (lane & 31);
    if (head >= num_heads) return;
    const int nb = (context_lens[b] + kLBS - 1) / kLBS;
    uint16_t *o = out + (static_cast<int64_t>(b) * num_heads + head) * kDV + 32 * dg +
                  4 * (lane >> 5);
    if (nb <= 0) {  // empty context: O = 0
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) *reinterpret_cast<uint2 *>(o + 8 * qd) = make_uint2(0, 0);
        return;
    }
    const int share = stream_share(ws_prefix[num_seqs], waves);
    const int seg_lo = ws_prefix[b];
    const int w0 = seg_lo / share;
    const int n = (seg_lo + nb - 1) / share - w0 + 1;  // partial slots of this sequence
    const int64_t first = static_cast<int64_t>(w0) + b;  // slot of w0

    float M = kNegInf;
    for (int p = 0; p < n; ++p) M = fmaxf(M, ws_ml[(first + p) * (HT * kHeads) + head].x);
    f32x4_t num[4] = {};
    float den = 0.f;
    for (int p = 0; p < n; ++p) {
        const float2 mp = ws_ml[(first + p) * (HT * kHeads) + head];
        const float wgt = exp2_fast(mp.x - M);
        den = fmaf(wgt, mp.y, den);
        const f32x4_t *a = reinterpret_cast<const f32x4_t *>(ws_acc) +
                           (first + p) * (16 * HT * 4 * kWave) + ((dg * HT + ht) * 4) * kWave + lane;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) num[qd] += wgt * a[qd * kWave];
    }
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
        const uint32_t lo = pack_bf16(num[qd][0] / den, num[qd][1] / den);
        const uint32_t hi = pack_bf16(num[qd][2] / den, num[qd][3] / den);
        *reinterpret_cast<uint2 *>(o + 8 * qd) = make_uint2(lo, hi);
    }
}

template <int NW>
pa_status enqueue_latent(const DecodeShape &s, const DecodeArgs &a, const DecodePlan &p,
                         float scale_log2, hipStream_t stream, std::string *why) {
    char *ws = static_cast<char *>(a.workspace);
    float *acc = reinterpret_cast<float *>(ws + p.acc_offset);
    float2 *ml = reinterpret_cast<float2 *>(ws + p.ml_offset);
    int32_t *prefix = reinterpret_cast<int32_t *>(ws + p.prefix_offset);
    const auto kernel = latent_partition_kernel<NW>;
    const int waves = stream_waves(kernel, NW * kWave, 1, kLatentWavesMax);
    hipLaunchKernelGGL(kernel, dim3(waves), dim3(NW * kWave), 0, stream, acc, ml, prefix,
                       static_cast<const uint16_t *>(a.q), static_cast<const uint16_t *>(a.k_cache),
                       a.block_tables, a.context_lens, scale_log2, s.num_seqs, s.num_q_heads,
                       s.max_blocks_per_seq);
    pa_status st = hip_status(hipGetLastError(), why, "latent partition launch");
    if (st != PA_OK) return st;
    hipLaunchKernelGGL(latent_reduce_kernel<NW>, dim3(kDimTiles, s.num_seqs), dim3(NW * kWave), 0,
                       stream, static_cast<uint16_t *>(a.out), acc, ml, prefix, a.context_lens,
                       s.num_seqs, s.num_q_heads, waves);
    return hip_status(hipGetLastError(), why, "latent reduce launch");
}

}  // namespace

pa_status launch_latent_decode(const DecodeShape &s, const DecodeArgs &a, const DecodePlan &p,
                               hipStream_t stream, std::string *why) {
    if (s.num_seqs == 0) return PA_OK;
    const float scale_log2 = static_cast<float>(static_cast<double>(a.scale) * 1.4426950408889634);
    switch (latent_waves(s.num_q_heads)) {
        case 1: return enqueue_latent<1>(s, a, p, scale_log2, stream, why);
        case 2: return enqueue_latent<2>(s, a, p, scale_log2, stream, why);
        default: return enqueue_latent<4>(s, a, p, scale_log2, stream, why);
    }
}

}  // namespace pa
