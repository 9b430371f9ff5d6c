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
// contraction and runs on the matrix cores (v_mfma_f32_16x16x32_bf16):
//  * A work-group of NW waves covers NW * 16 heads; wave w owns heads
//    16w..16w+15.  Each 64-token block (72 KB) is fetched once per
//    work-group by global_load_lds_dwordx4 into a two-slot LDS ring and read
//    by every wave from LDS.
//  * Scores are computed transposed, S^T[token, head] = L[token, :] . Q^T:
//    the latent rows are the A operand (16 contiguous bytes per lane) and q
//    sits in registers as the B operand for the whole segment.
//  * The S^T accumulator of a lane holds 16 tokens of one head, so the
//    running max is an in-lane max plus two lane exchanges, and the
//    probabilities, rounded to bf16, are already in the B-operand layout of
//    O^T[dim, head] += V^T[dim, token] . P^T[token, head].  V^T fragments come
//    from the row-major latent with ds_read_b64_tr_b16 (transposed reads).
//  * LDS layout of a block: the first 64 16-byte chunks of every row (dims
//    0..511) in a 64 KB region, the 8 RoPE chunks in an 8 KB region; chunk c
//    of row t sits at c ^ swz(t) within its row, which keeps both the
//    row-wise A reads and the transposed reads free of bank conflicts.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "launch.h"

namespace pa {
namespace {

constexpr int kLBS = 64;                      // tokens per cache block
constexpr int kDK = 576;                      // latent width (key)
constexpr int kDV = 512;                      // value width (leading part of the row)
constexpr int kRowB = kDK * 2;                // bytes per token row
constexpr int kMainChunks = kDV * 2 / 16;     // 64 chunks: dims 0..511
constexpr int kRopeChunks = kRowB / 16 - kMainChunks;  // 8 chunks: dims 512..575
constexpr int kMainB = kLBS * kMainChunks * 16;        // 64 KB region
constexpr int kBlockB = kLBS * kRowB;                  // 72 KB per block
constexpr int kDmaPerBlock = kBlockB / 1024;           // 64 lanes x 16 bytes each
constexpr int kHeadsPerWave = 16;
constexpr int kKSteps = kDK / 32;             // 18 k-steps of q . L
constexpr int kMainKSteps = kDV / 32;         // the first 16 of them read the main region
constexpr int kDimTiles = kDV / 16;           // 32 tiles of the output
constexpr float kLSlack = 8.0f;               // lazy-rescale threshold, log2 units

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Chunk c of token row t is stored at chunk c ^ swz(t) of its row.  Over any
// 8 rows swz is a permutation of 0..7 (row-wise reads of one chunk column
// hit 8 different bank groups), and over 4 aligned rows swz >> 1 is one too
// (a transposed read of 2 adjacent chunks x 4 rows hits 8 groups).
__host__ __device__ constexpr int swz(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }

__device__ __forceinline__ s16x4_t ds_read_tr(uint32_t byte_addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t *)(uintptr_t)byte_addr);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t ds_read_b128(uint32_t byte_addr) {
    return __builtin_bit_cast(
        bf16x8_t, *(const __attribute__((address_space(3))) u32x4_t *)(uintptr_t)byte_addr);
}

template <int NW>
__global__ __launch_bounds__(NW *kWave) void latent_partition_kernel(
    float *__restrict__ ws_acc, float2 *__restrict__ ws_ml, int32_t *__restrict__ ws_prefix,
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ latent,
    const int32_t *__restrict__ block_tables, const int32_t *__restrict__ context_lens,
    float scale_log2, int num_seqs, int max_blocks) {
    constexpr int HQ = NW * kHeadsPerWave;

    __shared__ __attribute__((aligned(16))) uint4 s_ring[2][kBlockB / 16];
    __shared__ __attribute__((aligned(16))) int32_t s_ids[2][kWave];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int grp = lane >> 4;     // 16-lane group: MFMA k-half / transposed-read group
    const int gi = lane & 15;      // MFMA row / column index of this lane
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
    // q . L A operand: token row t = 16 mt + gi, chunk 4 ks + grp.  swz(t) =
    // swz(gi) for every mt, and (4 ks + grp) ^ swz = 8 (ks >> 1) +
    // ((4 (ks & 1) + grp) ^ swz), so two per-lane bases cover every k-step.
    const int sq = swz(gi);
    uint32_t a_main[2], a_rope[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const uint32_t x = static_cast<uint32_t>(((4 * m + grp) ^ sq) * 16);
        a_main[m] = gi * (kMainChunks * 16) + x;
        a_rope[m] = kMainB + gi * (kRopeChunks * 16) + x;
    }
    // V^T A operand by transposed reads: lane (grp, gi) addresses row
    // t_base + (gi >> 2), dims 16 dt + 4 (gi & 3), with t_base = 32 kk +
    // 4 grp (+ 16).  swz of that row is F = 2 (gi >> 2) + (grp & 1) for every
    // kk, and the chunk is 2 dt + e, e = (gi & 3) >> 1, so (2 dt + e) ^ F =
    // 8 (dt >> 2) + ((2 (dt & 3) + e) ^ F): four per-lane bases.
    const int F = 2 * (gi >> 2) + (grp & 1);
    const int e = (gi & 3) >> 1;
    uint32_t v_base[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
        v_base[m] = (4 * grp + (gi >> 2)) * (kMainChunks * 16) + (((2 * m + e) ^ F) * 16) +
                    8 * (gi & 1);

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
        // q^T fragments of this wave's 16 heads: head 16 wave + gi, dims
        // 32 ks + 8 grp .. + 7 for every k-step.
        bf16x8_t qf[kKSteps];
        {
            const uint4 *qr = reinterpret_cast<const uint4 *>(
                q + (static_cast<int64_t>(b) * HQ + wave * kHeadsPerWave + gi) * kDK + 8 * grp);
#pragma unroll
            for (int ks = 0; ks < kKSteps; ++ks)
                qf[ks] = __builtin_bit_cast(bf16x8_t, qr[4 * ks]);
        }
        drain_vmem();
        __syncthreads();  // ids landed for every wave; the previous segment is done

        float m_run = kNegInf;  // running max of head 16 wave + gi (log2 units)
        float l_run = 0.f;      // this lane's share of its running sum
        f32x4_t acc[kDimTiles];  // O^T tile dt: dims 16 dt + 4 grp + j, head gi
#pragma unroll
        for (int dt = 0; dt < kDimTiles; ++dt) acc[dt] = f32x4_t{};

        // Start block n streaming into ring slot n & 1: this wave's DMA rows.
        auto issue = [&](int n) {
            if (wave == 0 && (n & (kWave - 1)) == 0 && n > 0 && n + kWave < nblk)
                fetch_ids((n >> 6) + 1);
            const int pb = __builtin_amdgcn_readfirstlane(s_ids[(n >> 6) & 1][n & (kWave - 1)]);
            const char *src = reinterpret_cast<const char *>(latent) +
                              static_cast<int64_t>(pb) * kBlockB;
            const uint32_t slot = ring_lds + (n & 1) * kBlockB;
            for (int i = wave; i < kDmaPerBlock; i += NW) {  // this wave's DMA rows
                uint32_t voff;
                if (i < kLBS) {  // main region: token i, lane = swizzled chunk
                    voff = i * kRowB + ((lane ^ swz(i)) * 16);
                } else {         // RoPE region: 8 tokens x 8 chunks
                    const int t = 8 * (i - kLBS) + (lane >> 3);
                    voff = t * kRowB + (kMainChunks + ((lane & 7) ^ swz(t))) * 16;
                }
                dma16(src, voff, slot + i * 1024);
            }
        };

        auto compute_block = [&](int n) {
            const uint32_t slot = ring_lds + (n & 1) * kBlockB;
            const int tok0 = (blk_start + n) * kLBS;
            // ---- S^T = L . Q^T: 4 tiles of 16 tokens x this wave's 16 heads ---
            // Reads go 3 k-steps ahead of their products; the scheduling
            // barriers keep the compiler from hoisting all of them.
            f32x4_t st[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                f32x4_t c = f32x4_t{};
#pragma unroll
                for (int k3 = 0; k3 < kKSteps; k3 += 3) {
                    bf16x8_t a[3];
#pragma unroll
                    for (int u = 0; u < 3; ++u) {
                        const int ks = k3 + u;
                        const uint32_t addr =
                            ks < kMainKSteps
                                ? slot + a_main[ks & 1] + 128 * (ks >> 1) +
                                      mt * 16 * (kMainChunks * 16)
                                : slot + a_rope[ks & 1] + mt * 16 * (kRopeChunks * 16);
                        a[u] = ds_read_b128(addr);
                    }
#pragma unroll
                    for (int u = 0; u < 3; ++u)
                        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], qf[k3 + u], c, 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
                st[mt] = c;
            }
            // ---- online softmax: lane holds tokens 16 mt + 4 grp + j of head gi
            float lmax = kNegInf;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int tok = tok0 + 16 * mt + 4 * grp + j;
                    st[mt][j] = tok < ctx ? st[mt][j] * scale_log2 : kNegInf;
                    lmax = fmaxf(lmax, st[mt][j]);
                }
            lmax = fmaxf(lmax, __shfl_xor(lmax, 16));
            const float bmax = fmaxf(lmax, __shfl_xor(lmax, 32));
            if (__builtin_amdgcn_ballot_w64(bmax > m_run + kLSlack) != 0) {
                const float m_new = fmaxf(m_run, bmax);
                const float alpha = exp2_fast(m_run - m_new);
                l_run *= alpha;
                m_run = m_new;
                if (n > 0) {  // before the first block the accumulators are zero
#pragma unroll
                    for (int dt = 0; dt < kDimTiles; ++dt) acc[dt] *= alpha;
                }
            }
            // ---- O^T += V^T . P^T over the 2 token k-steps ----------------------
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                // P^T B operand, k = 8 grp + jj: tokens 32 kk + 4 grp + jj (tile
                // 2 kk) for jj < 4, 32 kk + 16 + 4 grp + jj - 4 (tile 2 kk + 1)
                uint32_t w4[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int mt = 2 * kk + (u >> 1);
                    const float p0 = exp2_fast(st[mt][2 * (u & 1)] - m_run);
                    const float p1 = exp2_fast(st[mt][2 * (u & 1) + 1] - m_run);
                    w4[u] = pack_bf16(p0, p1);
                    l_run += bf16_lo(w4[u]) + bf16_hi(w4[u]);
                }
                const bf16x8_t pf =
                    __builtin_bit_cast(bf16x8_t, u32x4_t{w4[0], w4[1], w4[2], w4[3]});
                const uint32_t row0 = (32 * kk) * (kMainChunks * 16);
#pragma unroll
                for (int d4 = 0; d4 < kDimTiles; d4 += 4) {
                    bf16x8_t a[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int dt = d4 + u;
                        const uint32_t base = slot + v_base[dt & 3] + row0 + 128 * (dt >> 2);
                        const s16x4_t lo = ds_read_tr(base);
                        const s16x4_t hi = ds_read_tr(base + 16 * (kMainChunks * 16));
                        a[u] = __builtin_bit_cast(
                            bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        acc[d4 + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], pf, acc[d4 + u],
                                                                              0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };

        issue(0);
        for (int n = 0; n < nblk; ++n) {
            wait_vmem<0>();   // this wave's rows of block n have landed
            __syncthreads();  // every wave's rows landed; block n - 1 is no longer read
            if (n + 1 < nblk) issue(n + 1);
            const int tok0 = (blk_start + n) * kLBS;
            if (tok0 + kLBS > ctx) {
                // rows at or past the context: zero them so that nothing
                // (NaN included) reaches the products
                const int first = ctx - tok0;
                uint4 *blk = s_ring[n & 1];
                for (int idx = tid; idx < (kLBS - first) * (kMainChunks + kRopeChunks);
                     idx += NW * kWave) {
                    const int t = first + idx / (kMainChunks + kRopeChunks);
                    const int cidx = idx % (kMainChunks + kRopeChunks);
                    const int pos = cidx < kMainChunks
                                        ? t * kMainChunks + cidx
                                        : kMainB / 16 + t * kRopeChunks + (cidx - kMainChunks);
                    blk[pos] = make_uint4(0, 0, 0, 0);
                }
                __syncthreads();
            }
            compute_block(n);
        }

        // ---- this segment's partial -----------------------------------------
        float l_tot = l_run + __shfl_xor(l_run, 16);
        l_tot += __shfl_xor(l_tot, 32);
        const int64_t row = (static_cast<int64_t>(blockIdx.x) + b) * HQ + wave * kHeadsPerWave + gi;
        if (grp == 0) ws_ml[row] = make_float2(m_run, l_tot);
        float *dst = ws_acc + row * kDV + 4 * grp;
#pragma unroll
        for (int dt = 0; dt < kDimTiles; ++dt)
            *reinterpret_cast<f32x4_t *>(dst + 16 * dt) = acc[dt];

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
                       a.block_tables, a.context_lens, scale_log2, s.num_seqs,
                       s.max_blocks_per_seq);
    pa_status st = hip_status(hipGetLastError(), why, "latent partition launch");
    if (st != PA_OK) return st;
    const dim3 grid(s.num_q_heads, s.num_seqs);
    hipLaunchKernelGGL((stream_reduce_kernel<uint16_t, kDV, 4>), grid, dim3(kWave * 4), 0, stream,
                       static_cast<uint16_t *>(a.out), acc, ml, prefix, a.context_lens, s.num_seqs,
                       1, s.num_q_heads, kLBS, waves);
    return hip_status(hipGetLastError(), why, "latent reduce launch");
}

}  // namespace

pa_status launch_latent_decode(const DecodeShape &s, const DecodeArgs &a, const DecodePlan &p,
                               hipStream_t stream, std::string *why) {
    if (s.num_seqs == 0) return PA_OK;
    const float scale_log2 = static_cast<float>(static_cast<double>(a.scale) * 1.4426950408889634);
    switch (s.num_q_heads / kHeadsPerWave) {
        case 1: return enqueue_latent<1>(s, a, p, scale_log2, stream, why);
        case 2: return enqueue_latent<2>(s, a, p, scale_log2, stream, why);
        case 3: return enqueue_latent<3>(s, a, p, scale_log2, stream, why);
        case 4: return enqueue_latent<4>(s, a, p, scale_log2, stream, why);
        case 5: return enqueue_latent<5>(s, a, p, scale_log2, stream, why);
        case 6: return enqueue_latent<6>(s, a, p, scale_log2, stream, why);
        case 7: return enqueue_latent<7>(s, a, p, scale_log2, stream, why);
        default: return enqueue_latent<8>(s, a, p, scale_log2, stream, why);
    }
}

}  // namespace pa
