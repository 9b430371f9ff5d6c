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
//    (tp = lane / 8, c = lane % 8) loads rows 2tp and 2tp+1, 16-byte chunks
//    c, c+8, ...: every load is a 16-byte global_load_dwordx4 and each group
//    of 8 lanes reads one 128-byte line.
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
//  * P.V: probabilities are rounded to bf16 pairs (tokens 2tp, 2tp+1) and V
//    is staged in LDS as (token 2tp, token 2tp+1) bf16 pairs per dim, so one
//    v_dot2_f32_bf16 applies two tokens to one output dim.  Lane l owns
//    output dims {l * D/64 ...} of all G heads; the fp32 accumulators never
//    leave registers until the partition ends.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "launch.h"

namespace pa {
namespace {

constexpr int kWave = 64;
constexpr int kBS = 16;              // tokens per cache block on this path
constexpr float kSlack = 8.0f;       // lazy-rescale threshold, log2 units
constexpr float kNegInf = -__builtin_huge_valf();

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

// Position of output dim j inside one token pair's row of staged V pairs.
// Dim j = 64 i + 8 c + 4 h + e sits at 64 i + 32 h + 4 c + e, so each
// 16-byte LDS write of the staging lanes (fixed i, h) covers 128 contiguous
// bytes, and the dims a P.V lane reads (2 l, 2 l + 1) are adjacent.
__host__ __device__ constexpr int pair_pos(int j) {
    return ((j >> 6) * 2 + ((j >> 2) & 1)) * 32 + ((j >> 3) & 7) * 4 + (j & 3);
}

template <typename T, int D, int G>
struct Cfg {
    static constexpr bool kBf16 = sizeof(T) == 2;
    static constexpr int kRowBytes = D * static_cast<int>(sizeof(T));
    static constexpr int kChunks = kRowBytes / 16;  // 16-byte chunks per row
    static constexpr int kCPL = kChunks / 8;        // chunks per lane per token
    static constexpr int kDPL = D / kWave;          // output dims per lane
    static constexpr int kRowPad = 4;               // dwords of LDS padding per row
    // bf16: 8 token-pair rows of D pair-dwords; fp32: 16 token rows of D floats
    static constexpr int kVRows = kBf16 ? kBS / 2 : kBS;
    static constexpr int kVStride = D + kRowPad;
    static constexpr int kPWords = kBf16 ? G * 8 : G * 16;
    static_assert(kCPL >= 1 && kChunks % 8 == 0, "row must be a multiple of 128 bytes");
    static_assert(kDPL >= 1, "head dim must be a multiple of 64");
};

template <typename T, int D, int G>
__global__ __launch_bounds__(kWave) void grouped_partition_kernel(
    float *__restrict__ ws_acc, float2 *__restrict__ ws_ml, const T *__restrict__ q,
    const T *__restrict__ k_cache, const T *__restrict__ v_cache,
    const int32_t *__restrict__ block_tables, const int32_t *__restrict__ context_lens,
    float scale_log2, int num_kv_heads, int max_blocks, int part_blocks, int num_parts) {
    using C = Cfg<T, D, G>;
    constexpr int CPL = C::kCPL;
    constexpr int DPL = C::kDPL;

    const int part = blockIdx.x;
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int ctx = context_lens[b];
    const int seq_blocks = (ctx + kBS - 1) / kBS;
    const int blk0 = part * part_blocks;
    if (blk0 >= seq_blocks) return;  // past the end of this sequence
    const int nblk = min(part_blocks, seq_blocks - blk0);

    const int lane = threadIdx.x;
    const int tp = lane >> 3;
    const int c = lane & 7;
    const int hc = c % G;  // the head whose softmax this lane carries
    const int num_q_heads = num_kv_heads * G;

    __shared__ __attribute__((aligned(16))) uint32_t s_v[C::kVRows * C::kVStride];
    __shared__ __attribute__((aligned(16))) uint32_t s_p[C::kPWords];
    __shared__ float s_alpha[8];

    // Physical block ids of this partition: lane n holds entry n.
    const int32_t *bt = block_tables + static_cast<int64_t>(b) * max_blocks + blk0;
    const int my_block = lane < nblk ? bt[lane] : 0;

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
    const int64_t row_stride = static_cast<int64_t>(num_kv_heads) * C::kRowBytes;
    const int64_t blk_stride = kBS * row_stride;
    uint32_t off[2][CPL];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < CPL; ++i)
            off[j][i] = static_cast<uint32_t>((2 * tp + j) * row_stride + g * C::kRowBytes +
                                              (c + 8 * i) * 16);

    const char *kbase = reinterpret_cast<const char *>(k_cache);
    const char *vbase = reinterpret_cast<const char *>(v_cache);

    float m_run = kNegInf;  // running max of head hc (scaled, log2 units)
    float l_run = 0.f;      // this lane's share of the running sum of head hc
    float acc[G][DPL];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int d = 0; d < DPL; ++d) acc[h][d] = 0.f;

    uint4 kbuf[2][2][CPL], vbuf[2][2][CPL];

    auto load_block = [&](int n, uint4 (&kr)[2][CPL], uint4 (&vr)[2][CPL]) {
        const int pb = __builtin_amdgcn_readlane(my_block, n);
        const char *kb = kbase + static_cast<int64_t>(pb) * blk_stride;
        const char *vb = vbase + static_cast<int64_t>(pb) * blk_stride;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                kr[j][i] = *reinterpret_cast<const uint4 *>(kb + off[j][i]);
                vr[j][i] = *reinterpret_cast<const uint4 *>(vb + off[j][i]);
            }
    };

    // Pair-dword position (bf16) of this lane's P.V output dims.
    const int pv_pos = pair_pos(lane * DPL);

    auto compute_block = [&](int n, uint4 (&kr)[2][CPL], uint4 (&vr)[2][CPL]) {
        const int tok0 = (blk0 + n) * kBS;
        const bool partial = tok0 + kBS > ctx;  // only the sequence's last block
        bool valid[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) valid[j] = !partial || (tok0 + 2 * tp + j < ctx);

        // ---- scores for the G heads of both tokens -------------------------
        float s[2][G];
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
                s[j][h] = sum_over_c(a);
            }

        // ---- online softmax for head hc ------------------------------------
        float x[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            float v = s[j][0];
#pragma unroll
            for (int h = 1; h < G; ++h) v = (hc == h) ? s[j][h] : v;
            x[j] = valid[j] ? v * scale_log2 : kNegInf;
        }
        const float xmax = fmaxf(x[0], x[1]);
        if (__builtin_amdgcn_ballot_w64(xmax > m_run + kSlack) != 0) {
            const float bmax = max_over_tp(xmax);
            const float m_new = fmaxf(m_run, bmax);
            const float alpha = exp2_fast(m_run - m_new);
            l_run *= alpha;
            m_run = m_new;
            if (tp == 0 && c < G) s_alpha[c] = alpha;
            __syncthreads();
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float a = s_alpha[h];
#pragma unroll
                for (int d = 0; d < DPL; ++d) acc[h][d] *= a;
            }
        }
        const float p0 = exp2_fast(x[0] - m_run);
        const float p1 = exp2_fast(x[1] - m_run);

        __syncthreads();  // the previous block's LDS reads are done
        if constexpr (C::kBf16) {
            const uint32_t pk = pack_bf16(p0, p1);
            l_run += bf16_lo(pk) + bf16_hi(pk);
            if (c < G) s_p[c * 8 + tp] = pk;
            // ---- stage V as (token 2tp, token 2tp+1) pairs ------------------
            uint4 va[CPL], vb[CPL];
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                va[i] = vr[0][i];
                vb[i] = vr[1][i];
                if (partial) {  // masked rows contribute exactly zero, NaN or not
                    if (!valid[0]) va[i] = make_uint4(0, 0, 0, 0);
                    if (!valid[1]) vb[i] = make_uint4(0, 0, 0, 0);
                }
            }
            uint32_t *row = s_v + tp * C::kVStride;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const uint32_t a0 = va[i].x, a1 = va[i].y, a2 = va[i].z, a3 = va[i].w;
                const uint32_t b0 = vb[i].x, b1 = vb[i].y, b2 = vb[i].z, b3 = vb[i].w;
                uint4 lo, hi;  // dims 0..3 and 4..7 of chunk c + 8 i
                lo.x = __builtin_amdgcn_perm(b0, a0, 0x05040100u);
                lo.y = __builtin_amdgcn_perm(b0, a0, 0x07060302u);
                lo.z = __builtin_amdgcn_perm(b1, a1, 0x05040100u);
                lo.w = __builtin_amdgcn_perm(b1, a1, 0x07060302u);
                hi.x = __builtin_amdgcn_perm(b2, a2, 0x05040100u);
                hi.y = __builtin_amdgcn_perm(b2, a2, 0x07060302u);
                hi.z = __builtin_amdgcn_perm(b3, a3, 0x05040100u);
                hi.w = __builtin_amdgcn_perm(b3, a3, 0x07060302u);
                *reinterpret_cast<uint4 *>(row + (2 * i) * 32 + c * 4) = lo;
                *reinterpret_cast<uint4 *>(row + (2 * i + 1) * 32 + c * 4) = hi;
            }
        } else {
            l_run += p0 + p1;
            if (c < G)
                *reinterpret_cast<float2 *>(&s_p[c * 16 + 2 * tp]) = make_float2(p0, p1);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                uint32_t *row = s_v + (2 * tp + j) * C::kVStride;
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    uint4 v = vr[j][i];
                    if (partial && !valid[j]) v = make_uint4(0, 0, 0, 0);
                    *reinterpret_cast<uint4 *>(row + (c + 8 * i) * 4) = v;
                }
            }
        }
        __syncthreads();

        // ---- P.V for all G heads of this lane's dims -----------------------
        if constexpr (C::kBf16) {
#pragma unroll
            for (int quad = 0; quad < 2; ++quad) {
                uint4 pq[G];
#pragma unroll
                for (int h = 0; h < G; ++h)
                    pq[h] = *reinterpret_cast<const uint4 *>(&s_p[h * 8 + quad * 4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t *row = s_v + (quad * 4 + e) * C::kVStride + pv_pos;
                    uint32_t vp[DPL];
                    if constexpr (DPL == 2) {
                        const uint2 t = *reinterpret_cast<const uint2 *>(row);
                        vp[0] = t.x;
                        vp[1] = t.y;
                    } else {
                        vp[0] = row[0];
                    }
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        const uint32_t ph = e == 0 ? pq[h].x : e == 1 ? pq[h].y
                                          : e == 2 ? pq[h].z : pq[h].w;
#pragma unroll
                        for (int d = 0; d < DPL; ++d) acc[h][d] = dot2_bf16(ph, vp[d], acc[h][d]);
                    }
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < kBS; ++t) {
                const uint32_t *row = s_v + t * C::kVStride + lane * DPL;
                float vv[DPL];
#pragma unroll
                for (int d = 0; d < DPL; ++d) vv[d] = as_f(row[d]);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float ph = as_f(s_p[h * 16 + t]);
#pragma unroll
                    for (int d = 0; d < DPL; ++d) acc[h][d] = fmaf(ph, vv[d], acc[h][d]);
                }
            }
        }
    };

    // Software pipeline: block n+1's loads are in flight while block n computes.
    load_block(0, kbuf[0], vbuf[0]);
    int n = 0;
    for (; n + 2 <= nblk; n += 2) {
        load_block(n + 1, kbuf[1], vbuf[1]);
        compute_block(n, kbuf[0], vbuf[0]);
        if (n + 2 < nblk) load_block(n + 2, kbuf[0], vbuf[0]);
        compute_block(n + 1, kbuf[1], vbuf[1]);
    }
    if (n < nblk) compute_block(n, kbuf[0], vbuf[0]);

    // ---- partition result: unnormalised accumulator, running max and sum ---
    const float l_tot = sum_over_tp(l_run);
    const int64_t row0 = static_cast<int64_t>(b) * num_q_heads + g * G;
    if (tp == 0 && c < G)
        ws_ml[(row0 + c) * num_parts + part] = make_float2(m_run, l_tot);
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float *dst = ws_acc + ((row0 + h) * num_parts + part) * D + lane * DPL;
        if constexpr (DPL == 2)
            *reinterpret_cast<float2 *>(dst) = make_float2(acc[h][0], acc[h][1]);
        else
            dst[0] = acc[h][0];
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

template <typename T, int D, int G>
void enqueue_partition(const DecodeShape &s, const DecodeArgs &a, const DecodePlan &p,
                       float scale_log2, hipStream_t stream) {
    char *ws = static_cast<char *>(a.workspace);
    hipLaunchKernelGGL((grouped_partition_kernel<T, D, G>),
                       dim3(p.num_parts, s.num_kv_heads, s.num_seqs), dim3(kWave), 0, stream,
                       reinterpret_cast<float *>(ws + p.acc_offset),
                       reinterpret_cast<float2 *>(ws + p.ml_offset),
                       static_cast<const T *>(a.q), static_cast<const T *>(a.k_cache),
                       static_cast<const T *>(a.v_cache), a.block_tables, a.context_lens,
                       scale_log2, s.num_kv_heads, s.max_blocks_per_seq, p.part_blocks,
                       p.num_parts);
}

template <typename T, int D>
void enqueue_partition_g(const DecodeShape &s, const DecodeArgs &a, const DecodePlan &p,
                         float scale_log2, hipStream_t stream) {
    switch (p.group) {
        case 1: enqueue_partition<T, D, 1>(s, a, p, scale_log2, stream); break;
        case 2: enqueue_partition<T, D, 2>(s, a, p, scale_log2, stream); break;
        case 4: enqueue_partition<T, D, 4>(s, a, p, scale_log2, stream); break;
        default: enqueue_partition<T, D, 8>(s, a, p, scale_log2, stream); break;
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
        if (s.head_dim_k == 64) enqueue_partition_g<uint16_t, 64>(s, a, p, scale_log2, stream);
        else enqueue_partition_g<uint16_t, 128>(s, a, p, scale_log2, stream);
    } else {
        if (s.head_dim_k == 64) enqueue_partition_g<float, 64>(s, a, p, scale_log2, stream);
        else enqueue_partition_g<float, 128>(s, a, p, scale_log2, stream);
    }
    pa_status st = hip_status(hipGetLastError(), why, "partition launch");
    if (st != PA_OK) return st;
    return launch_lse_reduce(s, a, p, p.part_blocks * kBS, stream, why);
}

}  // namespace pa
