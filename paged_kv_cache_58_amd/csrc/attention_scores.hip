// Per-token attention mass for KV sparsity (gfx950).
//
// The KV-sparsity article ("Comment KV Sparsity permet une accélération de
// 1,5x pour vLLM", "Modification de l'Attention") keeps the row max and sum
// that the attention kernel already has, exports them, and then recomputes
// each cached token's softmax probability p = exp(q.k - rowmax) / l in a
// second, one-pass step; a token's score is a sum of such probabilities, and
// the lowest-scoring K/V are the ones a layer drops.  Here the attention
// kernel exports the log-sum-exp lse = rowmax + log(l) per (sequence, query
// head) (pa_decode_ex), and this kernel computes, for every cached token t of
// the sequence's window,
//     scores[b, g, t] = sum over query heads h of KV head g of exp(s - lse[b, h]),
//     s = scale * q[b, h] . k_t
// i.e. the attention mass the group's heads put on t (K/V are shared per KV
// head, so that is the unit a layer can drop); tokens outside the window or
// past the context score 0.  Each head's probabilities sum to 1, so a
// sequence's scores for a KV head sum to G.
//
// The streaming kernel: one wave per (sequence, KV head, run of 16
// consecutive 16-token blocks; PA_SCORE_RUN sets another run length).  The
// wave loads its slice of q for all G heads once, then streams the run's K
// rows four blocks at a time with non-temporal 16-byte loads (lane (tp =
// lane / 8, c = lane % 8) owns tokens 2tp, 2tp+1, chunks c, c+8, ... of the
// row); each lane forms partial dot products for every head, a DPP
// reduce-scatter leaves lane c with head c's scores, and three more lane
// exchanges sum the heads' probabilities per token.  The pass reads the
// window's K rows once (half of the decode's cache bytes).  Runs of 16
// blocks measured 196.5 us on the 70B-shape batch against 204.5 at 32 and
// 226.8 at 64, and 66.7 against 78.9 us with a 1024-token window (more
// waves share the few blocks a window leaves).  Group sizes other than 1, 2,
// 4, 8, 16 (and fp32 rows of 128 with 16 heads, whose q would not fit in
// registers) take the per-block kernel below, which loads q again for every
// block.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>

#include "device_common.h"
#include "hip_util.h"
#include "launch.h"

namespace pa {
namespace {

constexpr int kSBS = 16;  // tokens per cache block

constexpr int kScoreWaves = 4;  // waves (blocks of 16 tokens) per work-group

// n 16-byte chunks of a row, converted to fp32 (bf16: 8 values a chunk,
// fp32: 4).
template <typename T, int N>
__device__ __forceinline__ void load_row(const T *p, float *out) {
    const uint4 *v = reinterpret_cast<const uint4 *>(p);
    uint4 w[N];
#pragma unroll
    for (int i = 0; i < N; ++i) w[i] = v[i];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const uint32_t u[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (sizeof(T) == 2) {
                out[8 * i + 2 * j] = bf16_lo(u[j]);
                out[8 * i + 2 * j + 1] = bf16_hi(u[j]);
            } else {
                out[4 * i + j] = as_f(u[j]);
            }
        }
    }
}

// ---- streaming kernel -------------------------------------------------------
constexpr int kRunBlocks = 16;  // consecutive blocks one wave scores (PA_SCORE_RUN overrides)

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16 bytes the wave reads once: a non-temporal load (no reuse to keep in the caches).
__device__ __forceinline__ uint4 load_nt(const uint4 *p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <typename T, int D, int G>
struct ScoreCfg {
    static constexpr int kRowBytes = D * static_cast<int>(sizeof(T));
    static constexpr int kCPL = kRowBytes / 16 / 8;  // 16-byte chunks per lane per token
    static constexpr int kGS = G < 8 ? G : 8;        // heads per reduce-scatter set
    static constexpr int kSets = G / kGS;            // 1, or 2 for 16 heads
    static constexpr int kLPH = 8 / kGS;             // lanes of a token pair per head
    // blocks whose K rows a wave loads together (16 or 32 registers each)
    static constexpr int kInFlight = kCPL >= 4 ? 2 : 4;
    static_assert(kCPL >= 1 && kSets * kGS == G, "unsupported shape");
};

// The 8 lanes of a token pair hold partial dot products of one token with
// GS heads, lane c's slot i holding head i ^ hc (hc = c / (8 / GS), the
// head the lane ends with).  Each step pairs lane c with c ^ m (m = 7:
// row_half_mirror, 2: quad_perm 2301, 1: quad_perm 1032), keeps the slots
// whose heads share the lane's bit of hc and adds the partner's copy of the
// same head, which sits at the same slot index on every lane; with one head
// left the remaining steps are plain all-reduce adds.
template <int GS>
__device__ __forceinline__ float scatter_heads(const float (&a)[GS]) {
    if constexpr (GS == 8) {
        float r1[4], r2[2];
#pragma unroll
        for (int i = 0; i < 4; ++i) r1[i] = a[i] + dpp<0x141>(a[i ^ 7]);
#pragma unroll
        for (int i = 0; i < 2; ++i) r2[i] = r1[i] + dpp<0x4E>(r1[i ^ 2]);
        return r2[0] + dpp<0xB1>(r2[1]);
    } else if constexpr (GS == 4) {
        float r1[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) r1[i] = a[i] + dpp<0x141>(a[i ^ 3]);
        const float r2 = r1[0] + dpp<0x4E>(r1[1]);
        return r2 + dpp<0xB1>(r2);
    } else if constexpr (GS == 2) {
        float r1 = a[0] + dpp<0x141>(a[1]);
        r1 += dpp<0x4E>(r1);
        return r1 + dpp<0xB1>(r1);
    } else {
        float x = a[0] + dpp<0x141>(a[0]);
        x += dpp<0x4E>(x);
        return x + dpp<0xB1>(x);
    }
}

// Sum over the 8 lanes of a token pair.
__device__ __forceinline__ float sum8(float x) {
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    return x + dpp<0x141>(x);
}

template <typename T, int D, int G>
__global__ __launch_bounds__(kWave *kScoreWaves) void attention_scores_kernel(
    float *__restrict__ scores, const T *__restrict__ q, const T *__restrict__ k_cache,
    const int32_t *__restrict__ block_tables, const int32_t *__restrict__ context_lens,
    const float *__restrict__ lse, float scale_log2, int window, int num_kv_heads,
    int max_blocks, int max_context, int run_blocks) {
    using C = ScoreCfg<T, D, G>;
    constexpr int CPL = C::kCPL;
    constexpr int GS = C::kGS;
    constexpr int kInFlight = C::kInFlight;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = static_cast<int>(threadIdx.x / kWave);
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int k0 = (static_cast<int>(blockIdx.x) * kScoreWaves + wave) * run_blocks;
    const int nblk = (max_context + kSBS - 1) / kSBS;
    if (k0 >= nblk) return;
    const int kend = min(k0 + run_blocks, nblk);
    const int L = context_lens[b];
    const int start = window_start(L, window);
    // blocks of this run holding a scored token: [lo, hi)
    const int lo = max(start / kSBS, k0);
    const int hi = min((L + kSBS - 1) / kSBS, kend);
    float *row = scores + (static_cast<int64_t>(b) * num_kv_heads + g) * max_context;
    const int tend = min(kend * kSBS, max_context);
    for (int t = k0 * kSBS + lane; t < tend; t += kWave)
        if (t < lo * kSBS || t >= hi * kSBS) row[t] = 0.f;
    if (lo >= hi) return;

    const int tp = lane >> 3;
    const int c = lane & 7;
    const int hc = c / C::kLPH;
    const bool head_writer = (c % C::kLPH) == 0;
    const int num_q_heads = num_kv_heads * G;

    // q: chunk c + 8 i of head s GS + (slot ^ hc), for every set s and slot
    uint4 qv[C::kSets][GS][CPL];
    float lse2[C::kSets];  // lse of the lane's heads, in log2 units
    {
        const T *qb = q + (static_cast<int64_t>(b) * num_q_heads + g * G) * D;
#pragma unroll
        for (int st = 0; st < C::kSets; ++st) {
#pragma unroll
            for (int i = 0; i < GS; ++i) {
                const uint4 *qr = reinterpret_cast<const uint4 *>(qb + (st * GS + (i ^ hc)) * D);
#pragma unroll
                for (int ch = 0; ch < CPL; ++ch) qv[st][i][ch] = qr[c + 8 * ch];
            }
            lse2[st] = lse[static_cast<int64_t>(b) * num_q_heads + g * G + st * GS + hc] *
                       1.4426950408889634f;
        }
    }
    const int32_t *bt = block_tables + static_cast<int64_t>(b) * max_blocks;
    const int64_t row_elems = static_cast<int64_t>(num_kv_heads) * D;

    for (int k = lo; k < hi; k += kInFlight) {
        // K rows of blocks k .. k + kInFlight - 1 (past hi: block hi - 1 again)
        uint4 kr[kInFlight][2][CPL];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
            const int pb = bt[min(k + u, hi - 1)];
            const T *base = k_cache + (static_cast<int64_t>(pb) * kSBS + 2 * tp) * row_elems + g * D;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint4 *r = reinterpret_cast<const uint4 *>(base + j * row_elems);
#pragma unroll
                for (int ch = 0; ch < CPL; ++ch) kr[u][j][ch] = load_nt(r + c + 8 * ch);
            }
        }
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
            float mass[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                mass[j] = 0.f;
#pragma unroll
                for (int st = 0; st < C::kSets; ++st) {
                    float part[GS];
#pragma unroll
                    for (int i = 0; i < GS; ++i) {
                        float a = 0.f;
#pragma unroll
                        for (int ch = 0; ch < CPL; ++ch) {
                            const uint4 qq = qv[st][i][ch], kk = kr[u][j][ch];
                            if constexpr (sizeof(T) == 2) {
                                a = dot2_bf16(qq.x, kk.x, a);
                                a = dot2_bf16(qq.y, kk.y, a);
                                a = dot2_bf16(qq.z, kk.z, a);
                                a = dot2_bf16(qq.w, kk.w, a);
                            } else {
                                a = fmaf(as_f(qq.x), as_f(kk.x), a);
                                a = fmaf(as_f(qq.y), as_f(kk.y), a);
                                a = fmaf(as_f(qq.z), as_f(kk.z), a);
                                a = fmaf(as_f(qq.w), as_f(kk.w), a);
                            }
                        }
                        part[i] = a;
                    }
                    const float dot = scatter_heads<GS>(part);
                    // exp(scale q.k - lse) = 2^(scale log2(e) q.k - lse log2(e))
                    const float p = exp2_fast(fmaf(dot, scale_log2, -lse2[st]));
                    mass[j] += head_writer ? p : 0.f;
                }
                mass[j] = sum8(mass[j]);
            }
            const int kb = k + u;
            if (kb < hi && c == 0) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int t = kb * kSBS + 2 * tp + j;
                    if (t < max_context) row[t] = (t >= start && t < L) ? mass[j] : 0.f;
                }
            }
        }
    }
}

// ---- per-block kernel (other group sizes) ----------------------------------
// One wave per (sequence, KV head, 16-token block), four blocks per
// work-group: lane (token r = lane / 4, quarter c = lane % 4) loads dims
// c*D/4 .. of token r's K row with 16-byte loads and forms the G dot
// products with q over them; two lane exchanges finish each one.
template <typename T, int D>
__global__ __launch_bounds__(kWave *kScoreWaves) void attention_scores_block_kernel(
    float *__restrict__ scores, const T *__restrict__ q, const T *__restrict__ k_cache,
    const int32_t *__restrict__ block_tables, const int32_t *__restrict__ context_lens,
    const float *__restrict__ lse, float scale_log2, int window, int num_kv_heads, int group,
    int max_blocks, int max_context) {
    constexpr int DQ = D / 4;                              // dims per lane
    constexpr int NCH = DQ * static_cast<int>(sizeof(T)) / 16;  // 16-byte chunks per lane
    const int lane = threadIdx.x & (kWave - 1);
    const int blk = blockIdx.x * kScoreWaves + static_cast<int>(threadIdx.x / kWave);
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int r = lane >> 2;
    const int c = lane & 3;
    const int t = blk * kSBS + r;
    if (blk * kSBS >= max_context) return;
    const int L = context_lens[b];
    const int start = window_start(L, window);
    const int num_q_heads = num_kv_heads * group;
    float *row = scores + (static_cast<int64_t>(b) * num_kv_heads + g) * max_context;
    const bool in = t >= start && t < L;
    if (__builtin_amdgcn_ballot_w64(in) == 0) {  // no scored token in this block
        if (c == 0 && t < max_context) row[t] = 0.f;
        return;
    }
    const int pb = block_tables[static_cast<int64_t>(b) * max_blocks + blk];
    float kv[DQ];
    load_row<T, NCH>(k_cache + ((static_cast<int64_t>(pb) * kSBS + r) * num_kv_heads + g) * D + c * DQ,
                     kv);
    const float *lse_b = lse + static_cast<int64_t>(b) * num_q_heads + g * group;
    const T *q_g = q + (static_cast<int64_t>(b) * num_q_heads + g * group) * D + c * DQ;
    float sum = 0.f;
    for (int h = 0; h < group; ++h) {
        float qv[DQ];
        load_row<T, NCH>(q_g + static_cast<int64_t>(h) * D, qv);
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < DQ; ++i) dot = fmaf(qv[i], kv[i], dot);
        dot += __shfl_xor(dot, 1);
        dot += __shfl_xor(dot, 2);
        // exp(scale q.k - lse) = 2^(scale log2(e) q.k - lse log2(e))
        sum += exp2_fast(fmaf(dot, scale_log2, -lse_b[h] * 1.4426950408889634f));
    }
    if (c == 0 && t < max_context) row[t] = in ? sum : 0.f;
}

template <typename T, int D, int G>
void enqueue_stream(float *scores, const void *q, const void *k_cache, const int32_t *bt,
                    const int32_t *cl, const float *lse, float scale_log2, int window,
                    int num_seqs, int num_kv_heads, int max_blocks, int max_context,
                    hipStream_t stream) {
    const int nblk = (max_context + kSBS - 1) / kSBS;
    int run = kRunBlocks;
    if (const char *env = std::getenv("PA_SCORE_RUN")) {
        const int v = std::atoi(env);
        if (v >= 1 && v <= 4096) run = v;
    }
    const int runs = (nblk + run - 1) / run;
    const dim3 grid((runs + kScoreWaves - 1) / kScoreWaves, num_kv_heads, num_seqs);
    hipLaunchKernelGGL((attention_scores_kernel<T, D, G>), grid, dim3(kWave * kScoreWaves), 0,
                       stream, scores, static_cast<const T *>(q), static_cast<const T *>(k_cache),
                       bt, cl, lse, scale_log2, window, num_kv_heads, max_blocks, max_context, run);
}

template <typename T, int D>
void enqueue_scores(float *scores, const void *q, const void *k_cache, const int32_t *bt,
                    const int32_t *cl, const float *lse, float scale, int window, int num_seqs,
                    int num_kv_heads, int group, int max_blocks, int max_context,
                    hipStream_t stream) {
    const float scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
    switch (group) {
        case 1: return enqueue_stream<T, D, 1>(scores, q, k_cache, bt, cl, lse, scale_log2, window,
                                               num_seqs, num_kv_heads, max_blocks, max_context, stream);
        case 2: return enqueue_stream<T, D, 2>(scores, q, k_cache, bt, cl, lse, scale_log2, window,
                                               num_seqs, num_kv_heads, max_blocks, max_context, stream);
        case 4: return enqueue_stream<T, D, 4>(scores, q, k_cache, bt, cl, lse, scale_log2, window,
                                               num_seqs, num_kv_heads, max_blocks, max_context, stream);
        case 8: return enqueue_stream<T, D, 8>(scores, q, k_cache, bt, cl, lse, scale_log2, window,
                                               num_seqs, num_kv_heads, max_blocks, max_context, stream);
        case 16:
            // 16 heads of fp32 rows of 128 would hold 256 registers of q
            if constexpr (sizeof(T) == 2 || D == 64)
                return enqueue_stream<T, D, 16>(scores, q, k_cache, bt, cl, lse, scale_log2,
                                                window, num_seqs, num_kv_heads, max_blocks,
                                                max_context, stream);
            break;
        default: break;
    }
    const int nblk = (max_context + kSBS - 1) / kSBS;
    const dim3 grid((nblk + kScoreWaves - 1) / kScoreWaves, num_kv_heads, num_seqs);
    hipLaunchKernelGGL((attention_scores_block_kernel<T, D>), grid, dim3(kWave * kScoreWaves), 0,
                       stream, scores, static_cast<const T *>(q), static_cast<const T *>(k_cache),
                       bt, cl, lse, scale_log2, window, num_kv_heads, group, max_blocks,
                       max_context);
}

}  // namespace

pa_status launch_attention_scores(float *scores, const void *q, const void *k_cache,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  const float *lse, float scale, int32_t window, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_blocks_per_seq, int32_t max_context, int32_t dtype,
                                  void *stream_arg, std::string *why) {
    const hipStream_t stream = static_cast<hipStream_t>(stream_arg);
    const int group = num_q_heads / num_kv_heads;
    if (dtype == PA_BF16) {
        if (head_dim == 64)
            enqueue_scores<uint16_t, 64>(scores, q, k_cache, block_tables, context_lens, lse, scale,
                                         window, num_seqs, num_kv_heads, group, max_blocks_per_seq,
                                         max_context, stream);
        else
            enqueue_scores<uint16_t, 128>(scores, q, k_cache, block_tables, context_lens, lse,
                                          scale, window, num_seqs, num_kv_heads, group,
                                          max_blocks_per_seq, max_context, stream);
    } else {
        if (head_dim == 64)
            enqueue_scores<float, 64>(scores, q, k_cache, block_tables, context_lens, lse, scale,
                                      window, num_seqs, num_kv_heads, group, max_blocks_per_seq,
                                      max_context, stream);
        else
            enqueue_scores<float, 128>(scores, q, k_cache, block_tables, context_lens, lse, scale,
                                       window, num_seqs, num_kv_heads, group, max_blocks_per_seq,
                                       max_context, stream);
    }
    return hip_status(hipGetLastError(), why, "attention scores launch");
}

}  // namespace pa
