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
// One wave per (sequence, KV head, 16-token block), four blocks per
// work-group: lane (token r = lane / 4, quarter c = lane % 4) loads dims
// c*D/4 .. of token r's K row with 16-byte loads and forms the G dot
// products with q over them; two lane exchanges finish each one.  The pass
// reads the window's K rows once (half of the decode's cache bytes).
#include <hip/hip_runtime.h>

#include <cstdint>

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

template <typename T, int D>
__global__ __launch_bounds__(kWave *kScoreWaves) void attention_scores_kernel(
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

template <typename T, int D>
void enqueue_scores(float *scores, const void *q, const void *k_cache, const int32_t *bt,
                    const int32_t *cl, const float *lse, float scale, int window, int num_seqs,
                    int num_kv_heads, int group, int max_blocks, int max_context,
                    hipStream_t stream) {
    const int nblk = (max_context + kSBS - 1) / kSBS;
    const dim3 grid((nblk + kScoreWaves - 1) / kScoreWaves, num_kv_heads, num_seqs);
    const float scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
    hipLaunchKernelGGL((attention_scores_kernel<T, D>), grid, dim3(kWave * kScoreWaves), 0, stream,
                       scores, static_cast<const T *>(q), static_cast<const T *>(k_cache), bt, cl,
                       lse, scale_log2, window, num_kv_heads, group, max_blocks, max_context);
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
