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
// One wave per (sequence, KV head, 16-token block): lane (token r = lane / 4,
// quarter c = lane % 4) holds dims c*D/4 .. of token r's K row and forms the
// G dot products with q over them; two lane exchanges finish each one.  The
// pass reads the window's K rows once (half of the decode's cache bytes).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "hip_util.h"
#include "launch.h"

namespace pa {
namespace {

constexpr int kSBS = 16;  // tokens per cache block

template <typename T>
__device__ __forceinline__ float load_as_f32(const T *p, int i) {
    if constexpr (sizeof(T) == 4) {
        return reinterpret_cast<const float *>(p)[i];
    } else {
        return as_f(static_cast<uint32_t>(reinterpret_cast<const uint16_t *>(p)[i]) << 16);
    }
}

template <typename T, int D>
__global__ __launch_bounds__(kWave) void attention_scores_kernel(
    float *__restrict__ scores, const T *__restrict__ q, const T *__restrict__ k_cache,
    const int32_t *__restrict__ block_tables, const int32_t *__restrict__ context_lens,
    const float *__restrict__ lse, float scale, int window, int num_kv_heads, int group,
    int max_blocks, int max_context) {
    constexpr int DQ = D / 4;  // dims per lane
    const int blk = blockIdx.x;
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int lane = threadIdx.x;
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
    const T *krow = k_cache + ((static_cast<int64_t>(pb) * kSBS + r) * num_kv_heads + g) * D + c * DQ;
    float kv[DQ];
#pragma unroll
    for (int i = 0; i < DQ; ++i) kv[i] = load_as_f32(krow, i);
    float sum = 0.f;
    for (int h = 0; h < group; ++h) {
        const int hq = g * group + h;
        const T *qrow = q + (static_cast<int64_t>(b) * num_q_heads + hq) * D + c * DQ;
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < DQ; ++i) dot = fmaf(load_as_f32(qrow, i), kv[i], dot);
        dot += __shfl_xor(dot, 1);
        dot += __shfl_xor(dot, 2);
        sum += expf(dot * scale - lse[static_cast<int64_t>(b) * num_q_heads + hq]);
    }
    if (c == 0 && t < max_context) row[t] = in ? sum : 0.f;
}

template <typename T, int D>
void enqueue_scores(float *scores, const void *q, const void *k_cache, const int32_t *bt,
                    const int32_t *cl, const float *lse, float scale, int window, int num_seqs,
                    int num_kv_heads, int group, int max_blocks, int max_context,
                    hipStream_t stream) {
    const dim3 grid((max_context + kSBS - 1) / kSBS, num_kv_heads, num_seqs);
    hipLaunchKernelGGL((attention_scores_kernel<T, D>), grid, dim3(kWave), 0, stream, scores,
                       static_cast<const T *>(q), static_cast<const T *>(k_cache), bt, cl, lse,
                       scale, window, num_kv_heads, group, max_blocks, max_context);
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
