// Internal launchers shared by the C ABI (api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include <string>

#include "plan.h"

namespace pa {

// Slot-mapped K/V row copy.  Enqueues on `stream`; returns PA_OK or PA_ERR_HIP.
pa_status launch_append(const AppendArgs &a, const AppendPlan &plan, hipStream_t stream,
                        std::string *why);

// Grouped-query (and MHA) decode: split-context partition kernel followed by
// the log-sum-exp reduce.
pa_status launch_grouped_decode(const DecodeShape &s, const DecodeArgs &a,
                                const DecodePlan &plan, hipStream_t stream, std::string *why);

// The grouped decode with its per-block products on the matrix cores (bf16,
// head dim 128, block size 16); same workspace layout and reduce.
pa_status launch_gqa_mfma_decode(const DecodeShape &s, const DecodeArgs &a,
                                 const DecodePlan &plan, hipStream_t stream, std::string *why);

// Quantizing append into MXFP8 caches (one work-group per token and KV head).
pa_status launch_append_mxfp8(const MxAppendArgs &a, hipStream_t stream, std::string *why);

// The matrix-core grouped decode over MXFP8 caches, then the stream-K reduce.
pa_status launch_mxfp8_decode(const DecodeShape &s, const DecodeArgs &a,
                              const DecodePlan &plan, hipStream_t stream, std::string *why);

// Copies num_pairs whole blocks of block_bytes inside pool (src[i] -> dst[i]).
pa_status launch_copy_blocks(void *pool, int64_t block_bytes, const int32_t *src,
                             const int32_t *dst, int32_t num_pairs, hipStream_t stream,
                             std::string *why);

// Per-token attention mass of each KV head's group: scores[b, g, t] =
// sum over the group's query heads h of exp(scale q_h . k_t - lse[b, h]).
pa_status launch_attention_scores(float *scores, const void *q, const void *k_cache,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  const float *lse, float scale, int32_t window, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_blocks_per_seq, int32_t max_context, pa_dtype dtype,
                                  hipStream_t stream, std::string *why);

// Latent (576/512) decode on MFMA, followed by the same stream-K reduce.
pa_status launch_latent_decode(const DecodeShape &s, const DecodeArgs &a,
                               const DecodePlan &plan, hipStream_t stream, std::string *why);

inline pa_status hip_status(hipError_t e, std::string *why, const char *where) {
    if (e == hipSuccess) return PA_OK;
    if (why) *why = std::string(where) + ": " + hipGetErrorString(e);
    return PA_ERR_HIP;
}

}  // namespace pa
