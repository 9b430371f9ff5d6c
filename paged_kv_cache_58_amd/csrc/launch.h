// Internal launchers shared by the C ABI (api.cpp) and the kernel files.
// No HIP types here: the stream travels as the caller's void * (a
// hipStream_t), so api.cpp and the host checks build with any C++ compiler.
#pragma once

#include <string>

#include "plan.h"

namespace pa {

// Slot-mapped K/V row copy.  Enqueues on `stream`; returns PA_OK or PA_ERR_HIP.
pa_status launch_append(const AppendArgs &a, const AppendPlan &plan, void *stream,
                        std::string *why);

// Grouped-query (and MHA) decode: split-context partition kernel followed by
// the log-sum-exp reduce.
pa_status launch_grouped_decode(const DecodeShape &s, const DecodeArgs &a,
                                const DecodePlan &plan, void *stream, std::string *why);

// The grouped decode with its per-block products on the matrix cores (bf16,
// head dim 128, block size 16); same workspace layout and reduce.
pa_status launch_gqa_mfma_decode(const DecodeShape &s, const DecodeArgs &a,
                                 const DecodePlan &plan, void *stream, std::string *why);

// Quantizing append into MXFP8 caches (one work-group per token and KV head).
pa_status launch_append_mxfp8(const MxAppendArgs &a, void *stream, std::string *why);

// The matrix-core grouped decode over MXFP8 caches, then the stream-K reduce.
pa_status launch_mxfp8_decode(const DecodeShape &s, const DecodeArgs &a,
                              const DecodePlan &plan, void *stream, std::string *why);

// Copies num_pairs whole blocks of block_bytes inside pool (src[i] -> dst[i]).
pa_status launch_copy_blocks(void *pool, int64_t block_bytes, const int32_t *src,
                             const int32_t *dst, int32_t num_pairs, void *stream,
                             std::string *why);

// Per-token attention mass of each KV head's group: scores[b, g, t] =
// sum over the group's query heads h of exp(scale q_h . k_t - lse[b, h]).
pa_status launch_attention_scores(float *scores, const void *q, const void *k_cache,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  const float *lse, float scale, int32_t window, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_blocks_per_seq, int32_t max_context, int32_t dtype,
                                  void *stream, std::string *why);

// Latent (576/512) decode on MFMA, followed by the same stream-K reduce.
pa_status launch_latent_decode(const DecodeShape &s, const DecodeArgs &a,
                               const DecodePlan &plan, void *stream, std::string *why);


// Scratch of pa_decode_noalloc (noalloc.hip): the current device's copy of a
// file-scope device array of kNoAllocScratchBytes, looked up once per device.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
pa_status noalloc_scratch(void **out, std::string *why);

// PA_DEBUG builds only (debug_checks.hip): the device pass over a call's
// index arrays.  Each waits for the stream and returns PA_ERR_INDEX, naming
// the violation, when an index breaks the contract (validate.h).
pa_status debug_check_slots(const int32_t *slots, int32_t n, int64_t num_slots, void *stream,
                            std::string *why);
pa_status debug_check_tables(const int32_t *block_tables, const int32_t *context_lens,
                             int32_t num_seqs, int32_t max_blocks, int32_t block_size,
                             int32_t window, int32_t num_blocks, int64_t cap, void *stream,
                             std::string *why);
pa_status debug_check_copies(const int32_t *src, const int32_t *dst, int32_t n, void *stream,
                             std::string *why);

}  // namespace pa
