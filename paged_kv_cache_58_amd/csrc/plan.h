// Host-side argument checks and launch planning for libpa.
//
// Pure C++ with no HIP headers, so every rule here can be exercised on a host
// without a GPU.  The kernels rely on the shapes these checks admit.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "pa.h"

namespace pa {

struct AppendArgs {
    void *k_cache;
    void *v_cache;
    const void *k;
    int64_t k_token_stride;
    const void *v;
    int64_t v_token_stride;
    const int32_t *slot_mapping;
    int32_t num_tokens;
    int32_t num_blocks;
    int32_t block_size;
    int32_t num_kv_heads;
    int32_t head_dim_k;
    int32_t head_dim_v;
    pa_dtype dtype;
};

// Launch shape of the append copy: the widest vector (bytes) that divides both
// row lengths, both token strides and every base pointer.
struct AppendPlan {
    int vec_bytes;
    int64_t k_row_bytes;
    int64_t v_row_bytes;  // 0 in latent mode
};

pa_status check_append(const AppendArgs &a, AppendPlan *plan, std::string *why);

enum class DecodePath { kGrouped, kLatent };

struct DecodeShape {
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim_k;
    int32_t head_dim_v;
    int32_t block_size;
    int32_t max_blocks_per_seq;
    bool latent;  // v_cache == NULL
    pa_dtype dtype;
};

// Split-context plan: each sequence's context is cut into partitions of
// part_blocks cache blocks; one work-group handles one (partition, KV head,
// sequence) and leaves an unnormalised fp32 accumulator plus (max, sum) in
// the workspace for the log-sum-exp reduce.
struct DecodePlan {
    DecodePath path;
    int group;          // query heads per KV head
    int part_blocks;    // cache blocks per partition
    int num_parts;      // partitions per sequence at max_blocks_per_seq
    size_t acc_offset;  // float [num_seqs, num_q_heads, num_parts, head_dim_v]
    size_t ml_offset;   // float2 [num_seqs, num_q_heads, num_parts] = (max, sum)
    size_t bytes;       // total workspace bytes
};

// Validates the sizes and fills the plan.  Does not look at pointers.
pa_status plan_decode(const DecodeShape &s, DecodePlan *plan, std::string *why);

struct DecodeArgs {
    void *out;
    const void *q;
    const void *k_cache;
    const void *v_cache;
    const int32_t *block_tables;
    const int32_t *context_lens;
    float scale;
    int32_t num_blocks;
    void *workspace;
    size_t workspace_bytes;
};

// Pointer, alignment, scale and workspace checks against a plan.
pa_status check_decode(const DecodeShape &s, const DecodeArgs &a, const DecodePlan &plan,
                       std::string *why);

}  // namespace pa
