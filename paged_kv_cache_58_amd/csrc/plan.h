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
    int32_t dtype;  // a pa_dtype value, kept as an integer until validated
};

// Launch shape of the append copy: the widest vector (bytes) that divides both
// row lengths, both token strides and every base pointer.
struct AppendPlan {
    int vec_bytes;
    int64_t k_row_bytes;
    int64_t v_row_bytes;  // 0 in latent mode
};

pa_status check_append(const AppendArgs &a, AppendPlan *plan, std::string *why);

// MXFP8 caches (E4M3 codes with one E8M0 scale per 32 values of a head row):
// K codes [num_blocks, Hkv, bs, d], V codes [num_blocks, Hkv, d, bs], scales
// [num_blocks, Hkv, bs, d / 32].  The append quantizes fp32 or bf16 rows.
constexpr int kMxHeadDim = 128;  // head dim the MXFP8 kernels run
constexpr int kMxBlock = 32;     // values per E8M0 scale
struct MxAppendArgs {
    void *k_cache;
    void *v_cache;
    void *k_scale;
    void *v_scale;
    const void *k;
    int64_t k_token_stride;
    const void *v;
    int64_t v_token_stride;
    const int32_t *slot_mapping;
    int32_t num_tokens;
    int32_t num_blocks;
    int32_t block_size;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t dtype;  // of k and v (a pa_dtype value, kept as an integer until validated)
};

pa_status check_append_mxfp8(const MxAppendArgs &a, std::string *why);

// kGrouped: VALU dot products; kGroupedMfma: the same split and partials with
// the per-block products on the matrix cores (bf16, head dim 128); kMxfp8: that
// matrix-core kernel reading MXFP8 caches.
enum class DecodePath { kGrouped, kGroupedMfma, kMxfp8, kLatent };

// Most work-groups the grouped path's stream-K partition kernel launches
// (one per resident wave slot; 256 CUs x 16 waves), which sizes its
// workspace: a partial slot per work-group plus one per (sequence, KV head).
constexpr int kStreamWavesMax = 4096;

// Most work-groups of the latent path (one per CU; each covers every query
// head of a block), which sizes its workspace the same way.
constexpr int kLatentWavesMax = 512;
// Query heads one wave of the latent path covers in its scores.
constexpr int kLatentHeadTile = 32;
// Score tiles of 32 query heads in a latent work-group, rounded up to 1, 2 or
// 4 (its four waves split each tile's score contraction 4, 2 or 1 ways).
inline int latent_head_tiles(int num_q_heads) {
    return num_q_heads <= kLatentHeadTile ? 1 : num_q_heads <= 2 * kLatentHeadTile ? 2 : 4;
}

struct DecodeShape {
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim_k;
    int32_t head_dim_v;
    int32_t block_size;
    int32_t max_blocks_per_seq;
    bool latent;  // v_cache == NULL
    bool mxfp8;   // MXFP8 caches (dtype is then that of q and out)
    int32_t dtype;  // a pa_dtype value, kept as an integer until validated
    int32_t q_len = 1;  // new query tokens per sequence, causal among themselves
    int32_t window = 0; // > 0: attend only to the last `window` tokens (sliding window)
};

// Most (query, head) columns one KV head's work may carry on the matrix-core
// grouped kernel: G * q_len <= 16 * kMaxColTiles.
constexpr int kMaxColTiles = 4;

// Split-context plan.  Both paths leave, per partial result and query head,
// an unnormalised fp32 accumulator plus (max, sum) in the workspace for the
// log-sum-exp reduce.
//  * grouped: stream-K; slots = kStreamWavesMax + num_seqs * num_kv_heads,
//    each holding the G heads of one KV group; plus the per-sequence block
//    prefix sums (num_seqs + 1 int32) the partition kernel leaves for the
//    reduce.
//  * latent: each sequence cut into parts of near-equal size, one
//    work-group per part (at least one per CU, at least one per sequence);
//    slots = kLatentWavesMax + num_seqs (more than the work-groups), each
//    holding latent_head_tiles(num_q_heads) * 32 heads (the query heads,
//    padded); the prefix array holds the parts per sequence (num_seqs + 1).
//    There a slot holds the part's output divided by its sum l, in fp32, in
//    the partition kernel's register order (HT = latent_head_tiles:
//    16-byte index ((dt * HT + ht) * 4 + qd) * 64 + lane holds dims 32 dt +
//    8 qd + 4 (lane >> 5) .. + 3 of head 32 ht + (lane & 31)), and (max,
//    sum) in fp32.
struct DecodePlan {
    DecodePath path;
    int group;             // query heads per KV head
    int ring_depth;        // grouped path: cache blocks streaming into LDS per wave (2 or 4)
    size_t acc_offset;     // float [slots, heads per slot, head_dim_v]
    size_t ml_offset;      // float2 [slots, heads per slot] = (max, sum)
    size_t prefix_offset;  // grouped path: int32 [num_seqs + 1]
    size_t bytes;          // total workspace bytes
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
    const void *k_scale;  // MXFP8 caches only
    const void *v_scale;
    float scale;
    int32_t num_blocks;
    void *workspace;
    size_t workspace_bytes;
    float *lse = nullptr;  // optional [num_seqs, q_len, num_q_heads] log-sum-exp output
};

// Pointer, alignment, scale and workspace checks against a plan.
pa_status check_decode(const DecodeShape &s, const DecodeArgs &a, const DecodePlan &plan,
                       std::string *why);

}  // namespace pa
