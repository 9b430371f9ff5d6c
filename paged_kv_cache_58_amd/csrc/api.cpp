// C ABI of libpa.so (declared in include/pa.h): argument checks, planning and
// kernel launches on the caller's stream.  Only the pa_* symbols are exported.
#include <climits>
#include <string>

#include "launch.h"
#include "pa.h"
#include "plan.h"

#define PA_EXPORT extern "C" __attribute__((visibility("default")))

// PA_DEBUG builds check the call's index arrays on the device first (and
// return PA_ERR_INDEX on a violation); release builds compile this to nothing.
#ifdef PA_DEBUG
#define PA_DEBUG_CHECK(call)                                  \
    do {                                                      \
        std::string dbg_why;                                  \
        const pa_status dbg_st = (call);                      \
        if (dbg_st != PA_OK) return finish(dbg_st, dbg_why);  \
    } while (0)
#else
#define PA_DEBUG_CHECK(call) \
    do {                     \
    } while (0)
#endif

namespace {

thread_local std::string g_last_error;

pa_status finish(pa_status st, const std::string &why) {
    g_last_error = st == PA_OK ? std::string() : why;
    return st;
}

pa::DecodeShape make_shape(bool latent, int32_t num_seqs, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim_k, int32_t head_dim_v,
                           int32_t block_size, int32_t max_blocks_per_seq, int32_t dtype) {
    pa::DecodeShape s{};
    s.num_seqs = num_seqs;
    s.num_q_heads = num_q_heads;
    s.num_kv_heads = num_kv_heads;
    s.head_dim_k = head_dim_k;
    s.head_dim_v = head_dim_v;
    s.block_size = block_size;
    s.max_blocks_per_seq = max_blocks_per_seq;
    s.latent = latent;
    s.dtype = dtype;
    return s;
}

}  // namespace

PA_EXPORT pa_status pa_cache_append(void *k_cache, void *v_cache, const void *k,
                                    int64_t k_token_stride, const void *v,
                                    int64_t v_token_stride, const int32_t *slot_mapping,
                                    int32_t num_tokens, int32_t num_blocks, int32_t block_size,
                                    int32_t num_kv_heads, int32_t head_dim_k,
                                    int32_t head_dim_v, pa_dtype dtype, void *stream) {
    pa::AppendArgs a{k_cache, v_cache, k, k_token_stride, v, v_token_stride, slot_mapping,
                     num_tokens, num_blocks, block_size, num_kv_heads, head_dim_k,
                     head_dim_v, dtype};
    std::string why;
    pa::AppendPlan plan{};
    pa_status st = pa::check_append(a, &plan, &why);
    if (st != PA_OK || num_tokens == 0) return finish(st, why);
    PA_DEBUG_CHECK(pa::debug_check_slots(slot_mapping, num_tokens,
                                         static_cast<int64_t>(num_blocks) * block_size, stream,
                                         &dbg_why));
    st = pa::launch_append(a, plan, stream, &why);
    return finish(st, why);
}

PA_EXPORT size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                          int32_t num_kv_heads, int32_t head_dim_k,
                                          int32_t head_dim_v, int32_t block_size,
                                          int32_t max_blocks_per_seq) {
    // Latent mode is the only shape with head_dim_v != head_dim_k (the plan
    // rejects any unequal pair but 576 / 512, so nothing else is planned as latent).
    const bool latent = head_dim_k != head_dim_v;
    const pa::DecodeShape s = make_shape(latent, num_seqs, num_q_heads, num_kv_heads,
                                         head_dim_k, head_dim_v, block_size,
                                         max_blocks_per_seq, PA_BF16);
    pa::DecodePlan plan{};
    if (pa::plan_decode(s, &plan, nullptr) != PA_OK) return 0;
    return plan.bytes;
}

PA_EXPORT pa_status pa_decode(void *out, const void *q, const void *k_cache,
                              const void *v_cache, const int32_t *block_tables,
                              const int32_t *context_lens, float scale, int32_t num_seqs,
                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim_k,
                              int32_t head_dim_v, int32_t block_size, int32_t num_blocks,
                              int32_t max_blocks_per_seq, pa_dtype dtype, void *workspace,
                              size_t workspace_bytes, void *stream) {
    const pa::DecodeShape s =
        make_shape(v_cache == nullptr, num_seqs, num_q_heads, num_kv_heads, head_dim_k,
                   head_dim_v, block_size, max_blocks_per_seq, dtype);
    std::string why;
    pa::DecodePlan plan{};
    pa_status st = pa::plan_decode(s, &plan, &why);
    if (st != PA_OK) return finish(st, why);
    const pa::DecodeArgs a{out, q, k_cache, v_cache, block_tables, context_lens, nullptr,
                           nullptr, scale, num_blocks, workspace, workspace_bytes};
    st = pa::check_decode(s, a, plan, &why);
    if (st != PA_OK || num_seqs == 0) return finish(st, why);
    PA_DEBUG_CHECK(pa::debug_check_tables(block_tables, context_lens, num_seqs,
                                          max_blocks_per_seq, block_size, 0, num_blocks,
                                          static_cast<int64_t>(max_blocks_per_seq) * block_size,
                                          stream, &dbg_why));
    if (plan.path == pa::DecodePath::kLatent)
        st = pa::launch_latent_decode(s, a, plan, stream, &why);
    else if (plan.path == pa::DecodePath::kGroupedMfma)
        st = pa::launch_gqa_mfma_decode(s, a, plan, stream, &why);
    else
        st = pa::launch_grouped_decode(s, a, plan, stream, &why);
    return finish(st, why);
}

PA_EXPORT pa_status pa_decode_noalloc(void *out, const void *q, const void *k_cache,
                                      const void *v_cache, const int32_t *block_tables,
                                      const int32_t *context_lens, float scale, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim_k, int32_t head_dim_v, int32_t block_size,
                                      int32_t num_blocks, int32_t max_blocks_per_seq,
                                      pa_dtype dtype, void *stream) {
    const pa::DecodeShape s =
        make_shape(v_cache == nullptr, num_seqs, num_q_heads, num_kv_heads, head_dim_k,
                   head_dim_v, block_size, max_blocks_per_seq, dtype);
    std::string why;
    pa::DecodePlan plan{};
    pa_status st = pa::plan_decode(s, &plan, &why);
    if (st != PA_OK) return finish(st, why);
    if (plan.bytes > pa::kNoAllocScratchBytes)
        return finish(PA_ERR_WORKSPACE,
                      "decode_noalloc: these sizes need " + std::to_string(plan.bytes) +
                          " bytes of scratch, more than the " +
                          std::to_string(pa::kNoAllocScratchBytes) +
                          " the library holds per GPU; call pa_decode with a workspace");
    if (num_seqs == 0) return finish(PA_OK, why);
    void *scratch = nullptr;
    st = pa::noalloc_scratch(&scratch, &why);
    if (st != PA_OK) return finish(st, why);
    const pa::DecodeArgs a{out, q, k_cache, v_cache, block_tables, context_lens, nullptr,
                           nullptr, scale, num_blocks, scratch, pa::kNoAllocScratchBytes};
    st = pa::check_decode(s, a, plan, &why);
    if (st != PA_OK) return finish(st, why);
    PA_DEBUG_CHECK(pa::debug_check_tables(block_tables, context_lens, num_seqs,
                                          max_blocks_per_seq, block_size, 0, num_blocks,
                                          static_cast<int64_t>(max_blocks_per_seq) * block_size,
                                          stream, &dbg_why));
    if (plan.path == pa::DecodePath::kLatent)
        st = pa::launch_latent_decode(s, a, plan, stream, &why);
    else if (plan.path == pa::DecodePath::kGroupedMfma)
        st = pa::launch_gqa_mfma_decode(s, a, plan, stream, &why);
    else
        st = pa::launch_grouped_decode(s, a, plan, stream, &why);
    return finish(st, why);
}

PA_EXPORT pa_status pa_cache_append_mxfp8(void *k_cache, void *v_cache, void *k_scale,
                                          void *v_scale, const void *k, int64_t k_token_stride,
                                          const void *v, int64_t v_token_stride,
                                          const int32_t *slot_mapping, int32_t num_tokens,
                                          int32_t num_blocks, int32_t block_size,
                                          int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype,
                                          void *stream) {
    const pa::MxAppendArgs a{k_cache, v_cache, k_scale, v_scale, k, k_token_stride, v,
                             v_token_stride, slot_mapping, num_tokens, num_blocks, block_size,
                             num_kv_heads, head_dim, dtype};
    std::string why;
    pa_status st = pa::check_append_mxfp8(a, &why);
    if (st != PA_OK || num_tokens == 0) return finish(st, why);
    PA_DEBUG_CHECK(pa::debug_check_slots(slot_mapping, num_tokens,
                                         static_cast<int64_t>(num_blocks) * block_size, stream,
                                         &dbg_why));
    st = pa::launch_append_mxfp8(a, stream, &why);
    return finish(st, why);
}

PA_EXPORT pa_status pa_decode_mxfp8(void *out, const void *q, const void *k_cache,
                                    const void *v_cache, const void *k_scale,
                                    const void *v_scale, const int32_t *block_tables,
                                    const int32_t *context_lens, float scale, int32_t num_seqs,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int32_t num_blocks,
                                    int32_t max_blocks_per_seq, pa_dtype dtype, void *workspace,
                                    size_t workspace_bytes, void *stream) {
    pa::DecodeShape s = make_shape(false, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                   head_dim, block_size, max_blocks_per_seq, dtype);
    s.mxfp8 = true;
    std::string why;
    pa::DecodePlan plan{};
    pa_status st = pa::plan_decode(s, &plan, &why);
    if (st != PA_OK) return finish(st, why);
    const pa::DecodeArgs a{out, q, k_cache, v_cache, block_tables, context_lens, k_scale,
                           v_scale, scale, num_blocks, workspace, workspace_bytes};
    st = pa::check_decode(s, a, plan, &why);
    if (st != PA_OK || num_seqs == 0) return finish(st, why);
    PA_DEBUG_CHECK(pa::debug_check_tables(block_tables, context_lens, num_seqs,
                                          max_blocks_per_seq, block_size, 0, num_blocks,
                                          static_cast<int64_t>(max_blocks_per_seq) * block_size,
                                          stream, &dbg_why));
    st = pa::launch_mxfp8_decode(s, a, plan, stream, &why);
    return finish(st, why);
}

PA_EXPORT size_t pa_decode_multi_workspace_size(int32_t num_seqs, int32_t q_len,
                                                int32_t num_q_heads, int32_t num_kv_heads,
                                                int32_t head_dim, int32_t block_size,
                                                int32_t max_blocks_per_seq) {
    pa::DecodeShape s = make_shape(false, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                   head_dim, block_size, max_blocks_per_seq, PA_BF16);
    s.q_len = q_len;
    pa::DecodePlan plan{};
    if (pa::plan_decode(s, &plan, nullptr) != PA_OK) return 0;
    return plan.bytes;
}

PA_EXPORT pa_status pa_decode_multi(void *out, const void *q, const void *k_cache,
                                    const void *v_cache, const void *k_scale,
                                    const void *v_scale, const int32_t *block_tables,
                                    const int32_t *context_lens, float scale, int32_t num_seqs,
                                    int32_t q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                    int32_t max_blocks_per_seq, pa_dtype dtype, void *workspace,
                                    size_t workspace_bytes, void *stream) {
    std::string why;
    if ((k_scale == nullptr) != (v_scale == nullptr))
        return finish(PA_ERR_NULL, "decode (several queries): k_scale and v_scale must both be "
                                   "NULL (bf16 caches) or both set (MXFP8 caches)");
    pa::DecodeShape s = make_shape(false, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                   head_dim, block_size, max_blocks_per_seq, dtype);
    s.mxfp8 = k_scale != nullptr;
    s.q_len = q_len;
    pa::DecodePlan plan{};
    pa_status st = pa::plan_decode(s, &plan, &why);
    if (st != PA_OK) return finish(st, why);
    if (!v_cache && num_seqs > 0)
        return finish(PA_ERR_NULL, "decode (several queries): v_cache must be non-NULL");
    const pa::DecodeArgs a{out, q, k_cache, v_cache, block_tables, context_lens, k_scale,
                           v_scale, scale, num_blocks, workspace, workspace_bytes};
    st = pa::check_decode(s, a, plan, &why);
    if (st != PA_OK || num_seqs == 0) return finish(st, why);
    PA_DEBUG_CHECK(pa::debug_check_tables(block_tables, context_lens, num_seqs,
                                          max_blocks_per_seq, block_size, 0, num_blocks,
                                          static_cast<int64_t>(max_blocks_per_seq) * block_size,
                                          stream, &dbg_why));
    st = s.mxfp8 ? pa::launch_mxfp8_decode(s, a, plan, stream, &why)
                 : pa::launch_gqa_mfma_decode(s, a, plan, stream, &why);
    return finish(st, why);
}

PA_EXPORT pa_status pa_decode_ex(void *out, float *lse, const void *q, const void *k_cache,
                                 const void *v_cache, const int32_t *block_tables,
                                 const int32_t *context_lens, float scale, int32_t window,
                                 int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                 int32_t max_blocks_per_seq, pa_dtype dtype, void *workspace,
                                 size_t workspace_bytes, void *stream) {
    pa::DecodeShape s = make_shape(false, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                   head_dim, block_size, max_blocks_per_seq, dtype);
    s.window = window;
    std::string why;
    if (!v_cache && num_seqs > 0)
        return finish(PA_ERR_NULL, "decode_ex: v_cache must be non-NULL (no latent mode)");
    pa::DecodePlan plan{};
    pa_status st = pa::plan_decode(s, &plan, &why);
    if (st != PA_OK) return finish(st, why);
    if (lse && reinterpret_cast<uintptr_t>(lse) % 4 != 0)
        return finish(PA_ERR_ALIGN, "decode_ex: lse must be 4-byte aligned");
    pa::DecodeArgs a{out, q, k_cache, v_cache, block_tables, context_lens, nullptr, nullptr,
                     scale, num_blocks, workspace, workspace_bytes};
    a.lse = lse;
    st = pa::check_decode(s, a, plan, &why);
    if (st != PA_OK || num_seqs == 0) return finish(st, why);
    PA_DEBUG_CHECK(pa::debug_check_tables(block_tables, context_lens, num_seqs,
                                          max_blocks_per_seq, block_size, window, num_blocks,
                                          static_cast<int64_t>(max_blocks_per_seq) * block_size,
                                          stream, &dbg_why));
    st = plan.path == pa::DecodePath::kGroupedMfma ? pa::launch_gqa_mfma_decode(s, a, plan, stream, &why)
                                                   : pa::launch_grouped_decode(s, a, plan, stream, &why);
    return finish(st, why);
}

PA_EXPORT pa_status pa_attention_scores(float *scores, const void *q, const void *k_cache,
                                        const int32_t *block_tables, const int32_t *context_lens,
                                        const float *lse, float scale, int32_t window,
                                        int32_t num_seqs, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t block_size, int32_t max_blocks_per_seq,
                                        int32_t max_context, pa_dtype dtype, void *stream) {
    if (dtype != PA_F32 && dtype != PA_BF16) return finish(PA_ERR_DTYPE, "scores: unknown dtype");
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || max_blocks_per_seq <= 0 || max_context < 0 || window < 0 ||
        num_q_heads % num_kv_heads != 0)
        return finish(PA_ERR_SHAPE, "scores: sizes must be positive, num_q_heads a multiple of "
                                    "num_kv_heads");
    if ((head_dim != 64 && head_dim != 128) || block_size != 16 || num_q_heads / num_kv_heads > 16 ||
        num_kv_heads > 65535 || num_seqs > 65535)
        return finish(PA_ERR_UNSUPPORTED, "scores: runs head_dim 64 or 128, block_size 16, "
                                          "num_q_heads / num_kv_heads <= 16");
    if ((int64_t)max_context > (int64_t)max_blocks_per_seq * block_size)
        return finish(PA_ERR_SHAPE, "scores: max_context exceeds the block table's capacity");
    if (num_seqs == 0 || max_context == 0) return finish(PA_OK, "");
    if (!scores || !q || !k_cache || !block_tables || !context_lens || !lse)
        return finish(PA_ERR_NULL, "scores: scores, q, k_cache, block_tables, context_lens and "
                                   "lse must be non-NULL");
    if (reinterpret_cast<uintptr_t>(q) % 16 != 0 || reinterpret_cast<uintptr_t>(k_cache) % 16 != 0 ||
        reinterpret_cast<uintptr_t>(scores) % 4 != 0 || reinterpret_cast<uintptr_t>(lse) % 4 != 0)
        return finish(PA_ERR_ALIGN, "scores: q and k_cache must be 16-byte aligned");
    std::string why;
    PA_DEBUG_CHECK(pa::debug_check_tables(block_tables, context_lens, num_seqs,
                                          max_blocks_per_seq, block_size, window, INT32_MAX,
                                          max_context, stream, &dbg_why));
    const pa_status st = pa::launch_attention_scores(
        scores, q, k_cache, block_tables, context_lens, lse, scale, window, num_seqs, num_q_heads,
        num_kv_heads, head_dim, max_blocks_per_seq, max_context, dtype,
        stream, &why);
    return finish(st, why);
}

PA_EXPORT pa_status pa_copy_blocks(void *pool, int64_t block_bytes, const int32_t *src,
                                   const int32_t *dst, int32_t num_pairs, void *stream) {
    if (num_pairs < 0 || block_bytes <= 0)
        return finish(PA_ERR_SHAPE, "copy_blocks: num_pairs < 0 or block_bytes <= 0");
    if (num_pairs == 0) return finish(PA_OK, "");
    if (!pool || !src || !dst) return finish(PA_ERR_NULL, "copy_blocks: pool, src and dst must be non-NULL");
    if (num_pairs > 65535) return finish(PA_ERR_UNSUPPORTED, "copy_blocks: at most 65535 pairs per call");
    if (block_bytes % 16 != 0 || reinterpret_cast<uintptr_t>(pool) % 16 != 0 ||
        reinterpret_cast<uintptr_t>(src) % 4 != 0 || reinterpret_cast<uintptr_t>(dst) % 4 != 0)
        return finish(PA_ERR_ALIGN, "copy_blocks: pool and block_bytes must be multiples of 16 bytes");
    std::string why;
    PA_DEBUG_CHECK(pa::debug_check_copies(src, dst, num_pairs, stream, &dbg_why));
    const pa_status st = pa::launch_copy_blocks(pool, block_bytes, src, dst, num_pairs,
                                                stream, &why);
    return finish(st, why);
}

PA_EXPORT const char *pa_status_string(pa_status status) {
    switch (status) {
        case PA_OK: return "PA_OK";
        case PA_ERR_NULL: return "PA_ERR_NULL";
        case PA_ERR_SHAPE: return "PA_ERR_SHAPE";
        case PA_ERR_DTYPE: return "PA_ERR_DTYPE";
        case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
        case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
        case PA_ERR_HIP: return "PA_ERR_HIP";
        case PA_ERR_ALIGN: return "PA_ERR_ALIGN";
        case PA_ERR_INDEX: return "PA_ERR_INDEX";
    }
    return "PA_ERR_UNKNOWN";
}

PA_EXPORT const char *pa_last_error(void) { return g_last_error.c_str(); }

PA_EXPORT int32_t pa_build_flags(void) {
#ifdef PA_DEBUG
    return 1;
#else
    return 0;
#endif
}
