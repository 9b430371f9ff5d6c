// Host-side argument checks and launch planning (no HIP headers).
#include "plan.h"

#include <cmath>
#include <cstdlib>

namespace pa {
namespace {

constexpr size_t kWorkspaceAlign = 256;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int elt_bytes(int32_t d) { return d == PA_F32 ? 4 : 2; }

// A caller passing an int that is no pa_dtype value must get PA_ERR_DTYPE,
// so the value is compared as an integer, never loaded as the enum.
bool valid_dtype(int32_t d) { return d == PA_F32 || d == PA_BF16; }

pa_status fail(pa_status st, std::string *why, const std::string &msg) {
    if (why) *why = msg;
    return st;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Whether a single-query grouped-shape bf16 decode with head dim 128 runs its
// per-block products on the matrix cores.  The lane-wise dot-product kernel is
// the default: decode attention with one query row per head is a matrix-vector
// product per KV head, which the vector units cover within the memory time.
// PA_GQA_MFMA=1 selects the matrix-core variant (the same split, partials and
// reduce), which carries the several-query and MXFP8 paths in any case.
bool grouped_mfma_default(const DecodeShape &s) {
    if (s.dtype != PA_BF16 || s.head_dim_k != 128) return false;
    const char *env = std::getenv("PA_GQA_MFMA");
    return env && *env && std::atoi(env) != 0;
}

// Cache blocks each wave of the grouped paths streams into LDS (ring depth):
// two slots per wave, one block in flight while the wave computes on the
// other.  With the partials written at the share's end, two 8 KB bf16 slots
// per wave measure faster than four at the same four waves per CU (c3 299.6
// against 304.5 us, c4 328.7 against 334.8, c2 and the several-query shapes
// equal or faster), and MXFP8 slots, half the size, run two per wave at eight
// waves per CU.  PA_RING_DEPTH (2 or 4) overrides the default.
int grouped_ring_depth() {
    const char *env = std::getenv("PA_RING_DEPTH");
    if (env && *env) return std::atoi(env) == 4 ? 4 : 2;
    return 2;
}

}  // namespace

pa_status check_append(const AppendArgs &a, AppendPlan *plan, std::string *why) {
    if (!valid_dtype(a.dtype)) return fail(PA_ERR_DTYPE, why, "append: unknown dtype");
    if (a.num_tokens < 0) return fail(PA_ERR_SHAPE, why, "append: num_tokens < 0");
    if (a.num_blocks <= 0 || a.block_size <= 0 || a.num_kv_heads <= 0 || a.head_dim_k <= 0)
        return fail(PA_ERR_SHAPE, why,
                    "append: num_blocks, block_size, num_kv_heads and head_dim_k must be > 0");
    const bool latent = a.v_cache == nullptr;
    if (latent != (a.v == nullptr))
        return fail(PA_ERR_NULL, why, "append: v_cache and v must both be NULL or both set");
    if (!latent && a.head_dim_v <= 0)
        return fail(PA_ERR_SHAPE, why, "append: head_dim_v must be > 0 with a V cache");
    if (a.num_tokens > 0 && (!a.k_cache || !a.k || !a.slot_mapping))
        return fail(PA_ERR_NULL, why, "append: k_cache, k and slot_mapping must be non-NULL");
    if ((int64_t)a.num_blocks * a.block_size > INT32_MAX)
        return fail(PA_ERR_SHAPE, why, "append: more than 2^31-1 slots");
    const int eb = elt_bytes(a.dtype);
    const int64_t k_row = (int64_t)a.num_kv_heads * a.head_dim_k;
    const int64_t v_row = latent ? 0 : (int64_t)a.num_kv_heads * a.head_dim_v;
    if (a.k_token_stride < k_row)
        return fail(PA_ERR_SHAPE, why, "append: k_token_stride smaller than a K row");
    if (!latent && a.v_token_stride < v_row)
        return fail(PA_ERR_SHAPE, why, "append: v_token_stride smaller than a V row");
    int vec = 16;
    auto fits = [&](int64_t bytes) { return bytes % vec == 0; };
    auto ptr_fits = [&](const void *p) { return p == nullptr || aligned(p, vec); };
    while (vec > eb) {
        bool ok = fits(k_row * eb) && fits(a.k_token_stride * eb) && ptr_fits(a.k_cache) &&
                  ptr_fits(a.k);
        if (!latent)
            ok = ok && fits(v_row * eb) && fits(a.v_token_stride * eb) && ptr_fits(a.v_cache) &&
                 ptr_fits(a.v);
        if (ok) break;
        vec /= 2;
    }
    if (!ptr_fits(a.k_cache) || !ptr_fits(a.k) || !ptr_fits(a.v_cache) || !ptr_fits(a.v))
        return fail(PA_ERR_ALIGN, why, "append: pointers not aligned to the element size");
    if (plan) {
        plan->vec_bytes = vec;
        plan->k_row_bytes = k_row * eb;
        plan->v_row_bytes = v_row * eb;
    }
    return PA_OK;
}

pa_status check_append_mxfp8(const MxAppendArgs &a, std::string *why) {
    if (!valid_dtype(a.dtype)) return fail(PA_ERR_DTYPE, why, "append (mxfp8): unknown dtype");
    if (a.num_tokens < 0) return fail(PA_ERR_SHAPE, why, "append (mxfp8): num_tokens < 0");
    if (a.num_blocks <= 0 || a.block_size <= 0 || a.num_kv_heads <= 0 || a.head_dim <= 0)
        return fail(PA_ERR_SHAPE, why, "append (mxfp8): num_blocks, block_size, num_kv_heads "
                                       "and head_dim must be > 0");
    if (a.head_dim != kMxHeadDim)
        return fail(PA_ERR_UNSUPPORTED, why, "append (mxfp8): runs head_dim 128");
    if (a.num_kv_heads > 65535)
        return fail(PA_ERR_UNSUPPORTED, why, "append (mxfp8): runs at most 65535 KV heads");
    if (a.num_tokens > 0 && (!a.k_cache || !a.v_cache || !a.k_scale || !a.v_scale || !a.k ||
                             !a.v || !a.slot_mapping))
        return fail(PA_ERR_NULL, why, "append (mxfp8): caches, scales, k, v and slot_mapping "
                                      "must be non-NULL");
    if ((int64_t)a.num_blocks * a.block_size > INT32_MAX)
        return fail(PA_ERR_SHAPE, why, "append (mxfp8): more than 2^31-1 slots");
    const int64_t row = (int64_t)a.num_kv_heads * a.head_dim;
    if (a.k_token_stride < row || a.v_token_stride < row)
        return fail(PA_ERR_SHAPE, why, "append (mxfp8): a token stride is smaller than a row");
    const int eb = elt_bytes(a.dtype);
    if (!aligned(a.k, eb) || !aligned(a.v, eb) || !aligned(a.k_cache, 16) ||
        !aligned(a.v_cache, 16) || !aligned(a.k_scale, 16) || !aligned(a.v_scale, 16))
        return fail(PA_ERR_ALIGN, why, "append (mxfp8): caches and scales must be 16-byte "
                                       "aligned, k and v aligned to their element size");
    return PA_OK;
}

pa_status plan_decode(const DecodeShape &s, DecodePlan *plan, std::string *why) {
    if (!valid_dtype(s.dtype)) return fail(PA_ERR_DTYPE, why, "decode: unknown dtype");
    if (s.num_seqs < 0) return fail(PA_ERR_SHAPE, why, "decode: num_seqs < 0");
    if (s.num_q_heads <= 0 || s.num_kv_heads <= 0 || s.head_dim_k <= 0 || s.head_dim_v <= 0 ||
        s.block_size <= 0 || s.max_blocks_per_seq <= 0)
        return fail(PA_ERR_SHAPE, why, "decode: head counts, head dims, block_size and "
                                       "max_blocks_per_seq must be > 0");
    if (s.num_q_heads % s.num_kv_heads != 0)
        return fail(PA_ERR_SHAPE, why, "decode: num_q_heads is not a multiple of num_kv_heads");
    if ((int64_t)s.max_blocks_per_seq * s.block_size > INT32_MAX)
        return fail(PA_ERR_SHAPE, why, "decode: max context exceeds 2^31-1 tokens");
    if (s.num_seqs > 65535 || s.num_kv_heads > 65535)
        return fail(PA_ERR_UNSUPPORTED, why, "decode: runs at most 65535 sequences and KV heads");
    const int G = s.num_q_heads / s.num_kv_heads;
    DecodePlan p{};
    p.group = G;
    if (s.q_len < 1) return fail(PA_ERR_SHAPE, why, "decode: q_len must be >= 1");
    if (s.window < 0) return fail(PA_ERR_SHAPE, why, "decode: window must be >= 0");
    if (s.window > 0 && (s.latent || s.q_len > 1 || s.mxfp8))
        return fail(PA_ERR_UNSUPPORTED, why,
                    "decode: a sliding window runs single-query grouped decode on bf16 or fp32 "
                    "caches");
    if (s.q_len > 1 && (s.latent || (!s.mxfp8 && s.dtype != PA_BF16) || s.head_dim_k != 128 ||
                        s.head_dim_v != 128 || s.block_size != 16 ||
                        (int64_t)G * s.q_len > 16 * kMaxColTiles))
        return fail(PA_ERR_UNSUPPORTED, why,
                    "decode (several queries per sequence): runs bf16 q with bf16 or MXFP8 "
                    "caches, head_dim 128, block_size 16, (num_q_heads / num_kv_heads) * "
                    "q_len <= 64");
    if (s.mxfp8) {
        if (s.latent || s.head_dim_k != kMxHeadDim || s.head_dim_v != kMxHeadDim ||
            s.block_size != 16 || s.dtype != PA_BF16 || (G != 1 && G != 2 && G != 4 && G != 8))
            return fail(PA_ERR_UNSUPPORTED, why,
                        "decode (mxfp8): runs head_dim 128, block_size 16, bf16 q and out, "
                        "num_q_heads / num_kv_heads in {1, 2, 4, 8}, with a V cache");
        if ((int64_t)s.num_seqs * s.max_blocks_per_seq * s.num_kv_heads > INT32_MAX)
            return fail(PA_ERR_SHAPE, why,
                        "decode: num_seqs * max_blocks_per_seq * num_kv_heads exceeds 2^31-1");
        p.path = DecodePath::kMxfp8;
        // half-size MXFP8 slots: two per wave, at 8 waves per CU (the launch
        // caps it there), measure faster than four (c3: 171.8 against 175.7 us)
        p.ring_depth = grouped_ring_depth();
    } else if (s.latent) {
        if (s.head_dim_k != 576 || s.head_dim_v != 512 || s.num_kv_heads != 1 ||
            s.block_size != 64 || s.dtype != PA_BF16 || s.num_q_heads % 16 != 0 ||
            s.num_q_heads > 128)
            return fail(PA_ERR_UNSUPPORTED, why,
                        "decode (latent): runs head_dim_k 576, head_dim_v 512, one KV head, "
                        "block_size 64, bf16, num_q_heads a multiple of 16 up to 128");
        if ((int64_t)s.num_seqs * s.max_blocks_per_seq > INT32_MAX)
            return fail(PA_ERR_SHAPE, why, "decode: num_seqs * max_blocks_per_seq exceeds 2^31-1");
        p.path = DecodePath::kLatent;
    } else {
        if (s.head_dim_k != s.head_dim_v || (s.head_dim_k != 64 && s.head_dim_k != 128))
            return fail(PA_ERR_UNSUPPORTED, why,
                        "decode: runs head_dim_k == head_dim_v in {64, 128}");
        if (s.block_size != 16)
            return fail(PA_ERR_UNSUPPORTED, why, "decode: runs block_size 16");
        if (G != 1 && G != 2 && G != 4 && G != 8)
            return fail(PA_ERR_UNSUPPORTED, why,
                        "decode: runs num_q_heads / num_kv_heads in {1, 2, 4, 8}");
        if ((int64_t)s.num_seqs * s.max_blocks_per_seq * s.num_kv_heads > INT32_MAX)
            return fail(PA_ERR_SHAPE, why,
                        "decode: num_seqs * max_blocks_per_seq * num_kv_heads exceeds 2^31-1");
        p.path = s.q_len > 1 || grouped_mfma_default(s) ? DecodePath::kGroupedMfma
                                                         : DecodePath::kGrouped;
        p.ring_depth = grouped_ring_depth();
    }
    size_t rows;  // (slot, head) rows of partial results
    if (p.path != DecodePath::kLatent)
        rows = ((size_t)kStreamWavesMax + (size_t)s.num_seqs * s.num_kv_heads) * (size_t)G *
               (size_t)s.q_len;
    else
        rows = ((size_t)kLatentWavesMax + (size_t)s.num_seqs) *
               (size_t)(latent_head_tiles(s.num_q_heads) * kLatentHeadTile);
    p.acc_offset = 0;
    p.ml_offset = round_up(rows * s.head_dim_v * sizeof(float), kWorkspaceAlign);
    p.prefix_offset = round_up(p.ml_offset + rows * 2 * sizeof(float), kWorkspaceAlign);
    p.bytes = round_up(p.prefix_offset + ((size_t)s.num_seqs + 1) * sizeof(int32_t),
                       kWorkspaceAlign);
    if (plan) *plan = p;
    return PA_OK;
}

pa_status check_decode(const DecodeShape &s, const DecodeArgs &a, const DecodePlan &plan,
                       std::string *why) {
    if (s.num_seqs == 0) return PA_OK;
    if (!a.out || !a.q || !a.k_cache || !a.block_tables || !a.context_lens)
        return fail(PA_ERR_NULL, why,
                    "decode: out, q, k_cache, block_tables and context_lens must be non-NULL");
    if (a.num_blocks <= 0) return fail(PA_ERR_SHAPE, why, "decode: num_blocks must be > 0");
    if (!std::isfinite(a.scale)) return fail(PA_ERR_SHAPE, why, "decode: scale is not finite");
    if (!aligned(a.out, 16) || !aligned(a.q, 16) || !aligned(a.k_cache, 16) ||
        (a.v_cache && !aligned(a.v_cache, 16)) || !aligned(a.block_tables, 4) ||
        !aligned(a.context_lens, 4))
        return fail(PA_ERR_ALIGN, why, "decode: q, caches and out must be 16-byte aligned");
    if (s.mxfp8 && (!a.v_cache || !a.k_scale || !a.v_scale))
        return fail(PA_ERR_NULL, why, "decode (mxfp8): v_cache, k_scale and v_scale must be "
                                      "non-NULL");
    if (s.mxfp8 && (!aligned(a.k_scale, 16) || !aligned(a.v_scale, 16)))
        return fail(PA_ERR_ALIGN, why, "decode (mxfp8): scales must be 16-byte aligned");
    if (!a.workspace || a.workspace_bytes < plan.bytes)
        return fail(PA_ERR_WORKSPACE, why,
                    "decode: workspace missing or smaller than pa_decode_workspace_size()");
    if (!aligned(a.workspace, kWorkspaceAlign))
        return fail(PA_ERR_ALIGN, why, "decode: workspace must be 256-byte aligned");
    return PA_OK;
}

}  // namespace pa
