/*
 * pa.h — C ABI of libpa.so: decode-phase attention over a paged KV cache on
 * AMD Instinct MI355X (gfx950), plus the slot-mapped append that fills it.
 *
 * The operations follow the pages this library is built from:
 *
 *  - The KV cache is a pool of fixed-size blocks ("pages" of block_size
 *    tokens) that may sit anywhere in device memory; each sequence reaches
 *    its tokens through a block table mapping logical block index ->
 *    physical block ("PagedAttention" in "Optimisation de l'inférence";
 *    "PagedAttention KV cache comme mémoire virtuelle" in "Cache KV,
 *    attention et optimisation de l'inference").
 *  - One layer's cache is a tensor [num_blocks, block_size, num_kv_heads,
 *    head_dim], one for K and one for V (the pool of "Implémentation du
 *    cache" in the nano-vLLM article, sliced per layer).
 *  - New K/V rows are written through a slot mapping, slot = physical block *
 *    block_size + offset, with -1 meaning "skip this token" ("Écriture dans
 *    le cache", same article).
 *  - Decode attention is one query token per sequence attending to all of its
 *    cached tokens: O = softmax(q K^T * scale) V, max-subtracted, with no mask
 *    ("Étape 2: Attention avec KV Cache", "Optimisation de l'inférence"),
 *    where query head h reads KV head h / (num_q_heads / num_kv_heads)
 *    (grouped-query attention, CS336 lecture 10 notes, "核心概念与定义").
 *  - Latent mode (v_cache == NULL): one cached 576-wide latent row per token
 *    serves as the key, and its first head_dim_v = 512 values serve as the
 *    value (the MLA bullet of the same notes: 512 latent + 64 RoPE dims).
 *
 * Conventions for every call:
 *  - All array pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or keeps them after returning.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work on it; they never synchronise and never read device arrays
 *    from the host, so slot_mapping, block_tables and context_lens are
 *    trusted (see "Undefined" below).
 *  - Errors: host-checkable faults return a status and enqueue nothing.
 *    pa_last_error() then holds a message for the calling thread.  A failed
 *    kernel launch returns PA_ERR_HIP.  No call prints or throws.
 *  - Undefined (not checked, the contract is the caller's): a slot or block id
 *    outside the pool, a context longer than max_blocks_per_seq * block_size,
 *    duplicate non-negative slots in one append, negative context lengths.
 *  - Debug builds (libpa_debug.so, compiled with PA_DEBUG): every call first
 *    runs a device pass over the index arrays it will use (slot_mapping;
 *    context_lens and the block-table entries of the blocks it reads;
 *    copy pairs), waits for the stream, and returns PA_ERR_INDEX, naming the
 *    rule and the element, without enqueuing its own kernels when one is
 *    broken (duplicates are looked for among the first 4096 slots or pairs).
 *    Debug calls therefore synchronise and cannot be captured into a graph;
 *    their results are bitwise those of the release build.
 *  - Results are deterministic: no atomics, bitwise identical run to run and
 *    independent of where the physical blocks sit in the pool.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_NULL = 1,        /* a required pointer is NULL */
    PA_ERR_SHAPE = 2,       /* sizes inconsistent or out of range */
    PA_ERR_DTYPE = 3,       /* unknown dtype */
    PA_ERR_UNSUPPORTED = 4, /* valid but outside the shapes the library runs */
    PA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required */
    PA_ERR_HIP = 6,         /* the HIP runtime reported an error */
    PA_ERR_ALIGN = 7,       /* a pointer or stride breaks the 16-byte alignment rule */
    PA_ERR_INDEX = 8        /* PA_DEBUG builds only: an index array broke the contract */
} pa_status;

typedef enum pa_dtype {
    PA_F32 = 0,  /* IEEE binary32 */
    PA_BF16 = 1  /* bfloat16 (upper 16 bits of binary32), round-to-nearest-even */
} pa_dtype;

/*
 * pa_cache_append — write each new token's K (and V) row into its cache slot.
 *
 * For i in [0, num_tokens): s = slot_mapping[i]; if s == -1 the token is
 * skipped, otherwise row s of k_cache viewed as [num_blocks * block_size,
 * num_kv_heads * head_dim_k] becomes a bitwise copy of k[i], and likewise for
 * v_cache / v with head_dim_v.  No other byte of either cache changes.
 *
 *   k_cache, v_cache  [num_blocks, block_size, num_kv_heads, head_dim_{k,v}],
 *                     contiguous, element type `dtype`.  v_cache == NULL
 *                     selects latent mode: only k is written, and v must be NULL.
 *   k, v              token i's row starts at element i * {k,v}_token_stride;
 *                     the num_kv_heads * head_dim elements of a row are
 *                     contiguous.  Strides are in elements, >= the row length.
 *   slot_mapping      int32 [num_tokens]; -1 = skip.  Non-negative slots must be
 *                     distinct and < num_blocks * block_size.
 *   dtype             element type of k, v and both caches (the copy never
 *                     converts).
 * num_tokens == 0 is a no-op.  Returns PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE
 * or PA_ERR_HIP as described above.
 */
pa_status pa_cache_append(void *k_cache, void *v_cache,
                          const void *k, int64_t k_token_stride,
                          const void *v, int64_t v_token_stride,
                          const int32_t *slot_mapping, int32_t num_tokens,
                          int32_t num_blocks, int32_t block_size,
                          int32_t num_kv_heads, int32_t head_dim_k,
                          int32_t head_dim_v, pa_dtype dtype, void *stream);

/*
 * pa_decode_workspace_size — bytes of device workspace pa_decode needs for
 * these sizes (the split-context partial results: an fp32 accumulator of
 * head_dim_v values plus a running max and a running sum per sequence, query
 * head and context partition).  Returns 0 when the sizes are not valid.
 * pa_decode must be called with the same sizes.  The sizes carry no v_cache
 * pointer, so head_dim_k != head_dim_v is what names latent mode here; the
 * only unequal pair accepted is the latent shape (576, 512, one KV head,
 * block size 64), and any other returns 0.
 */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim_k,
                                int32_t head_dim_v, int32_t block_size,
                                int32_t max_blocks_per_seq);

/*
 * pa_decode — decode attention for one query token per sequence.
 *
 * For b < num_seqs, h < num_q_heads, with G = num_q_heads / num_kv_heads,
 * g = h / G and L = context_lens[b]: token t < L sits at row t % block_size of
 * physical block block_tables[b * max_blocks_per_seq + t / block_size];
 *   s_t = scale * dot(q[b,h,:], K[t, g, :])
 *   out[b,h,:] = sum_t exp(s_t - max s) V[t, g, :] / sum_t exp(s_t - max s)
 * and out[b,h,:] = 0 when L == 0.  Cache slots at or beyond L are never used,
 * whatever they hold (NaN included).
 *
 *   out            [num_seqs, num_q_heads, head_dim_v], element type dtype
 *                  (fp32 accumulation, rounded once to nearest-even for bf16).
 *   q              [num_seqs, num_q_heads, head_dim_k], dtype, contiguous.
 *   k_cache        [num_blocks, block_size, num_kv_heads, head_dim_k], dtype.
 *   v_cache        [num_blocks, block_size, num_kv_heads, head_dim_v], dtype,
 *                  or NULL for latent mode (V = first head_dim_v values of
 *                  each k_cache row).
 *   block_tables   int32 [num_seqs, max_blocks_per_seq]; entries past the
 *                  blocks a sequence uses are never read.
 *   context_lens   int32 [num_seqs], each in [0, max_blocks_per_seq*block_size].
 *   scale          softmax scale (finite), e.g. 1/sqrt(head_dim_k).
 *   workspace      device buffer of at least pa_decode_workspace_size(...)
 *                  bytes, 256-byte aligned; its contents on entry do not matter
 *                  and on return are scratch.
 *
 * Shapes the library runs (anything else returns PA_ERR_UNSUPPORTED):
 *   - head_dim_k == head_dim_v in {64, 128}, block_size 16,
 *     num_q_heads / num_kv_heads in {1, 2, 4, 8}, dtype PA_F32 or PA_BF16;
 *   - latent mode: head_dim_k 576, head_dim_v 512, num_kv_heads 1,
 *     block_size 64, PA_BF16, num_q_heads a multiple of 16 up to 128.
 * q, caches, out and workspace must be 16-byte aligned (PA_ERR_ALIGN).
 */
pa_status pa_decode(void *out, const void *q, const void *k_cache,
                    const void *v_cache, const int32_t *block_tables,
                    const int32_t *context_lens, float scale, int32_t num_seqs,
                    int32_t num_q_heads, int32_t num_kv_heads,
                    int32_t head_dim_k, int32_t head_dim_v, int32_t block_size,
                    int32_t num_blocks, int32_t max_blocks_per_seq,
                    pa_dtype dtype, void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * pa_decode_noalloc — pa_decode without a workspace argument, for callers
 * that cannot allocate device memory (code under graph capture, tight
 * serving loops, harnesses that forbid allocation).  The same kernels and
 * results as pa_decode (bitwise); the split-context partials go to a scratch
 * array of 32 MiB that the library holds on each GPU it runs on until the
 * process ends (the first call on a device looks its address up; no call
 * allocates or frees anything).  Sizes whose pa_decode_workspace_size
 * exceeds 32 MiB return PA_ERR_WORKSPACE without enqueuing anything: the
 * grouped shapes fit up to 496 sequences of 64/8 heads (any context
 * length), the latent shape, whose workspace holds 512 partial slots of
 * every head, does not fit.  Every call on one GPU uses
 * that GPU's one array: calls that overlap on a device (two streams, two
 * threads) race and must be ordered by the caller.  Arguments and errors
 * otherwise as for pa_decode.
 */
pa_status pa_decode_noalloc(void *out, const void *q, const void *k_cache,
                            const void *v_cache, const int32_t *block_tables,
                            const int32_t *context_lens, float scale, int32_t num_seqs,
                            int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim_k, int32_t head_dim_v, int32_t block_size,
                            int32_t num_blocks, int32_t max_blocks_per_seq,
                            pa_dtype dtype, void *stream);

/*
 * MXFP8 KV cache.  Fewer bytes per cached value make memory-bound decode
 * faster, fp8 being one of the formats (CS336 lecture 10 notes, "第 10 讲：
 * 推理", "核心概念与定义", quantization bullet), and the scales should be
 * blockwise rather than per tensor, MXFP8 being the example given (same
 * notes, "常见陷阱").  MXFP8 is the OCP Microscaling format: every 32
 * consecutive values share one E8M0 scale byte e (value 2^(e - 127); 0xFF
 * is NaN) and each value is an FP8 E4M3 byte (sign, 4 exponent bits with
 * bias 7, 3 mantissa bits; S.1111.111 is NaN; largest magnitude 448).  A
 * cached value is code * 2^(e - 127).  Cache layouts, one layer, uint8:
 *
 *   k_cache  [num_blocks, num_kv_heads, block_size, head_dim]   E4M3 codes
 *   v_cache  [num_blocks, num_kv_heads, head_dim, block_size]   E4M3 codes,
 *            each (block, head) tile transposed (dims x tokens)
 *   k_scale, v_scale  [num_blocks, num_kv_heads, block_size, head_dim / 32]
 *            E8M0 bytes; byte j of a token row scales its values
 *            32 j .. 32 j + 31
 *
 * Slots, block tables and context lengths mean what they mean for pa_decode.
 * Supported: head_dim 128; decode also needs block_size 16, bf16 q and out,
 * num_q_heads / num_kv_heads in {1, 2, 4, 8}.  All cache and scale pointers
 * must be 16-byte aligned.
 */

/*
 * pa_cache_append_mxfp8 — quantize each new token's K and V rows into its
 * slot of MXFP8 caches.
 *
 * For i < num_tokens with s = slot_mapping[i] != -1, p = s / block_size,
 * r = s % block_size, and each KV head h: every 32-value block of the row
 * k[i, h, :] gets X = floor(log2(max |value|)) - 8, clamped to [-127, 127]
 * (X = -127 for an all-zero block); scale byte X + 127 goes to
 * k_scale[p, h, r, block] and each value * 2^-X, rounded to the nearest
 * E4M3 value (ties to even, saturating at +-448), to k_cache[p, h, r, :].
 * v[i, h, :] is quantized the same way into column r of v_cache[p, h] and
 * v_scale[p, h, r, :].  Nothing else changes.
 *
 *   k, v      [num_tokens, num_kv_heads, head_dim] rows of element type
 *             dtype (PA_F32 or PA_BF16), token i at element i * stride;
 *             values must be finite (otherwise the codes are unspecified).
 *   slot_mapping  int32 [num_tokens]; -1 = skip; other slots distinct and
 *             < num_blocks * block_size.
 * num_tokens == 0 is a no-op.  Returns PA_ERR_NULL, PA_ERR_SHAPE,
 * PA_ERR_DTYPE, PA_ERR_UNSUPPORTED (head_dim != 128), PA_ERR_ALIGN or
 * PA_ERR_HIP.
 */
pa_status pa_cache_append_mxfp8(void *k_cache, void *v_cache, void *k_scale,
                                void *v_scale, const void *k,
                                int64_t k_token_stride, const void *v,
                                int64_t v_token_stride,
                                const int32_t *slot_mapping, int32_t num_tokens,
                                int32_t num_blocks, int32_t block_size,
                                int32_t num_kv_heads, int32_t head_dim,
                                pa_dtype dtype, void *stream);

/*
 * pa_decode_mxfp8 — pa_decode over MXFP8 caches: the same attention with
 * every cached K and V value taken as code * 2^(e - 127) (products with
 * magnitude below 2^-126 may be flushed to zero).  q and out are bf16
 * (dtype must be PA_BF16), [num_seqs, num_q_heads, head_dim].  The
 * workspace is the one pa_decode_workspace_size(num_seqs, num_q_heads,
 * num_kv_heads, head_dim, head_dim, block_size, max_blocks_per_seq) sizes.
 * Slots at or beyond a sequence's length are never used, whatever their
 * codes and scales hold.  Errors as for pa_decode.
 */
pa_status pa_decode_mxfp8(void *out, const void *q, const void *k_cache,
                          const void *v_cache, const void *k_scale,
                          const void *v_scale, const int32_t *block_tables,
                          const int32_t *context_lens, float scale,
                          int32_t num_seqs, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t num_blocks,
                          int32_t max_blocks_per_seq, pa_dtype dtype,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * Several new query tokens per sequence, causal among themselves: the shape
 * of verifying k drafted tokens in one pass of the target model (section
 * "Décodage spéculatif" of "Optimisation de l'inférence": the candidates are
 * scored in one forward pass that looks like a prefill) and of a prefill
 * chunk over a paged context.  The last q_len of a sequence's L = context_lens[b] cached
 * tokens are its queries (appended to the cache beforehand), and query i,
 * at position L - q_len + i, attends to tokens 0 .. L - q_len + i: the
 * upper-triangular mask of "Étape 2: Attention avec KV Cache" on the same
 * page.  A query whose position is negative (L < q_len - i) gets O = 0.
 *
 * pa_decode_multi_workspace_size — bytes of workspace pa_decode_multi needs
 * (0 when the sizes are not valid); the same for both cache formats.
 */
size_t pa_decode_multi_workspace_size(int32_t num_seqs, int32_t q_len,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size,
                                      int32_t max_blocks_per_seq);

/*
 * pa_decode_multi — for b < num_seqs, i < q_len, h < num_q_heads:
 *   out[b, i, h, :] = softmax_t(scale * q[b, i, h, :] . K[t, g, :]) V[t, g, :]
 * over t < L_b - q_len + i + 1, g = h / (num_q_heads / num_kv_heads).
 *
 *   q, out       [num_seqs, q_len, num_q_heads, head_dim], bf16 (dtype must
 *                be PA_BF16).
 *   k_cache, v_cache  bf16 [num_blocks, block_size, num_kv_heads, head_dim]
 *                when k_scale == v_scale == NULL; MXFP8 codes in the
 *                layouts of pa_cache_append_mxfp8 when both scales are set.
 *   other arguments as for pa_decode.
 * Runs head_dim 128, block_size 16, (num_q_heads / num_kv_heads) * q_len
 * <= 64; q_len == 1 is the single-query decode.  Errors as for pa_decode;
 * PA_ERR_NULL when exactly one scale pointer is NULL.
 */
pa_status pa_decode_multi(void *out, const void *q, const void *k_cache,
                          const void *v_cache, const void *k_scale,
                          const void *v_scale, const int32_t *block_tables,
                          const int32_t *context_lens, float scale,
                          int32_t num_seqs, int32_t q_len, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t num_blocks,
                          int32_t max_blocks_per_seq, pa_dtype dtype,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * Sliding window and exported log-sum-exp, for per-layer KV sparsity.  The
 * KV-sparsity article ("Comment KV Sparsity permet une accélération de 1,5x
 * pour vLLM") lets each layer run a full cache or a sliding window
 * ("Sparsité par couche et parallélisme de tenseurs"; local attention over a
 * window is in the CS336 lecture 10 notes, "核心概念与定义"), has the
 * attention kernel export its row max and sum, and recomputes each cached
 * token's softmax probability from them to score the tokens a layer keeps
 * ("Modification de l'Attention").
 *
 * pa_decode_ex — pa_decode with two options:
 *   window  > 0: the query of a sequence of length L attends only to tokens
 *           [max(0, L - window), L); 0 attends to all of them.
 *   lse     optional fp32 [num_seqs, num_q_heads] output (NULL skips it):
 *           log(sum_t exp(s_t)) over the attended tokens, s_t = scale *
 *           q . k_t, natural log; -inf for an empty context.  It is
 *           accumulated from the same bf16-rounded weights as the output.
 * bf16 or fp32 caches [num_blocks, block_size, num_kv_heads, head_dim] (no
 * latent mode); shapes and workspace as for pa_decode.
 */
pa_status pa_decode_ex(void *out, float *lse, const void *q, const void *k_cache,
                       const void *v_cache, const int32_t *block_tables,
                       const int32_t *context_lens, float scale, int32_t window,
                       int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t num_blocks,
                       int32_t max_blocks_per_seq, pa_dtype dtype, void *workspace,
                       size_t workspace_bytes, void *stream);

/*
 * pa_attention_scores — the attention mass each cached token gets from the
 * query heads sharing its KV head:
 *   scores[b, g, t] = sum over h with h / G == g of exp(scale * q[b, h] .
 *                     k_t - lse[b, h])
 * for t in the window [max(0, L - window), L) (window 0: all of [0, L)), and
 * 0 for every other t < max_context.  With the lse of pa_decode_ex each
 * head's values sum to 1 over the window, so a row sums to G.
 *   scores   fp32 [num_seqs, num_kv_heads, max_context], written whole.
 *   q, k_cache, block_tables, context_lens as for pa_decode (dtype PA_F32 or
 *   PA_BF16); lse fp32 [num_seqs, num_q_heads].
 * Runs head_dim 64 or 128, block_size 16, num_q_heads / num_kv_heads <= 16;
 * every context must be <= max_context <= max_blocks_per_seq * block_size.
 */
pa_status pa_attention_scores(float *scores, const void *q, const void *k_cache,
                              const int32_t *block_tables, const int32_t *context_lens,
                              const float *lse, float scale, int32_t window,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size,
                              int32_t max_blocks_per_seq, int32_t max_context,
                              pa_dtype dtype, void *stream);

/*
 * Host block manager: the caller side that turns token ids into block tables
 * and slot mappings.  It follows the block manager of "Implémentation du
 * cache" in the nano-vLLM article (a pool allocated once, a chained hash per
 * full block built from the previous block's hash and the block's own token
 * ids so that shared prefixes map to the same physical blocks, and reference
 * counts that keep shared blocks alive) and PagedAttention's prefix sharing
 * and copy-on-write in the CS336 lecture 10 notes ("核心概念与定义").
 * Host memory only, no GPU calls; not thread-safe.  Sequence ids are the
 * caller's.  Status codes: PA_ERR_NULL (NULL handle or array), PA_ERR_SHAPE
 * (unknown or duplicate sequence id, table too small), PA_ERR_WORKSPACE (no
 * free block; nothing changes).
 */
typedef struct pa_block_manager pa_block_manager;

/* A manager of num_blocks blocks of block_size token slots, all free; NULL
 * for non-positive sizes or when memory runs out. */
pa_block_manager *pa_bm_create(int32_t num_blocks, int32_t block_size);
void pa_bm_destroy(pa_block_manager *m);
int32_t pa_bm_num_free(const pa_block_manager *m);
/* Sequences holding the block (-1 for an id outside the pool). */
int32_t pa_bm_ref_count(const pa_block_manager *m, int32_t block);

/*
 * pa_bm_add_sequence — admit a sequence whose first num_tokens tokens are
 * tokens[].  Each full block of tokens whose chained hash and token ids match
 * a block already held (for the same preceding blocks) reuses that block;
 * the first miss and everything after it take fresh blocks, as does a partly
 * filled last block.  *num_cached (may be NULL) receives the number of
 * leading tokens whose K/V are already in shared blocks: the caller appends
 * K/V only for tokens from there on, at slot block_table[t / block_size] *
 * block_size + t % block_size.
 */
pa_status pa_bm_add_sequence(pa_block_manager *m, int64_t seq_id, const int32_t *tokens,
                             int32_t num_tokens, int32_t *num_cached);

/*
 * pa_bm_append_token — one more token for the sequence; *slot receives the
 * cache slot its K/V go to.  A full last block gets a fresh block after it;
 * a partly filled last block shared with another sequence (after a fork) is
 * first replaced by a fresh block, and the (shared, fresh) pair is queued
 * for pa_copy_blocks, which must run before the token's K/V are written.
 * A block that fills up becomes shareable under its chained hash.
 */
pa_status pa_bm_append_token(pa_block_manager *m, int64_t seq_id, int32_t token,
                             int32_t *slot);

/* pa_bm_fork — child starts as a copy of parent, sharing all its blocks. */
pa_status pa_bm_fork(pa_block_manager *m, int64_t parent, int64_t child);

/* pa_bm_free_sequence — release the sequence's blocks (a block returns to
 * the free list when no sequence holds it). */
pa_status pa_bm_free_sequence(pa_block_manager *m, int64_t seq_id);

/* Tokens of the sequence so far (-1 for an unknown id). */
int64_t pa_bm_num_tokens(const pa_block_manager *m, int64_t seq_id);

/* The sequence's block ids into out[0 .. max_blocks), padded with -1. */
pa_status pa_bm_block_table(const pa_block_manager *m, int64_t seq_id, int32_t *out,
                            int32_t max_blocks);

/* Moves up to max_pairs queued copy-on-write pairs into src[], dst[] (host
 * arrays); returns how many. */
int32_t pa_bm_take_copies(pa_block_manager *m, int32_t *src, int32_t *dst,
                          int32_t max_pairs);

/*
 * pa_copy_blocks — on the GPU, block dst[i] of pool becomes a copy of block
 * src[i] (block i occupies bytes [i * block_bytes, (i + 1) * block_bytes)),
 * for i < num_pairs.  Call it once per pool array: K and V, and k_scale and
 * v_scale of an MXFP8 cache (their block sizes differ).  src and dst are
 * int32 DEVICE arrays; no destination may also be a source.  pool and
 * block_bytes must be multiples of 16 bytes (PA_ERR_ALIGN); at most 65535
 * pairs per call (PA_ERR_UNSUPPORTED).
 */
pa_status pa_copy_blocks(void *pool, int64_t block_bytes, const int32_t *src,
                         const int32_t *dst, int32_t num_pairs, void *stream);

/* Build flags of the loaded library: bit 0 set in a PA_DEBUG build. */
int32_t pa_build_flags(void);

/* Static text for a status code ("PA_OK", ...); never NULL. */
const char *pa_status_string(pa_status status);

/* Detail of the calling thread's last failed call ("" if none). */
const char *pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
