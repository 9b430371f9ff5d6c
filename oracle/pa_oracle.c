/*
 * CPU oracle for paged decode attention and the slot-mapped KV append.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * helper with the HIP library; it is plain C, computes in double precision and
 * makes no attempt to be fast beyond an OpenMP loop over (sequence, head).
 *
 * What it computes is the plain definition, not a tiled replay:
 *
 *   decode  For each sequence b and query head h, with G = Hq / Hkv, KV head
 *           g = floor(h / G) and L = context_lens[b], token t < L lives in
 *           physical block block_tables[b][t / bs], row t % bs (the page table
 *           of "PagedAttention KV cache comme mémoire virtuelle", page "Cache
 *           KV, attention et optimisation de l'inference"; the pool layout
 *           [num_blocks, block_size, kv_heads, head_dim] of the nano-vLLM
 *           article, "Implémentation du cache").  Then
 *              s_t = scale * sum_i q[b,h,i] * k_t[i]
 *              O[b,h,:] = sum_t exp(s_t - max s) v_t / sum_t exp(s_t - max s)
 *           which is the scaled dot-product attention of "Étape 2: Attention
 *           avec KV Cache" (page "Optimisation de l'inférence") for a single
 *           query, where no mask applies.  Consecutive query heads share a KV
 *           head (GQA as in the CS336 lecture 10 notes, "核心概念与定义").
 *           With no V cache (latent mode) V is the first head_dim_v values of
 *           the same K row (the 512 + 64 = 576-dim latent of the MLA bullet).
 *           A context of length 0 yields O = 0.
 *
 *   append  For each token i with slot s = slot_mapping[i] != -1, row s of
 *           the cache viewed as [num_blocks * block_size, kv_heads * head_dim]
 *           becomes a byte copy of k[i] (and v[i]); nothing else changes
 *           (the cache-write kernel of "Écriture dans le cache", nano-vLLM
 *           article).
 *
 * Inputs are float32 (dtype 0) or bf16 bit patterns (dtype 1); both widen to
 * double exactly.  The output of decode is double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_BAD_SLOT 2
#define ORACLE_NO_MEM 3

static double widen(const void *base, int64_t idx, int dtype) {
    if (dtype == 0) {
        return (double)((const float *)base)[idx];
    }
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* One (b, h) output row. Returns 0, or ORACLE_NO_MEM. */
static int decode_row(double *out_row, const void *q, const void *k_cache,
                      const void *v_cache, const int32_t *block_tables,
                      const int32_t *context_lens, double scale, int b, int h,
                      int Hq, int Hkv, int dk, int dv, int bs, int max_blocks,
                      int dtype) {
    const int G = Hq / Hkv;
    const int g = h / G;
    const int L = context_lens[b];
    if (L <= 0) {
        for (int j = 0; j < dv; ++j) out_row[j] = 0.0;
        return ORACLE_OK;
    }

    /* scores and the output are built in private buffers and stored once */
    double *s = (double *)malloc(sizeof(double) * ((size_t)L + (size_t)dv));
    if (!s) return ORACLE_NO_MEM;
    double *o = s + L;
    for (int j = 0; j < dv; ++j) o[j] = 0.0;

    const int64_t q_off = ((int64_t)b * Hq + h) * dk;
    for (int t = 0; t < L; ++t) {
        const int64_t p = block_tables[(int64_t)b * max_blocks + t / bs];
        const int r = t % bs;
        const int64_t k_off = ((p * bs + r) * Hkv + g) * (int64_t)dk;
        double dot = 0.0;
        for (int i = 0; i < dk; ++i)
            dot += widen(q, q_off + i, dtype) * widen(k_cache, k_off + i, dtype);
        s[t] = scale * dot;
    }

    double m = s[0];
    for (int t = 1; t < L; ++t)
        if (s[t] > m) m = s[t];

    double denom = 0.0;
    for (int t = 0; t < L; ++t) {
        const double w = exp(s[t] - m);
        denom += w;
        const int64_t p = block_tables[(int64_t)b * max_blocks + t / bs];
        const int r = t % bs;
        int64_t v_off;
        const void *vbase;
        if (v_cache) {
            v_off = ((p * bs + r) * Hkv + g) * (int64_t)dv;
            vbase = v_cache;
        } else { /* latent: V is the leading dv values of the K row */
            v_off = ((p * bs + r) * Hkv + g) * (int64_t)dk;
            vbase = k_cache;
        }
        for (int j = 0; j < dv; ++j) o[j] += w * widen(vbase, v_off + j, dtype);
    }
    for (int j = 0; j < dv; ++j) out_row[j] = o[j] / denom;
    free(s);
    return ORACLE_OK;
}

/*
 * out: [num_seqs, Hq, dv] doubles (only listed rows are written when
 * pairs != NULL).  pairs: n_pairs (b, h) int32 pairs, or NULL for every row.
 */
int oracle_decode(double *out, const void *q, const void *k_cache,
                  const void *v_cache, const int32_t *block_tables,
                  const int32_t *context_lens, double scale, int num_seqs,
                  int Hq, int Hkv, int dk, int dv, int bs, int max_blocks,
                  int dtype, const int32_t *pairs, int n_pairs, int n_threads) {
    if (!out || !q || !k_cache || !block_tables || !context_lens) return ORACLE_BAD_ARG;
    if (Hkv <= 0 || Hq % Hkv != 0 || dk <= 0 || dv <= 0 || bs <= 0) return ORACLE_BAD_ARG;
    if (!v_cache && dv > dk) return ORACLE_BAD_ARG;
    const int64_t rows = pairs ? n_pairs : (int64_t)num_seqs * Hq;
    int err = ORACLE_OK;
    (void)n_threads;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 0 ? n_threads : 1)
    for (int64_t r = 0; r < rows; ++r) {
        const int b = pairs ? pairs[2 * r] : (int)(r / Hq);
        const int h = pairs ? pairs[2 * r + 1] : (int)(r % Hq);
        double *row = out + ((int64_t)b * Hq + h) * dv;
        int e = decode_row(row, q, k_cache, v_cache, block_tables, context_lens,
                           scale, b, h, Hq, Hkv, dk, dv, bs, max_blocks, dtype);
        if (e) {
#pragma omp critical
            err = e;
        }
    }
    return err;
}

int oracle_append(void *k_cache, void *v_cache, const void *k,
                  int64_t k_token_stride, const void *v, int64_t v_token_stride,
                  const int32_t *slot_mapping, int num_tokens, int num_blocks,
                  int bs, int Hkv, int dk, int dv, int elt_bytes) {
    if (!k_cache || !k || !slot_mapping) return ORACLE_BAD_ARG;
    if ((v_cache == NULL) != (v == NULL)) return ORACLE_BAD_ARG;
    const int64_t n_slots = (int64_t)num_blocks * bs;
    const size_t k_row = (size_t)Hkv * dk * elt_bytes;
    const size_t v_row = (size_t)Hkv * dv * elt_bytes;
    for (int i = 0; i < num_tokens; ++i)
        if (slot_mapping[i] != -1 && (slot_mapping[i] < 0 || slot_mapping[i] >= n_slots))
            return ORACLE_BAD_SLOT;
    for (int i = 0; i < num_tokens; ++i) {
        const int64_t s = slot_mapping[i];
        if (s == -1) continue;
        memcpy((char *)k_cache + s * k_row,
               (const char *)k + (int64_t)i * k_token_stride * elt_bytes, k_row);
        if (v_cache)
            memcpy((char *)v_cache + s * v_row,
                   (const char *)v + (int64_t)i * v_token_stride * elt_bytes, v_row);
    }
    return ORACLE_OK;
}
