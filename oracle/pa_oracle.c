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

/* ------------------------------------------------------------------------
 * MXFP8 KV cache (test infrastructure, like everything in this file).
 *
 * The CS336 lecture 10 notes ("第 10 讲：推理") list quantization as fewer
 * bytes, hence faster memory-bound decode, with fp8 among the formats
 * ("核心概念与定义"), and warn that one scale per tensor loses outlier
 * channels, naming blockwise scales with MXFP8 as the example ("常见陷阱");
 * the KV-cache page ("Cache KV, attention et optimisation de l'inference",
 * "Utilisez-le") serves with an fp8 KV cache.  MXFP8 is the OCP Microscaling
 * format: each block of 32 consecutive values shares one power-of-two scale
 * stored as an E8M0 byte (value 2^(e - 127), 0xFF = NaN) and each value is an
 * FP8 E4M3 byte (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
 * infinities; S.1111.111 is NaN, so the largest magnitude is 1.75 * 2^8 = 448).
 * Converting a block: X = floor(log2(max |v|)) - 8 (8 being the exponent of
 * E4M3's largest power of two), each v / 2^X rounded to the nearest E4M3
 * value, ties to even, saturating at +-448.
 *
 * Readings where the format leaves a choice: X is clamped to the E8M0 range
 * [-127, 127], and an all-zero block takes X = -127; inputs are finite.
 *
 * Cache layouts (one layer; a "row" is the head_dim values one token writes
 * for one KV head, cut into head_dim / 32 blocks):
 *   K codes   [num_blocks, Hkv, bs, d]     (token rows of a block and head)
 *   V codes   [num_blocks, Hkv, d, bs]     (the same tile, transposed)
 *   K, V scales [num_blocks, Hkv, bs, d / 32]
 * ------------------------------------------------------------------------ */

/* Value of an E4M3 byte (NaN for S.1111.111). */
double oracle_e4m3_value(uint8_t c) {
    const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    const double mag = e == 0 ? ldexp((double)m, -9)          /* m/8 * 2^-6 */
                              : ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
    return s ? -mag : mag;
}

/* Value of an E8M0 scale byte. */
double oracle_e8m0_value(uint8_t e) { return e == 255 ? NAN : ldexp(1.0, (int)e - 127); }

/* Nearest E4M3 byte to y, ties to even, saturating at +-448 (y finite). */
uint8_t oracle_e4m3_encode(double y) {
    const uint8_t sign = signbit(y) ? 0x80 : 0x00;
    const double a = fabs(y);
    if (a >= 448.0) return sign | 0x7E;
    int e2;
    frexp(a, &e2);             /* a in [2^(e2-1), 2^e2), or a == 0 */
    int ex = e2 - 1;           /* floor(log2 a) */
    if (a == 0.0 || ex < -6) ex = -6; /* subnormal range shares the quantum 2^-9 */
    const double quantum = ldexp(1.0, ex - 3);
    const double r = nearbyint(a / quantum) * quantum; /* ties to even (default mode) */
    if (r == 0.0) return sign;
    if (r < ldexp(1.0, -6)) return sign | (uint8_t)(r / ldexp(1.0, -9));
    frexp(r, &e2);
    const int er = e2 - 1;                                 /* r may have carried up a binade */
    const int m = (int)(r / ldexp(1.0, er - 3)) - 8;       /* 0..7 */
    return sign | (uint8_t)(((er + 7) << 3) | m);
}

/* Scale exponent X of a block of n values. */
static int mx_scale_exp(const double *v, int n) {
    double amax = 0.0;
    for (int i = 0; i < n; ++i)
        if (fabs(v[i]) > amax) amax = fabs(v[i]);
    if (amax == 0.0) return -127;
    int e2;
    frexp(amax, &e2);
    int x = (e2 - 1) - 8;
    if (x < -127) x = -127;
    if (x > 127) x = 127;
    return x;
}

/* Quantize one row of d values (d a multiple of 32) into d codes and d/32 scale bytes. */
static void mx_quantize_row(const double *v, int d, uint8_t *codes, uint8_t *scales) {
    for (int j = 0; j < d / 32; ++j) {
        const int x = mx_scale_exp(v + 32 * j, 32);
        scales[j] = (uint8_t)(x + 127);
        for (int i = 0; i < 32; ++i) codes[32 * j + i] = oracle_e4m3_encode(ldexp(v[32 * j + i], -x));
    }
}

/* rows x d inputs (float32 or bf16 bits, dtype 0/1) -> codes [rows, d], scales [rows, d/32]. */
int oracle_mx_quantize(const void *x, int dtype, int64_t rows, int d, uint8_t *codes,
                       uint8_t *scales) {
    if (!x || !codes || !scales || d <= 0 || d % 32 != 0) return ORACLE_BAD_ARG;
    double *buf = (double *)malloc(sizeof(double) * (size_t)d);
    if (!buf) return ORACLE_NO_MEM;
    for (int64_t r = 0; r < rows; ++r) {
        for (int i = 0; i < d; ++i) buf[i] = widen(x, r * d + i, dtype);
        mx_quantize_row(buf, d, codes + r * d, scales + r * (d / 32));
    }
    free(buf);
    return ORACLE_OK;
}

/*
 * Append into MXFP8 caches: for each token i with slot s != -1, p = s / bs,
 * r = s % bs, and each KV head h, the row k[i, h, :] is quantized into K codes
 * row (p, h, r) and its scales, and v[i, h, :] into column r of the V tile
 * (p, h) and its scales.  Nothing else changes.
 */
int oracle_append_mxfp8(uint8_t *k8, uint8_t *v8, uint8_t *ks, uint8_t *vs, const void *k,
                        int64_t k_token_stride, const void *v, int64_t v_token_stride,
                        const int32_t *slot_mapping, int num_tokens, int num_blocks, int bs,
                        int Hkv, int d, int dtype) {
    if (!k8 || !v8 || !ks || !vs || !k || !v || !slot_mapping) return ORACLE_BAD_ARG;
    if (d <= 0 || d % 32 != 0 || bs <= 0 || Hkv <= 0) return ORACLE_BAD_ARG;
    const int64_t n_slots = (int64_t)num_blocks * bs;
    for (int i = 0; i < num_tokens; ++i)
        if (slot_mapping[i] != -1 && (slot_mapping[i] < 0 || slot_mapping[i] >= n_slots))
            return ORACLE_BAD_SLOT;
    double *buf = (double *)malloc(sizeof(double) * (size_t)d);
    uint8_t *row = (uint8_t *)malloc((size_t)d);
    if (!buf || !row) {
        free(buf);
        free(row);
        return ORACLE_NO_MEM;
    }
    const int nsc = d / 32;
    for (int i = 0; i < num_tokens; ++i) {
        const int64_t s = slot_mapping[i];
        if (s == -1) continue;
        const int64_t p = s / bs;
        const int r = (int)(s % bs);
        for (int h = 0; h < Hkv; ++h) {
            const int64_t tile = p * Hkv + h;
            for (int e = 0; e < d; ++e) buf[e] = widen(k, (int64_t)i * k_token_stride + (int64_t)h * d + e, dtype);
            mx_quantize_row(buf, d, k8 + (tile * bs + r) * d, ks + (tile * bs + r) * nsc);
            for (int e = 0; e < d; ++e) buf[e] = widen(v, (int64_t)i * v_token_stride + (int64_t)h * d + e, dtype);
            mx_quantize_row(buf, d, row, vs + (tile * bs + r) * nsc);
            for (int e = 0; e < d; ++e) v8[(tile * d + e) * bs + r] = row[e];
        }
    }
    free(buf);
    free(row);
    return ORACLE_OK;
}

/* One (b, h) row of decode over MXFP8 caches: the plain definition of
 * oracle_decode with every cached value dequantized (code value * 2^X). */
static int decode_row_mxfp8(double *out_row, const void *q, const uint8_t *k8, const uint8_t *v8,
                            const uint8_t *ks, const uint8_t *vs, const int32_t *block_tables,
                            const int32_t *context_lens, double scale, int b, int h, int Hq,
                            int Hkv, int d, int bs, int max_blocks, int q_dtype) {
    const int G = Hq / Hkv;
    const int kvh = h / G;
    const int L = context_lens[b];
    const int nsc = d / 32;
    if (L <= 0) {
        for (int j = 0; j < d; ++j) out_row[j] = 0.0;
        return ORACLE_OK;
    }
    double *s = (double *)malloc(sizeof(double) * ((size_t)L + (size_t)d));
    if (!s) return ORACLE_NO_MEM;
    double *o = s + L;
    for (int j = 0; j < d; ++j) o[j] = 0.0;
    const int64_t q_off = ((int64_t)b * Hq + h) * d;
    for (int t = 0; t < L; ++t) {
        const int64_t tile = (int64_t)block_tables[(int64_t)b * max_blocks + t / bs] * Hkv + kvh;
        const int r = t % bs;
        double dot = 0.0;
        for (int i = 0; i < d; ++i) {
            const double kv = oracle_e4m3_value(k8[(tile * bs + r) * d + i]) *
                              oracle_e8m0_value(ks[(tile * bs + r) * nsc + i / 32]);
            dot += widen(q, q_off + i, q_dtype) * kv;
        }
        s[t] = dot * scale;
    }
    double smax = s[0];
    for (int t = 1; t < L; ++t)
        if (s[t] > smax) smax = s[t];
    double total = 0.0;
    for (int t = 0; t < L; ++t) {
        const double w = exp(s[t] - smax);
        total += w;
        const int64_t tile = (int64_t)block_tables[(int64_t)b * max_blocks + t / bs] * Hkv + kvh;
        const int r = t % bs;
        for (int j = 0; j < d; ++j)
            o[j] += w * oracle_e4m3_value(v8[(tile * d + j) * bs + r]) *
                    oracle_e8m0_value(vs[(tile * bs + r) * nsc + j / 32]);
    }
    for (int j = 0; j < d; ++j) out_row[j] = o[j] / total;
    free(s);
    return ORACLE_OK;
}

int oracle_decode_mxfp8(double *out, const void *q, const uint8_t *k8, const uint8_t *v8,
                        const uint8_t *ks, const uint8_t *vs, const int32_t *block_tables,
                        const int32_t *context_lens, double scale, int num_seqs, int Hq,
                        int Hkv, int d, int bs, int max_blocks, int q_dtype,
                        const int32_t *pairs, int n_pairs, int n_threads) {
    if (!out || !q || !k8 || !v8 || !ks || !vs || !block_tables || !context_lens)
        return ORACLE_BAD_ARG;
    if (Hkv <= 0 || Hq % Hkv != 0 || d <= 0 || d % 32 != 0 || bs <= 0) return ORACLE_BAD_ARG;
    const int64_t rows = pairs ? n_pairs : (int64_t)num_seqs * Hq;
    int err = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 0 ? n_threads : 1)
    for (int64_t r = 0; r < rows; ++r) {
        const int b = pairs ? pairs[2 * r] : (int)(r / Hq);
        const int h = pairs ? pairs[2 * r + 1] : (int)(r % Hq);
        int e = decode_row_mxfp8(out + ((int64_t)b * Hq + h) * d, q, k8, v8, ks, vs,
                                 block_tables, context_lens, scale, b, h, Hq, Hkv, d, bs,
                                 max_blocks, q_dtype);
        if (e) {
#pragma omp critical
            err = e;
        }
    }
    return err;
}

/* Element-wise oracle_e4m3_encode over n doubles. */
void oracle_e4m3_encode_array(const double *y, int64_t n, uint8_t *codes) {
    for (int64_t i = 0; i < n; ++i) codes[i] = oracle_e4m3_encode(y[i]);
}
