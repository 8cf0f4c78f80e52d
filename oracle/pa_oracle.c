/*
 * pa_oracle.c -- plain, slow, fp64 CPU oracle for attention over a paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or calls this
 * file; only the tests, the smoke check and the benchmark's CPU-baseline leg use it.  It
 * shares no source, header, table or helper with the GPU library.
 *
 * What it computes, and where each step comes from (the three pages of the reference):
 *
 *  - Cache layout.  Both pages give the paged cache the shape
 *    [2, num_blocks, block_size * num_kv_heads * head_size] (aphrodite-engine
 *    "xformers.py", XFormersImpl.forward docstring; vLLM "cpu_attn",
 *    TorchSDPABackendImpl.forward docstring).  Plane 0 holds keys, plane 1 values.  The
 *    order of the elements inside one block is not printed anywhere; this oracle reads
 *    the flat factor list literally, row-major [block_size][num_kv_heads][head_size].
 *    That choice is a contract, not something the pages pin.
 *
 *  - Slot mapping.  A token's slot s lives in block s / block_size at offset
 *    s % block_size (vLLM "cpu_attn", TorchSDPAMetadata.slot_mapping comment and its
 *    worked example).  A negative slot marks a padded token that is not written.
 *
 *  - Block tables.  Row i maps logical block n of sequence i to a physical block
 *    (vLLM "cpu_attn", TorchSDPAMetadata.decode_block_tables comment).
 *
 *  - Lengths.  In decode, the sequence length counts the new token, whose K/V is already
 *    in the cache; in prefill, context_len counts only cached tokens before the new
 *    subquery tokens (aphrodite-engine "xformers.py", XFormersMetadata NOTE/WARNING).
 *
 *  - Grouped-query heads: query head h reads KV head h / (H / Hkv)
 *    (aphrodite-engine "xformers.py", _run_memory_efficient_xformers_forward view into
 *    [Hkv, H/Hkv]; vLLM "cpu_attn", _run_sdpa_forward repeat_interleave).
 *
 *  - Scores: scale * <q, k_j>, plus slope_h * (j - pos) when ALiBi slopes are given
 *    (aphrodite-engine "xformers.py", _make_alibi_bias: bias is key index minus query
 *    index, times the head's slope, added to the scaled logits).  Key j is visible to
 *    the query at absolute position pos when j <= pos (causal) and, with a sliding
 *    window W > 0, when pos - j < W.  The pages never print the window helper; "W keys
 *    including the query's own" is this oracle's reading.  ALiBi and the window are
 *    both applied when both are given (the pages drop the window under ALiBi; the
 *    built method takes both).
 *
 *  - Softmax attention in fp64: m = max s_j, p_j = exp(s_j - m), out = sum p_j v_j /
 *    sum p_j (vLLM "cpu_attn", _run_sdpa_forward, scaled_dot_product_attention).
 *
 *  - Logits soft-cap and attention sinks.  The pages only name them: a logits_soft_cap
 *    argument of the backend constructor (vLLM "cpu_attn", TorchSDPABackendImpl.__init__,
 *    which warns that SDPA ignores it) and per-layer logits_soft_cap / has_sinks parameters
 *    (vLLM "utils" page, PerLayerParameters).  Readings taken here:
 *      soft-cap c > 0: the scaled dot product x = scale * <q, k_j> becomes c * tanh(x / c)
 *      before the ALiBi bias and the mask; c <= 0 leaves it alone;
 *      sink sigma_h: one extra logit per query head that joins the softmax normalisation
 *      but carries no value, so out = sum_j e^(s_j) v_j / (e^(sigma_h) + sum_j e^(s_j)).
 *
 *  - fp8 KV cache.  The pages pass a kv_cache_dtype and per-tensor scales to the cache write
 *    and to the attention calls (aphrodite-engine "xformers.py", write_to_paged_cache and
 *    forward_decode with kv_cache_dtype and kv_scale; vLLM "cpu_attn", write_to_paged_cache and
 *    forward_decode with layer._k_scale and layer._v_scale) but never show the encoding.
 *    Reading taken here: kv_cache_dtype 1 stores OCP FP8 E4M3 codes (1 sign, 4 exponent bits
 *    with bias 7, 3 fraction bits, no infinities, S.1111.111 = NaN, largest finite 448); a key
 *    element x is stored as the code nearest to the fp32 quotient fp32(x) / k_scale (ties to
 *    the even code, magnitudes above 448 saturate to 448, NaN stays NaN), a value element with
 *    v_scale; attention reads code_value * k_scale (or v_scale) in fp64.
 *
 * Inputs are promoted exactly to double: fp32 directly, bf16 by placing its 16 bits in
 * the high half of an fp32, fp16 from its sign, exponent and fraction fields.  Outputs are
 * double.  Element types: 0 = fp32, 1 = bf16, 2 = fp16 (the pages list all three as
 * supported dtypes: vLLM "cpu_attn", TorchSDPABackend.get_supported_dtypes).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_BAD_ARG 1
#define ORC_BAD_INDEX 2
#define ORC_NO_MEMORY 3

typedef struct {
    int32_t num_heads;      /* H */
    int32_t num_kv_heads;   /* Hkv, divides H */
    int32_t head_size;      /* D */
    int32_t block_size;     /* tokens per cache block */
    int64_t num_blocks;     /* physical blocks in each plane */
    int32_t dtype;          /* 0 = fp32, 1 = bf16, 2 = fp16 */
    float scale;            /* multiplies <q, k> */
    const float *alibi_slopes; /* [H] or NULL */
    int32_t sliding_window; /* <= 0: no window */
    float logits_soft_cap;  /* <= 0: no soft-cap */
    const float *sinks;     /* [H] sink logits, or NULL */
    int32_t kv_cache_dtype; /* 0: the cache holds dtype elements; 1: FP8 E4M3 codes */
    float k_scale;          /* fp8 cache: key element = code value * k_scale */
    float v_scale;          /* fp8 cache: value element = code value * v_scale */
} orc_layer;

static int elt_bytes(int32_t dtype) { return dtype == 0 ? 4 : 2; }

/* Bytes of one element of the paged cache. */
static int cache_elt_bytes(const orc_layer *L) { return L->kv_cache_dtype == 1 ? 1 : elt_bytes(L->dtype); }

/* Value of an FP8 E4M3 code (OCP "e4m3fn"). */
static double e4m3_to_double(uint8_t c)
{
    const int sign = c >> 7, e = (c >> 3) & 15, f = c & 7;
    double v;
    if (e == 15 && f == 7) v = NAN;
    else if (e == 0) v = ldexp((double)f, -9);             /* subnormal: f/8 * 2^-6 */
    else v = ldexp((double)(8 + f), e - 10);               /* (1 + f/8) * 2^(e-7) */
    return sign ? -v : v;
}

/* The E4M3 code nearest to x: ties go to the code with an even fraction, magnitudes above 448
 * saturate to 448, NaN gives the NaN code.  Found by scanning the 127 finite non-negative codes,
 * whose values the caller passes in (value[c] = e4m3_to_double(c)). */
static uint8_t float_to_e4m3(float x, const double *value)
{
    if (x != x) return signbit(x) ? 0xFF : 0x7F;
    const uint8_t sign = signbit(x) ? 0x80 : 0x00;
    const double a = fabs((double)x);
    if (a >= 448.0) return sign | 0x7E;
    int best = 0;
    double best_err = INFINITY;
    for (int c = 0; c < 127; ++c) {
        const double err = fabs(a - value[c]);
        if (err < best_err || (err == best_err && (c & 1) == 0)) {
            best = c;
            best_err = err;
        }
    }
    return sign | (uint8_t)best;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double half_to_double(uint16_t h)
{
    const int sign = h >> 15, e = (h >> 10) & 31, f = h & 1023;
    double v;
    if (e == 31) v = f ? NAN : INFINITY;
    else if (e == 0) v = ldexp((double)f, -24);            /* subnormal: f * 2^-24 */
    else v = ldexp((double)(1024 + f), e - 25);            /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* Exact promotion of one stored element to double. */
static double elt_to_double(const void *base, int64_t idx, int32_t dtype)
{
    if (dtype == 0) {
        return (double)((const float *)base)[idx];
    } else if (dtype == 2) {
        return half_to_double(((const uint16_t *)base)[idx]);
    } else {
        uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
}

/* Element offset, inside one cache plane, of (block, offset-in-block, kv head, dim). */
static int64_t cache_index(const orc_layer *L, int64_t block, int64_t offset, int64_t g, int64_t d)
{
    return ((block * L->block_size + offset) * L->num_kv_heads + g) * L->head_size + d;
}

static int layer_ok(const orc_layer *L)
{
    if (!L || L->num_heads <= 0 || L->num_kv_heads <= 0 || L->head_size <= 0 || L->block_size <= 0)
        return 0;
    if (L->num_heads % L->num_kv_heads != 0) return 0;
    if (L->dtype < 0 || L->dtype > 2) return 0;
    if (L->kv_cache_dtype != 0 && L->kv_cache_dtype != 1) return 0;
    if (L->kv_cache_dtype == 1 && !(L->k_scale > 0.0f && L->v_scale > 0.0f && isfinite(L->k_scale) &&
                                    isfinite(L->v_scale)))
        return 0;
    if (L->num_blocks < 0) return 0;
    return 1;
}

/*
 * Block moves (aphrodite-engine "xformers.py", XFormersBackend.copy_blocks and swap_blocks,
 * which hand a block map to the paged-attention ops).  One block of one plane is
 * block_size * num_kv_heads * head_size contiguous elements; a move carries both planes.
 *
 * copy_blocks: a map from a source block to a list of destination blocks, applied to the
 * cache of every layer in the list.  Here the map arrives flattened into (src, dst) pairs; a
 * pair naming a block outside [0, num_blocks) is skipped.  The pairs are applied in order.
 * swap_blocks: a map from source block to destination block between two caches (which may
 * hold different numbers of blocks); an index out of range is an error and nothing moves.
 */
static int64_t block_bytes(const orc_layer *L)
{
    return (int64_t)L->block_size * L->num_kv_heads * L->head_size * cache_elt_bytes(L);
}

int orc_copy_blocks(const orc_layer *L, void *const *caches, int32_t num_layers, const int64_t *pairs,
                    int64_t num_pairs)
{
    if (!layer_ok(L) || num_layers < 0 || num_pairs < 0) return ORC_BAD_ARG;
    if (num_layers > 0 && num_pairs > 0 && (!caches || !pairs)) return ORC_BAD_ARG;
    const int64_t bb = block_bytes(L);
    const int64_t plane = L->num_blocks * bb;
    for (int32_t l = 0; l < num_layers; ++l) {
        char *c = (char *)caches[l];
        if (!c) return ORC_BAD_ARG;
        for (int64_t i = 0; i < num_pairs; ++i) {
            const int64_t src = pairs[2 * i], dst = pairs[2 * i + 1];
            if (src < 0 || src >= L->num_blocks || dst < 0 || dst >= L->num_blocks) continue;
            for (int pl = 0; pl < 2; ++pl) memmove(c + pl * plane + dst * bb, c + pl * plane + src * bb, (size_t)bb);
        }
    }
    return ORC_OK;
}

int orc_swap_blocks(const orc_layer *L, const void *src_cache, int64_t src_blocks, void *dst_cache,
                    int64_t dst_blocks, const int64_t *pairs, int64_t num_pairs)
{
    if (!layer_ok(L) || src_blocks < 0 || dst_blocks < 0 || num_pairs < 0) return ORC_BAD_ARG;
    if (num_pairs > 0 && (!src_cache || !dst_cache || !pairs)) return ORC_BAD_ARG;
    for (int64_t i = 0; i < num_pairs; ++i) {
        const int64_t src = pairs[2 * i], dst = pairs[2 * i + 1];
        if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return ORC_BAD_INDEX;
    }
    const int64_t bb = block_bytes(L);
    for (int64_t i = 0; i < num_pairs; ++i) {
        const int64_t src = pairs[2 * i], dst = pairs[2 * i + 1];
        for (int pl = 0; pl < 2; ++pl)
            memcpy((char *)dst_cache + (pl * dst_blocks + dst) * bb,
                   (const char *)src_cache + (pl * src_blocks + src) * bb, (size_t)bb);
    }
    return ORC_OK;
}

/*
 * Cache write: for every token t whose slot s = slot_mapping[t] is >= 0, copy the bits of
 * key row t into the key plane at (s / block_size, s % block_size) and the bits of value
 * row t into the value plane at the same place.  key/value rows are num_kv_heads *
 * head_size elements long and row_stride elements apart.
 */
int orc_cache_write(const orc_layer *L, const void *key, const void *value, int64_t row_stride,
                    int64_t num_tokens, const int64_t *slot_mapping, void *kv_cache)
{
    if (!layer_ok(L) || num_tokens < 0) return ORC_BAD_ARG;
    const int eb = elt_bytes(L->dtype);
    const int cb = cache_elt_bytes(L);
    const int64_t plane = L->num_blocks * L->block_size * L->num_kv_heads * L->head_size;
    const int64_t row = (int64_t)L->num_kv_heads * L->head_size;
    char *kc = (char *)kv_cache;
    char *vc = kc + plane * cb;
    double e4m3_value[127];
    for (int c = 0; c < 127; ++c) e4m3_value[c] = e4m3_to_double((uint8_t)c);
    for (int64_t t = 0; t < num_tokens; ++t) {
        int64_t s = slot_mapping[t];
        if (s < 0) continue;
        int64_t block = s / L->block_size;
        int64_t offset = s % L->block_size;
        if (block >= L->num_blocks) return ORC_BAD_INDEX;
        for (int64_t g = 0; g < L->num_kv_heads; ++g) {
            for (int64_t d = 0; d < L->head_size; ++d) {
                int64_t src = t * row_stride + g * L->head_size + d;
                int64_t dst = cache_index(L, block, offset, g, d);
                if (L->kv_cache_dtype == 1) {
                    /* quantize: the fp32 quotient, then the nearest code */
                    const float kq = (float)elt_to_double(key, src, L->dtype) / L->k_scale;
                    const float vq = (float)elt_to_double(value, src, L->dtype) / L->v_scale;
                    ((uint8_t *)kc)[dst] = float_to_e4m3(kq, e4m3_value);
                    ((uint8_t *)vc)[dst] = float_to_e4m3(vq, e4m3_value);
                } else {
                    memcpy(kc + dst * eb, (const char *)key + src * eb, eb);
                    memcpy(vc + dst * eb, (const char *)value + src * eb, eb);
                }
            }
        }
    }
    (void)row;
    return ORC_OK;
}

/*
 * Un-page the first n tokens of one sequence for KV head g: logical token j lives in
 * physical block table_row[j / block_size] at offset j % block_size.  Writes n x D
 * doubles to K and V.
 */
static int unpage(const orc_layer *L, const void *kv_cache, const int32_t *table_row, int64_t n,
                  int64_t g, double *K, double *V)
{
    const int64_t plane = L->num_blocks * L->block_size * L->num_kv_heads * L->head_size;
    const char *kc = (const char *)kv_cache;
    const char *vc = kc + plane * cache_elt_bytes(L);
    for (int64_t j = 0; j < n; ++j) {
        int64_t block = table_row[j / L->block_size];
        int64_t offset = j % L->block_size;
        if (block < 0 || block >= L->num_blocks) return ORC_BAD_INDEX;
        for (int64_t d = 0; d < L->head_size; ++d) {
            int64_t idx = cache_index(L, block, offset, g, d);
            if (L->kv_cache_dtype == 1) {
                K[j * L->head_size + d] = e4m3_to_double(((const uint8_t *)kc)[idx]) * (double)L->k_scale;
                V[j * L->head_size + d] = e4m3_to_double(((const uint8_t *)vc)[idx]) * (double)L->v_scale;
            } else {
                K[j * L->head_size + d] = elt_to_double(kc, idx, L->dtype);
                V[j * L->head_size + d] = elt_to_double(vc, idx, L->dtype);
            }
        }
    }
    return ORC_OK;
}

/*
 * One query row of masked softmax attention.  K and V hold the sequence's keys and values
 * for this KV head, indexed by absolute token position 0 .. pos.  q is D doubles.  Writes
 * D doubles to out.
 */
static void attend_row(const orc_layer *L, const double *q, const double *K, const double *V,
                       int64_t pos, int64_t h, double *out)
{
    const int has_alibi = L->alibi_slopes != NULL;
    const double slope = has_alibi ? (double)L->alibi_slopes[h] : 0.0;
    const double cap = (double)L->logits_soft_cap;
    const int64_t D = L->head_size;
    const int64_t W = L->sliding_window;
    const int64_t first = (W > 0 && pos - W + 1 > 0) ? pos - W + 1 : 0;
    const int64_t n = pos - first + 1;
    double *s = (double *)malloc((size_t)n * sizeof(double));
    /* scores */
    double m = -INFINITY;
    for (int64_t j = first; j <= pos; ++j) {
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += q[d] * K[j * D + d];
        double sj = (double)L->scale * dot;
        if (cap > 0.0) sj = cap * tanh(sj / cap);
        if (has_alibi) sj += slope * (double)(j - pos);
        s[j - first] = sj;
        if (sj > m) m = sj;
    }
    /* softmax-weighted sum of values; a sink logit only adds to the denominator */
    double sink = -INFINITY;
    if (L->sinks) {
        sink = (double)L->sinks[h];
        if (sink > m) m = sink;
    }
    double denom = L->sinks ? exp(sink - m) : 0.0;
    for (int64_t d = 0; d < D; ++d) out[d] = 0.0;
    for (int64_t j = first; j <= pos; ++j) {
        double p = exp(s[j - first] - m);
        denom += p;
        for (int64_t d = 0; d < D; ++d) out[d] += p * V[j * D + d];
    }
    for (int64_t d = 0; d < D; ++d) out[d] /= denom;
    free(s);
}

static int set_threads(int num_threads)
{
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
    return omp_get_max_threads();
#else
    (void)num_threads;
    return 1;
#endif
}

/*
 * Single-token decode.  query row i ([H * D], row stride q_stride elements) attends to the
 * first seq_lens[i] tokens of sequence i, the last of which is the query's own position.
 * seq_lens[i] == 0 is a padded row and gives zeros.  out is [num_seqs, H, D] doubles.
 * Returns ORC_OK or an error code; *threads_used gets the thread count.
 */
int orc_decode(const orc_layer *L, double *out, const void *query, int64_t q_stride,
               const void *kv_cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
               const int32_t *seq_lens, int32_t num_seqs, int num_threads, int *threads_used)
{
    if (!layer_ok(L) || num_seqs < 0) return ORC_BAD_ARG;
    int nt = set_threads(num_threads);
    if (threads_used) *threads_used = nt;
    const int64_t H = L->num_heads, Hkv = L->num_kv_heads, D = L->head_size;
    const int64_t G = H / Hkv;
    int status = ORC_OK;
    for (int32_t i = 0; i < num_seqs; ++i) {
        if (seq_lens[i] < 0 || (int64_t)seq_lens[i] > (int64_t)max_blocks_per_seq * L->block_size)
            return ORC_BAD_INDEX;
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t work = 0; work < (int64_t)num_seqs * Hkv; ++work) {
        const int64_t i = work / Hkv, g = work % Hkv;
        const int64_t n = seq_lens[i];
        if (n == 0) {
            for (int64_t h = g * G; h < (g + 1) * G; ++h)
                for (int64_t d = 0; d < D; ++d) out[(i * H + h) * D + d] = 0.0;
            continue;
        }
        double *K = (double *)malloc((size_t)(n * D) * sizeof(double));
        double *V = (double *)malloc((size_t)(n * D) * sizeof(double));
        double *q = (double *)malloc((size_t)D * sizeof(double));
        if (!K || !V || !q) {
#pragma omp atomic write
            status = ORC_NO_MEMORY;
            free(K); free(V); free(q);
            continue;
        }
        int st = unpage(L, kv_cache, block_tables + i * max_blocks_per_seq, n, g, K, V);
        if (st != ORC_OK) {
#pragma omp atomic write
            status = st;
        } else {
            for (int64_t h = g * G; h < (g + 1) * G; ++h) {
                for (int64_t d = 0; d < D; ++d) q[d] = elt_to_double(query, i * q_stride + h * D + d, L->dtype);
                attend_row(L, q, K, V, n - 1, h, out + (i * H + h) * D);
            }
        }
        free(K); free(V); free(q);
    }
    return status;
}

/*
 * Multi-token decode (the utils page's uniform batches of 1 + speculative tokens treated as
 * decodes): sequence i has query_len query rows (rows i * query_len + t of query), all of whose
 * K/V are already in the cache; row t sits at position seq_lens[i] - query_len + t and attends
 * to the cached keys up to it.  seq_lens[i] == 0 is a padded sequence (zero rows); otherwise
 * seq_lens[i] >= query_len.  out is [num_seqs * query_len, H, D] doubles.  query_len == 1 is
 * orc_decode.
 */
int orc_decode_multi(const orc_layer *L, double *out, const void *query, int64_t q_stride,
                     const void *kv_cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
                     const int32_t *seq_lens, int32_t num_seqs, int32_t query_len, int num_threads,
                     int *threads_used)
{
    if (!layer_ok(L) || num_seqs < 0 || query_len < 1) return ORC_BAD_ARG;
    int nt = set_threads(num_threads);
    if (threads_used) *threads_used = nt;
    const int64_t H = L->num_heads, Hkv = L->num_kv_heads, D = L->head_size, Q = query_len;
    const int64_t G = H / Hkv;
    int status = ORC_OK;
    for (int32_t i = 0; i < num_seqs; ++i) {
        if (seq_lens[i] < 0 || (int64_t)seq_lens[i] > (int64_t)max_blocks_per_seq * L->block_size) return ORC_BAD_INDEX;
        if (seq_lens[i] != 0 && seq_lens[i] < query_len) return ORC_BAD_ARG;
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t work = 0; work < (int64_t)num_seqs * Hkv; ++work) {
        const int64_t i = work / Hkv, g = work % Hkv;
        const int64_t n = seq_lens[i];
        if (n == 0) {
            for (int64_t t = 0; t < Q; ++t)
                for (int64_t h = g * G; h < (g + 1) * G; ++h)
                    for (int64_t d = 0; d < D; ++d) out[((i * Q + t) * H + h) * D + d] = 0.0;
            continue;
        }
        double *K = (double *)malloc((size_t)(n * D) * sizeof(double));
        double *V = (double *)malloc((size_t)(n * D) * sizeof(double));
        double *q = (double *)malloc((size_t)D * sizeof(double));
        if (!K || !V || !q) {
#pragma omp atomic write
            status = ORC_NO_MEMORY;
            free(K); free(V); free(q);
            continue;
        }
        int st = unpage(L, kv_cache, block_tables + i * max_blocks_per_seq, n, g, K, V);
        if (st != ORC_OK) {
#pragma omp atomic write
            status = st;
        } else {
            for (int64_t t = 0; t < Q; ++t)
                for (int64_t h = g * G; h < (g + 1) * G; ++h) {
                    for (int64_t d = 0; d < D; ++d)
                        q[d] = elt_to_double(query, (i * Q + t) * q_stride + h * D + d, L->dtype);
                    attend_row(L, q, K, V, n - Q + t, h, out + ((i * Q + t) * H + h) * D);
                }
        }
        free(K); free(V); free(q);
    }
    return status;
}

/*
 * Variable-length causal prefill with a cached context.  Sequence i has context_lens[i]
 * cached tokens (reached through its block-table row) followed by the
 * n_i = cu_subquery[i+1] - cu_subquery[i] new tokens whose query/key/value rows are
 * cu_subquery[i] .. cu_subquery[i+1]-1 of the flattened inputs.  New token t of
 * sequence i sits at position c_i + t and attends to positions 0 .. c_i + t; keys below
 * c_i come from the cache, the rest from the key/value rows.  context_lens == NULL means
 * no cached context.  out is [num_tokens, H, D] doubles.  If row_select is non-NULL, only
 * rows with row_select[row] != 0 are computed (others are left untouched).
 */
int orc_prefill(const orc_layer *L, double *out, const void *query, int64_t q_stride,
                const void *key, const void *value, int64_t kv_stride, const void *kv_cache,
                const int32_t *block_tables, int32_t max_blocks_per_seq,
                const int32_t *context_lens, const int32_t *cu_subquery, int32_t num_seqs,
                const uint8_t *row_select, int num_threads, int *threads_used)
{
    if (!layer_ok(L) || num_seqs < 0) return ORC_BAD_ARG;
    int nt = set_threads(num_threads);
    if (threads_used) *threads_used = nt;
    const int64_t H = L->num_heads, Hkv = L->num_kv_heads, D = L->head_size;
    const int64_t G = H / Hkv;
    for (int32_t i = 0; i < num_seqs; ++i) {
        int64_t c = context_lens ? context_lens[i] : 0;
        if (c < 0 || cu_subquery[i + 1] < cu_subquery[i]) return ORC_BAD_ARG;
        if (c > 0 && (!block_tables || c > (int64_t)max_blocks_per_seq * L->block_size))
            return ORC_BAD_INDEX;
    }
    int status = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t work = 0; work < (int64_t)num_seqs * Hkv; ++work) {
        const int64_t i = work / Hkv, g = work % Hkv;
        const int64_t c = context_lens ? context_lens[i] : 0;
        const int64_t start = cu_subquery[i];
        const int64_t n_new = cu_subquery[i + 1] - start;
        if (n_new == 0) continue;
        int any = 0;
        for (int64_t t = 0; t < n_new; ++t)
            if (!row_select || row_select[start + t]) { any = 1; break; }
        if (!any) continue;
        const int64_t total = c + n_new;
        double *K = (double *)malloc((size_t)(total * D) * sizeof(double));
        double *V = (double *)malloc((size_t)(total * D) * sizeof(double));
        double *q = (double *)malloc((size_t)D * sizeof(double));
        if (!K || !V || !q) {
#pragma omp atomic write
            status = ORC_NO_MEMORY;
            free(K); free(V); free(q);
            continue;
        }
        int st = ORC_OK;
        /* cached context, un-paged through the block table */
        if (c > 0) st = unpage(L, kv_cache, block_tables + i * max_blocks_per_seq, c, g, K, V);
        /* new tokens, straight from the key/value rows */
        for (int64_t t = 0; t < n_new; ++t)
            for (int64_t d = 0; d < D; ++d) {
                K[(c + t) * D + d] = elt_to_double(key, (start + t) * kv_stride + g * D + d, L->dtype);
                V[(c + t) * D + d] = elt_to_double(value, (start + t) * kv_stride + g * D + d, L->dtype);
            }
        if (st != ORC_OK) {
#pragma omp atomic write
            status = st;
        } else {
            for (int64_t t = 0; t < n_new; ++t) {
                if (row_select && !row_select[start + t]) continue;
                for (int64_t h = g * G; h < (g + 1) * G; ++h) {
                    for (int64_t d = 0; d < D; ++d)
                        q[d] = elt_to_double(query, (start + t) * q_stride + h * D + d, L->dtype);
                    attend_row(L, q, K, V, c + t, h, out + ((start + t) * H + h) * D);
                }
            }
        }
        free(K); free(V); free(q);
    }
    return status;
}
