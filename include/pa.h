/*
 * pa.h -- attention over a paged KV cache on AMD Instinct MI355X (gfx950).
 *
 * A plain C ABI: every argument is a scalar, a host pointer to a small struct, or a device
 * pointer.  The library (libpa.so) never allocates device memory, never synchronizes the
 * device and never reads device buffers on the host; all work is enqueued on the HIP stream
 * the caller passes (NULL = the legacy default stream).  Calls are reentrant: the only
 * global state is a per-device attribute cache, a thread-local error message and the fixed
 * scratch array that pa_decode_noalloc uses in place of a workspace.
 *
 * The problem statement follows the reference pages:
 *   - query  [num_tokens, num_heads * head_size]
 *   - key, value [num_tokens, num_kv_heads * head_size]
 *   - kv_cache [2, num_blocks, block_size * num_kv_heads * head_size]
 *     (aphrodite-engine "xformers.py", XFormersImpl.forward docstring; vLLM "cpu_attn",
 *     TorchSDPABackendImpl.forward docstring).
 *
 * Cache layout (a contract of this library; the pages print only the flat size): plane 0
 * holds keys, plane 1 values; inside a plane, element (block b, offset o, kv head g, dim d)
 * is at ((b * block_size + o) * num_kv_heads + g) * head_size + d, i.e. each block is
 * row-major [block_size][num_kv_heads][head_size] and one token's K (or V) is one
 * contiguous row of num_kv_heads * head_size elements.
 *
 * Masking and bias, shared by decode and prefill: a query at absolute position pos of its
 * sequence sees key j when j <= pos and, with sliding_window W > 0, pos - j < W (W keys
 * including its own).  Scores are scale * <q, k_j>, plus alibi_slopes[h] * (j - pos) when
 * slopes are given (aphrodite-engine "xformers.py", _make_alibi_bias).  ALiBi and the window
 * compose.  Query head h reads KV head h / (num_heads / num_kv_heads) (grouped-query
 * attention; aphrodite-engine "xformers.py", _run_memory_efficient_xformers_forward).
 *
 * Optional logits soft-cap and attention sinks (named on the pages -- vLLM "cpu_attn",
 * TorchSDPABackendImpl.__init__ logits_soft_cap; vLLM "utils", PerLayerParameters
 * logits_soft_cap and has_sinks -- but not defined there; these are this library's readings):
 * with a cap c > 0 the scaled dot product x = scale * <q, k_j> becomes c * tanh(x / c), and the
 * ALiBi bias and the mask apply after it; a sink sigma_h is one extra logit of query head h
 * that joins the softmax denominator only: out = sum_j e^(s_j) v_j / (e^(sigma_h) + sum_j e^(s_j)).
 *
 * Numerics: products and softmax in fp32; for bf16 and fp16 layers the softmax weights are
 * rounded to the element type (nearest even) before they multiply V, and outputs are rounded to
 * nearest even.  Over an fp8 cache the codes enter the products exactly and the scales are
 * applied in fp32, except in prefill at head size 256 with both ALiBi and a soft-cap, where
 * cached V rows are staged as code * v_scale rounded to the element type.
 *
 * Errors: every entry point returns a pa_status and launches nothing when it fails.  Only
 * host-visible scalars and pointers are validated.  Device contents (slots, block ids,
 * lengths, start locations) are preconditions; values out of range never cause an access
 * outside the buffers described here (they are clamped or skipped), but the affected rows'
 * results are unspecified.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_INVALID_ARGUMENT = 1, /* a NULL pointer, a negative size, a misaligned buffer, a bad geometry */
    PA_ERR_UNSUPPORTED = 2,      /* a head size, block size or dtype the library has no kernel for */
    PA_ERR_WORKSPACE = 3,        /* decode workspace missing or smaller than pa_decode_workspace_size() */
    PA_ERR_HIP = 4               /* a HIP runtime call or kernel launch failed */
} pa_status;

typedef enum pa_dtype {
    PA_DTYPE_F32 = 0,
    PA_DTYPE_BF16 = 1,
    PA_DTYPE_F16 = 2
} pa_dtype;

/*
 * Element type of the paged cache (the pages' kv_cache_dtype: aphrodite-engine "xformers.py",
 * write_to_paged_cache / forward_decode with kv_cache_dtype and kv_scale; vLLM "cpu_attn", the
 * same calls with layer._k_scale and layer._v_scale).  The pages do not define the fp8 encoding;
 * this library's reading: OCP FP8 E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 fraction
 * bits, no infinities, S.1111.111 = NaN, largest finite 448).  The cache write stores for a key
 * element x the code nearest to the fp32 quotient x / k_scale (IEEE division; ties to the even
 * code; magnitudes of 448 and above saturate to 448; NaN stays NaN), for a value element the
 * same with v_scale; attention reads code value * k_scale (or v_scale).  New tokens of a prefill
 * still come from the key/value rows of the call, at full precision.
 */
typedef enum pa_kv_cache_dtype {
    PA_KV_CACHE_AUTO = 0,        /* the cache holds elements of the layer dtype */
    PA_KV_CACHE_FP8_E4M3 = 1     /* the cache holds one-byte E4M3 codes */
} pa_kv_cache_dtype;

/*
 * Geometry of one attention layer; mirrors the backend constructor of the pages
 * (num_heads, head_size, scale, num_kv_heads, alibi_slopes, sliding_window).
 *   num_heads       H, > 0
 *   num_kv_heads    Hkv, > 0, divides H
 *   head_size       D: 64, 128 or 256 (others: PA_ERR_UNSUPPORTED)
 *   block_size      tokens per cache block: a power of two in [8, 256]
 *   num_blocks      physical blocks per plane, > 0
 *   dtype           PA_DTYPE_F32, PA_DTYPE_BF16 or PA_DTYPE_F16 (the cache, query, key, value
 *                   and out; vLLM "cpu_attn", TorchSDPABackend.get_supported_dtypes lists all
 *                   three)
 *   scale           fp32 multiplier of <q, k>
 *   alibi_slopes    device fp32 [H], or NULL for no ALiBi
 *   sliding_window  W; <= 0 disables the window
 *   logits_soft_cap c; <= 0 disables the soft-cap (NaN or infinity: PA_ERR_INVALID_ARGUMENT)
 *   sinks           device fp32 [H] sink logits, or NULL for none
 *   kv_cache_dtype  PA_KV_CACHE_AUTO or PA_KV_CACHE_FP8_E4M3 (then the cache is
 *                   [2, num_blocks, block_size * num_kv_heads * head_size] bytes)
 *   k_scale, v_scale  fp8 cache scales: finite and > 0 (ignored for PA_KV_CACHE_AUTO)
 */
typedef struct pa_layer {
    int32_t num_heads;
    int32_t num_kv_heads;
    int32_t head_size;
    int32_t block_size;
    int64_t num_blocks;
    int32_t dtype;
    float scale;
    const float *alibi_slopes;
    int32_t sliding_window;
    float logits_soft_cap;
    const float *sinks;
    int32_t kv_cache_dtype;
    float k_scale;
    float v_scale;
} pa_layer;

/*
 * Cache write: for every token t in [0, num_tokens) with s = slot_mapping[t] >= 0, copy
 * key row t into the key plane at block s / block_size, offset s % block_size, and value row
 * t into the value plane at the same place; bits are copied unchanged.  A negative slot is a
 * padded token and is skipped; a slot >= num_blocks * block_size is skipped too.  Duplicate
 * slots in one call leave an unspecified one of the rows.
 * (vLLM "cpu_attn", TorchSDPAMetadata.slot_mapping comment and worked example;
 * aphrodite-engine "xformers.py", XFormersImpl.forward, write_to_paged_cache.)
 *   key, value       device [num_tokens, num_kv_heads * head_size], rows kv_row_stride
 *                    elements apart (>= num_kv_heads * head_size); 16-byte aligned base
 *                    and row stride
 *   slot_mapping     device int64 [num_tokens]
 *   kv_cache         device, the whole [2, num_blocks, ...] cache, 16-byte aligned; mutated
 *                    in place
 * num_tokens == 0 returns PA_OK and launches nothing.
 */
pa_status pa_cache_write(const pa_layer *layer, const void *key, const void *value, int64_t kv_row_stride,
                         int64_t num_tokens, const int64_t *slot_mapping, void *kv_cache, void *stream);

/*
 * Bytes of device workspace pa_decode needs for this batch shape (> 0 whenever num_seqs > 0).
 * Depends on the layer's head counts, head size, block size and dtype, on num_seqs and on the
 * current device (its compute-unit count sizes the split); max_seq_len does not change it.
 * Returns 0 for invalid arguments or num_seqs <= 0.
 */
size_t pa_decode_workspace_size(const pa_layer *layer, int32_t num_seqs, int32_t max_seq_len);

/*
 * Single-token decode.  Row i of query attends, through block_tables row i, to the first
 * seq_lens[i] tokens of sequence i; seq_lens counts the new token, whose K/V must already be
 * in the cache, so the query's position is seq_lens[i] - 1.
 * (aphrodite-engine "xformers.py", XFormersMetadata NOTE on context_len and
 * XFormersImpl.forward, forward_decode; vLLM "cpu_attn", TorchSDPAMetadata.decode_seq_lens
 * and decode_block_tables comments.)
 *   out              device [num_seqs, num_heads * head_size], contiguous, written
 *   query            device [num_seqs, num_heads * head_size], rows q_row_stride elements
 *                    apart; 16-byte aligned
 *   kv_cache         device cache as above, read only
 *   block_tables     device int32 [num_seqs, max_blocks_per_seq]
 *   seq_lens         device int32 [num_seqs]; 0 marks a padded row, whose output is zeros
 *   max_seq_len      host upper bound of seq_lens (a larger device value is clamped to it
 *                    and to max_blocks_per_seq * block_size)
 *   workspace        device scratch of pa_decode_workspace_size() bytes, 256-byte aligned,
 *                    overwritten; calls that share one workspace must not overlap
 * The key tiles of all (sequence, KV head group) pairs are split evenly over as many wavefronts
 * as the device holds at once; a group is one KV head, or (VALU path, 16-bit or FP8 cache) 2 or
 * 4 adjacent KV heads read as one run per token where that count divides num_kv_heads and the
 * rows fit the wavefront's registers.  Each wavefront finds its share from seq_lens on the
 * device (above 2048 sequences a small planning kernel does it first); a pair cut between wavefronts leaves
 * (max, sum, weighted-V) partials that a second kernel merges with the log-sum-exp rule.  The
 * dot products run on the VALU, or on the matrix unit at head size 128 (block size >= 16) with
 * an FP8 cache and 5 to 32 query heads per KV head, or 9 to 32 query heads per KV head.
 */
pa_status pa_decode(const pa_layer *layer, void *out, const void *query, int64_t q_row_stride,
                    const void *kv_cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
                    const int32_t *seq_lens, int32_t num_seqs, int32_t max_seq_len, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * Decode without any allocation, for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses that forbid it).  The
 * same computation and kernels as pa_decode; the workspace is a fixed device array of
 * 32 MiB (33554432 bytes) inside the library, one per GPU, held until the process ends.
 *   Arguments as in pa_decode, without workspace / workspace_bytes.
 *   A batch whose pa_decode_workspace_size() exceeds 32 MiB returns PA_ERR_WORKSPACE and
 *   launches nothing (use pa_decode with a caller workspace for it).
 *   The array of the calling thread's current device is used; the stream must belong to that
 *   device.  Every call on one GPU shares that GPU's array: calls that overlap on one GPU (other
 *   streams, other host threads) race and give unspecified results.  Nothing in the array needs
 *   to start at zero; each call writes every byte it later reads.
 * No hipMalloc, hipFree or other allocating call is made; the array's device address is looked up
 * once per device (hipGetSymbolAddress) on the first call there.
 */
pa_status pa_decode_noalloc(const pa_layer *layer, void *out, const void *query, int64_t q_row_stride,
                            const void *kv_cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
                            const int32_t *seq_lens, int32_t num_seqs, int32_t max_seq_len, void *stream);

/*
 * Multi-token decode: the uniform batches of 1 + speculative tokens that the pages let a backend
 * treat as decodes (vLLM "utils", AttentionCGSupport.UNIFORM_BATCH and
 * _init_reorder_batch_threshold).  Every sequence has query_len query rows, rows
 * i * query_len .. i * query_len + query_len - 1 of query, whose K/V are already in the cache;
 * row t of sequence i sits at position seq_lens[i] - query_len + t and attends causally (with
 * the window, ALiBi, soft-cap and sinks as in decode) to the cached keys up to it.  The query
 * rows of a sequence and the query heads of a KV head ("virtual heads", query_len *
 * num_heads / num_kv_heads of them) share every K/V byte read: up to 8 of them (and for fp32
 * layers) on the decode kernels; 9 to 32 at head size 128 (block size >= 16) on the MFMA decode
 * kernel; beyond that, for bf16 and fp16 layers, on the MFMA prefill kernel (a chunked prefill of
 * query_len rows whose keys all come from the cache), which also shares each K/V tile among them.
 *   out              device [num_seqs * query_len, num_heads * head_size], contiguous, written
 *   query            device [num_seqs * query_len, ...], rows q_row_stride elements apart
 *   seq_lens         device int32 [num_seqs], counting every query row; 0 marks a padded
 *                    sequence (zero output rows); otherwise it must be >= query_len (rows
 *                    without a visible key have unspecified output)
 *   query_len        1 .. 64 (1 is pa_decode); other values: PA_ERR_INVALID_ARGUMENT
 *   workspace        pa_decode_multi_workspace_size(layer, num_seqs, query_len, max_seq_len) bytes
 * Other arguments as in pa_decode.
 */
size_t pa_decode_multi_workspace_size(const pa_layer *layer, int32_t num_seqs, int32_t query_len,
                                      int32_t max_seq_len);
pa_status pa_decode_multi(const pa_layer *layer, void *out, const void *query, int64_t q_row_stride,
                          const void *kv_cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
                          const int32_t *seq_lens, int32_t num_seqs, int32_t query_len, int32_t max_seq_len,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * Variable-length causal prefill with an optional cached context (chunked prefill).
 * Sequence i owns query/key/value rows cu_subquery[i] .. cu_subquery[i+1]-1 (its subquery
 * tokens) and has context_lens[i] tokens already in the cache before them.  Subquery token
 * t sits at position context_lens[i] + t and attends to positions 0 .. that position: keys
 * below context_lens[i] are read from the cache through block_tables row i, the others from
 * the key/value rows.
 * (aphrodite-engine "xformers.py", XFormersMetadata NOTE on context_len / subquery_len /
 * seqlen and subquery_start_loc, XFormersImpl.forward, forward_prefix and
 * _run_memory_efficient_xformers_forward; vLLM "cpu_attn", flash_attn_varlen_func call.)
 *   out              device [num_tokens, num_heads * head_size], contiguous, written
 *   query            device [num_tokens, ...], rows q_row_stride elements apart
 *   key, value       device [num_tokens, num_kv_heads * head_size], rows kv_row_stride apart
 *   kv_cache         device cache, read only; may be NULL when max_context_len == 0
 *   block_tables     device int32 [num_seqs, max_blocks_per_seq]; may be NULL when
 *                    max_context_len == 0
 *   context_lens     device int32 [num_seqs], or NULL for no cached context
 *   cu_subquery      device int32 [num_seqs + 1]: 0, then cumulative subquery lengths
 *                    (e.g. lengths [4, 6] give [0, 4, 10]); cu_subquery[num_seqs] == num_tokens
 *   max_subquery_len host upper bound of the subquery lengths (sizes the grid)
 *   max_context_len  host upper bound of context_lens (0 when there is no context)
 * All device pointers 16-byte aligned, row strides multiples of 16 bytes.
 * Workgroups of 4 wavefronts take up to 128 (query row, head) pairs of one KV head and stage
 * K/V tiles in LDS; the products run on the matrix unit (bf16 / fp16 MFMAs, fp32 MFMAs for
 * fp32 layers) with the softmax online in fp32.
 */
pa_status pa_prefill_varlen(const pa_layer *layer, void *out, const void *query, int64_t q_row_stride,
                            const void *key, const void *value, int64_t kv_row_stride, const void *kv_cache,
                            const int32_t *block_tables, int32_t max_blocks_per_seq,
                            const int32_t *context_lens, const int32_t *cu_subquery, int32_t num_seqs,
                            int64_t num_tokens, int32_t max_subquery_len, int32_t max_context_len,
                            void *stream);

/*
 * Block copy inside the caches of several layers (copy-on-write of blocks shared between
 * sequences): for every pair (src, dst) of block_pairs and every layer l, block src of both
 * planes of cache l is copied to block dst; bits are copied unchanged.
 * (aphrodite-engine "xformers.py", XFormersBackend.copy_blocks: a map from a source block to a
 * list of destination blocks over the list of per-layer caches; here flattened to pairs.)
 *   kv_caches    device array of num_layers device pointers, each a whole cache of this layer
 *                geometry ([2, num_blocks, ...], 16-byte aligned -- a device-side precondition)
 *   block_pairs  device int64 [num_pairs][2]: (src, dst).  A pair naming a block outside
 *                [0, num_blocks) is skipped.  A destination must not also be a source in the
 *                same call: the pairs are copied concurrently.
 * One kernel launch; num_layers == 0 or num_pairs == 0 returns PA_OK and launches nothing.
 */
pa_status pa_copy_blocks(const pa_layer *layer, void *const *kv_caches, int32_t num_layers,
                         const int64_t *block_pairs, int64_t num_pairs, void *stream);

/*
 * Block swap between two caches of one layer geometry, e.g. device and pinned host memory:
 * for every pair (src, dst) of block_pairs, block src of both planes of src_cache is copied to
 * block dst of dst_cache.  (aphrodite-engine "xformers.py", XFormersBackend.swap_blocks: a
 * source -> destination block map between two caches.)
 *   src_cache, dst_cache  whole caches [2, src_num_blocks, ...] and [2, dst_num_blocks, ...]
 *                         in device or host memory (host memory should be pinned for the
 *                         copies to be asynchronous); they must not overlap
 *   block_pairs           HOST int64 [num_pairs][2]: (src, dst), checked on the host; any
 *                         index out of range returns PA_ERR_INVALID_ARGUMENT and enqueues
 *                         nothing
 * Enqueued as hipMemcpyAsync copies on the stream, one per plane for every run of pairs
 * (s, d), (s + 1, d + 1), ...  A failure of the HIP runtime part way returns PA_ERR_HIP; copies
 * already enqueued stay enqueued.
 */
pa_status pa_swap_blocks(const pa_layer *layer, const void *src_cache, int64_t src_num_blocks, void *dst_cache,
                         int64_t dst_num_blocks, const int64_t *block_pairs, int64_t num_pairs, void *stream);

/* Static text for a status code. */
const char *pa_status_string(pa_status status);

/* Detail of the last failure on the calling thread ("" when none). */
const char *pa_last_error_message(void);

/* Library version string. */
const char *pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
