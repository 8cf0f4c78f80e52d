// Host-side launch interface between the C-ABI layer (pa_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

struct CacheWriteParams {
    const char *key;          // [T] rows of row_bytes, key_stride_bytes apart
    const char *value;
    int64_t kv_stride_bytes;
    int64_t num_tokens;
    const int64_t *slot_mapping;
    char *kv_cache;           // plane 0 (K) then plane 1 (V)
    int64_t plane_bytes;      // num_blocks * block_size * row_bytes
    int64_t num_slots;        // num_blocks * block_size
    int32_t row_bytes;        // cache row: num_kv_heads * head_size * cache element bytes, multiple of 8
    int32_t fp8;              // 1: quantize to FP8 E4M3 codes (cache element = 1 byte)
    int32_t src_dtype;        // element type of key/value (pa_dtype) when quantizing
    float k_scale, v_scale;   // quantization scales (fp8 only)
};
hipError_t launch_cache_write(const CacheWriteParams &p, hipStream_t stream);

struct CopyBlocksParams {
    void *const *caches;      // device array of per-layer cache bases
    const int64_t *pairs;     // device [num_pairs][2]: (src, dst)
    int64_t num_pairs;
    int64_t num_blocks;       // blocks per plane
    int64_t block_bytes;      // block_size * num_kv_heads * head_size * elt, multiple of 16
    int64_t plane_bytes;      // num_blocks * block_bytes
};
hipError_t launch_copy_blocks(const CopyBlocksParams &p, int32_t num_layers, hipStream_t stream);

// Decode policy shared by pa_decode and pa_decode_workspace_size.
struct DecodePlan {
    int32_t head_groups;      // query heads of one KV head are processed in this many groups
    int32_t heads_per_group;  // real heads per group (<= 8; <= 16 for the MFMA kernel)
    int32_t padded_group;     // heads_per_group rounded up to 1, 2, 4 or 8 (16 for the MFMA kernel)
    int32_t kv_per_unit;      // KV heads per work unit (1 or 2)
    int32_t units_per_seq;    // num_kv_heads / kv_per_unit * head_groups work units per sequence
    int32_t chunk;            // keys per block-id chunk
    int32_t tile;             // keys per tile of the kernel instance
    int32_t num_waves;        // wavefronts of the even split (resident at once on the device)
    int32_t mfma;             // 1: the MFMA kernel (one unit per sequence and KV head, <= 16 virtual heads)
    size_t ws_prefix_off, ws_wseq_off, ws_acc_off, ws_ml_off;   // workspace layout (bytes)
    size_t workspace_bytes;
};
// Kernel element codes (the `dtype` of plan_decode / launch_decode / launch_prefill): 0 fp32,
// 1 bf16, 2 fp16, 3 bf16 with an FP8 E4M3 cache, 4 fp16 with an FP8 E4M3 cache.
DecodePlan plan_decode(int32_t num_heads, int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                       int32_t dtype, int32_t num_seqs, int32_t max_seq_len, int32_t query_len);

struct DecodeParams {
    void *out;                // [B, H*D]
    const void *query;        // [B, q_stride]
    int64_t q_stride;         // elements
    const void *k_cache;      // plane 0
    const void *v_cache;      // plane 1
    const int32_t *block_tables;
    int32_t max_blocks;
    const int32_t *seq_lens;
    int32_t num_seqs;
    int32_t max_seq_len;
    int32_t num_heads;
    int32_t num_kv_heads;
    int32_t block_shift;      // log2(block_size)
    int64_t num_blocks;
    float scale;
    const float *alibi_slopes;
    int32_t window;
    float softcap;            // <= 0: off
    const float *sinks;       // [H] natural-log sink logits, or null
    float out_scale;          // multiplies the normalized output (an FP8 cache's v_scale, else 1)
    int32_t qlen;             // query rows per sequence (1: plain decode; more: multi-token decode)
    int64_t *ws_prefix;       // [B + 1] tiles of the work units of sequences before q
    int32_t *ws_wseq;         // [num_waves] sequence of each wavefront's first tile
    float *ws_acc;            // [slots, D] partial weighted V
    float *ws_ml;             // [slots, 2] partial (max, sum)
};
hipError_t launch_decode(const DecodeParams &p, const DecodePlan &plan, int dtype, int head_size,
                         hipStream_t stream);

struct PrefillParams {
    void *out;                // [T, H*D]
    const void *query;
    int64_t q_stride;
    const void *key;
    const void *value;
    int64_t kv_stride;
    const void *k_cache;
    const void *v_cache;
    const int32_t *block_tables;
    int32_t max_blocks;
    const int32_t *context_lens;
    const int32_t *cu_subquery;
    int32_t num_seqs;
    int64_t num_tokens;
    int32_t num_heads;
    int32_t num_kv_heads;
    int32_t block_shift;
    int64_t num_blocks;
    float scale;
    const float *alibi_slopes;
    int32_t window;
    float softcap;            // <= 0: off
    const float *sinks;       // [H] natural-log sink logits, or null
    int32_t max_subquery_len;
    int32_t max_context_len;
    float k_scale, v_scale;   // FP8 cache scales (element types 3 and 4)
    // Uniform multi-token mode (> 0, 16-bit kernels only): uniform_qlen query rows per sequence,
    // all keys in the cache, lengths from seq_lens (cu_subquery and context_lens unused).
    int32_t uniform_qlen;
    const int32_t *seq_lens;
};
hipError_t launch_prefill(const PrefillParams &p, int dtype, int head_size, hipStream_t stream);

}  // namespace pa
