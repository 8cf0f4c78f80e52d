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
    int32_t row_bytes;        // num_kv_heads * head_size * elt, multiple of 16
};
hipError_t launch_cache_write(const CacheWriteParams &p, hipStream_t stream);

// Split-KV policy shared by pa_decode and pa_decode_workspace_size.
struct DecodePlan {
    int32_t head_groups;      // query heads of one KV head are processed in this many groups
    int32_t heads_per_group;  // real heads per group (<= 8)
    int32_t padded_group;     // heads_per_group rounded up to 1, 2, 4 or 8
    int32_t part_size;        // keys per split-KV partition (multiple of 256, <= 128 blocks)
    int32_t num_parts;        // partitions of the longest sequence
    size_t workspace_bytes;   // 0 when num_parts == 1
};
DecodePlan plan_decode(int32_t num_heads, int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                       int32_t num_seqs, int32_t max_seq_len);

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
    int32_t num_heads;
    int32_t num_kv_heads;
    int32_t block_shift;      // log2(block_size)
    int64_t num_blocks;
    float scale;
    const float *alibi_slopes;
    int32_t window;
    float *ws_acc;            // [B, H, num_parts, D]
    float *ws_ml;             // [B, H, num_parts, 2]
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
    int32_t max_subquery_len;
    int32_t max_context_len;
};
hipError_t launch_prefill(const PrefillParams &p, int dtype, int head_size, hipStream_t stream);

}  // namespace pa
