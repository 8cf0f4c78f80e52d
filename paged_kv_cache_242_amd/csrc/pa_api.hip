// C ABI of libpa: argument validation, dispatch to the kernels, status codes and messages.
// Nothing here allocates device memory, synchronizes, or reads device buffers.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/pa.h"
#include "pa_kernels.h"

#define PA_VERSION_STRING "pa 0.1.0 (gfx950)"

namespace {

thread_local char g_last_error[512] = "";

pa_status fail(pa_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

pa_status ok() {
    g_last_error[0] = '\0';
    return PA_OK;
}

bool aligned16(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

int log2_exact(int x) {
    int s = 0;
    while ((1 << s) < x) ++s;
    return (1 << s) == x ? s : -1;
}

int elt_bytes(int32_t dtype) { return dtype == PA_DTYPE_F32 ? 4 : 2; }

bool fp8_cache(const pa_layer *L) { return L->kv_cache_dtype == PA_KV_CACHE_FP8_E4M3; }

// Bytes of one element of the paged cache.
int cache_elt_bytes(const pa_layer *L) { return fp8_cache(L) ? 1 : elt_bytes(L->dtype); }

// Kernel element code: the dtype, or 3 / 4 for bf16 / fp16 layers with an FP8 cache.
int kernel_dtype(const pa_layer *L) { return fp8_cache(L) ? L->dtype + 2 : L->dtype; }

pa_status check_layer(const pa_layer *L, const char *fn) {
    if (!L) return fail(PA_ERR_INVALID_ARGUMENT, "%s: layer is NULL", fn);
    if (L->num_heads <= 0 || L->num_kv_heads <= 0)
        return fail(PA_ERR_INVALID_ARGUMENT, "%s: num_heads (%d) and num_kv_heads (%d) must be positive", fn,
                    L->num_heads, L->num_kv_heads);
    if (L->num_heads % L->num_kv_heads != 0)
        return fail(PA_ERR_INVALID_ARGUMENT, "%s: num_kv_heads (%d) must divide num_heads (%d)", fn, L->num_kv_heads,
                    L->num_heads);
    if (L->dtype != PA_DTYPE_F32 && L->dtype != PA_DTYPE_BF16 && L->dtype != PA_DTYPE_F16)
        return fail(PA_ERR_UNSUPPORTED, "%s: dtype %d is not supported (fp32 = 0, bf16 = 1, fp16 = 2)", fn,
                    L->dtype);
    if (L->head_size != 64 && L->head_size != 128 && L->head_size != 256)
        return fail(PA_ERR_UNSUPPORTED, "%s: head size %d is not supported; supported head sizes are 64, 128 and 256",
                    fn, L->head_size);
    const int bs_shift = log2_exact(L->block_size);
    if (L->block_size < 8 || L->block_size > 256 || bs_shift < 0)
        return fail(PA_ERR_UNSUPPORTED, "%s: block size %d is not supported (powers of two from 8 to 256)", fn,
                    L->block_size);
    if (L->num_blocks <= 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: num_blocks must be positive", fn);
    if (L->num_blocks > (int64_t(1) << 31))
        return fail(PA_ERR_INVALID_ARGUMENT, "%s: num_blocks %lld exceeds int32 block ids", fn,
                    (long long)L->num_blocks);
    if (int64_t(L->block_size) * L->num_kv_heads * L->head_size * 4 >= (int64_t(1) << 31))
        return fail(PA_ERR_UNSUPPORTED, "%s: one cache block (block_size * num_kv_heads * head_size elements) must "
                    "stay below 2^31 bytes", fn);
    if (!(L->scale == L->scale)) return fail(PA_ERR_INVALID_ARGUMENT, "%s: scale is NaN", fn);
    if (!(L->logits_soft_cap == L->logits_soft_cap) || L->logits_soft_cap > 3.0e38f)
        return fail(PA_ERR_INVALID_ARGUMENT, "%s: logits_soft_cap must be finite", fn);
    if (L->kv_cache_dtype != PA_KV_CACHE_AUTO && L->kv_cache_dtype != PA_KV_CACHE_FP8_E4M3)
        return fail(PA_ERR_UNSUPPORTED, "%s: kv_cache_dtype %d is not supported (auto = 0, fp8 e4m3 = 1)", fn,
                    L->kv_cache_dtype);
    if (fp8_cache(L) && !(L->k_scale > 0.f && L->k_scale <= 3.0e38f && L->v_scale > 0.f && L->v_scale <= 3.0e38f))
        return fail(PA_ERR_INVALID_ARGUMENT, "%s: fp8 cache scales must be finite and > 0 (k_scale %g, v_scale %g)",
                    fn, double(L->k_scale), double(L->v_scale));
    return PA_OK;
}

// Query rows per sequence that multi-token decode takes (1 + speculative tokens).
constexpr int32_t kMaxQueryLen = 64;

pa_status decode_impl(const char *fn, const pa_layer *layer, void *out, const void *query, int64_t q_row_stride,
                      const void *kv_cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
                      const int32_t *seq_lens, int32_t num_seqs, int32_t query_len, int32_t max_seq_len,
                      void *workspace, size_t workspace_bytes, void *stream);

// ---- pa_decode_noalloc: the decode workspace lives in a fixed device array instead of caller
// memory.  Every GPU the library runs on holds its own copy of `scratch` (at its own address) until
// the process ends.  In host code the name is only a stand-in for the symbol, never a device
// address: the address is looked up once per device with hipGetSymbolAddress, with that device
// current, and only that address is passed to kernels.
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];

pa_status scratch_address(const char *fn, void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(PA_ERR_UNSUPPORTED, "%s: device %d out of range", fn, dev);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(PA_ERR_HIP, "%s: hipGetSymbolAddress of the scratch array failed on device %d: %s", fn, dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return PA_OK;
}

}  // namespace

extern "C" {

const char *pa_version(void) { return PA_VERSION_STRING; }

const char *pa_last_error_message(void) { return g_last_error; }

const char *pa_status_string(pa_status status) {
    switch (status) {
        case PA_OK: return "PA_OK";
        case PA_ERR_INVALID_ARGUMENT: return "PA_ERR_INVALID_ARGUMENT";
        case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
        case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
        case PA_ERR_HIP: return "PA_ERR_HIP";
    }
    return "PA_ERR_UNKNOWN";
}

pa_status pa_cache_write(const pa_layer *layer, const void *key, const void *value, int64_t kv_row_stride,
                         int64_t num_tokens, const int64_t *slot_mapping, void *kv_cache, void *stream) {
    const char *fn = "pa_cache_write";
    pa_status st = check_layer(layer, fn);
    if (st != PA_OK) return st;
    if (num_tokens < 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: num_tokens is negative", fn);
    if (num_tokens == 0) return ok();
    if (!key || !value || !slot_mapping || !kv_cache)
        return fail(PA_ERR_INVALID_ARGUMENT, "%s: key, value, slot_mapping and kv_cache must be non-NULL", fn);
    const int eb = elt_bytes(layer->dtype);
    const int64_t row = int64_t(layer->num_kv_heads) * layer->head_size;
    if (kv_row_stride < row)
        return fail(PA_ERR_INVALID_ARGUMENT, "%s: kv_row_stride %lld < num_kv_heads * head_size %lld", fn,
                    (long long)kv_row_stride, (long long)row);
    if (!aligned16(key) || !aligned16(value) || !aligned16(kv_cache) || (kv_row_stride * eb) % 16 != 0)
        return fail(PA_ERR_INVALID_ARGUMENT, "%s: key/value/kv_cache must be 16-byte aligned with 16-byte row strides",
                    fn);
    const int cb = cache_elt_bytes(layer);
    pa::CacheWriteParams p;
    p.key = static_cast<const char *>(key);
    p.value = static_cast<const char *>(value);
    p.kv_stride_bytes = kv_row_stride * eb;
    p.num_tokens = num_tokens;
    p.slot_mapping = slot_mapping;
    p.kv_cache = static_cast<char *>(kv_cache);
    p.num_slots = layer->num_blocks * layer->block_size;
    p.row_bytes = int32_t(row * cb);
    p.plane_bytes = p.num_slots * p.row_bytes;
    p.fp8 = fp8_cache(layer) ? 1 : 0;
    p.src_dtype = layer->dtype;
    p.k_scale = layer->k_scale;
    p.v_scale = layer->v_scale;
    hipError_t e = pa::launch_cache_write(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

pa_status pa_copy_blocks(const pa_layer *layer, void *const *kv_caches, int32_t num_layers, const int64_t *block_pairs,
                         int64_t num_pairs, void *stream) {
    const char *fn = "pa_copy_blocks";
    pa_status st = check_layer(layer, fn);
    if (st != PA_OK) return st;
    if (num_layers < 0 || num_pairs < 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: negative count", fn);
    if (num_layers == 0 || num_pairs == 0) return ok();
    if (!kv_caches || !block_pairs) return fail(PA_ERR_INVALID_ARGUMENT, "%s: kv_caches and block_pairs must be non-NULL", fn);
    if ((reinterpret_cast<uintptr_t>(kv_caches) & 7) != 0)
        return fail(PA_ERR_INVALID_ARGUMENT, "%s: kv_caches must be 8-byte aligned", fn);
    if ((reinterpret_cast<uintptr_t>(block_pairs) & 7) != 0)
        return fail(PA_ERR_INVALID_ARGUMENT, "%s: block_pairs must be 8-byte aligned", fn);
    pa::CopyBlocksParams p;
    p.caches = kv_caches;
    p.pairs = block_pairs;
    p.num_pairs = num_pairs;
    p.num_blocks = layer->num_blocks;
    p.block_bytes = int64_t(layer->block_size) * layer->num_kv_heads * layer->head_size * cache_elt_bytes(layer);
    p.plane_bytes = p.num_blocks * p.block_bytes;
    hipError_t e = pa::launch_copy_blocks(p, num_layers, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

pa_status pa_swap_blocks(const pa_layer *layer, const void *src_cache, int64_t src_num_blocks, void *dst_cache,
                         int64_t dst_num_blocks, const int64_t *block_pairs, int64_t num_pairs, void *stream) {
    const char *fn = "pa_swap_blocks";
    pa_status st = check_layer(layer, fn);
    if (st != PA_OK) return st;
    if (num_pairs < 0 || src_num_blocks <= 0 || dst_num_blocks <= 0)
        return fail(PA_ERR_INVALID_ARGUMENT, "%s: num_pairs must be >= 0 and the block counts > 0", fn);
    if (num_pairs == 0) return ok();
    if (!src_cache || !dst_cache || !block_pairs)
        return fail(PA_ERR_INVALID_ARGUMENT, "%s: src_cache, dst_cache and block_pairs must be non-NULL", fn);
    for (int64_t i = 0; i < num_pairs; ++i) {
        const int64_t s = block_pairs[2 * i], d = block_pairs[2 * i + 1];
        if (s < 0 || s >= src_num_blocks || d < 0 || d >= dst_num_blocks)
            return fail(PA_ERR_INVALID_ARGUMENT, "%s: pair %lld (%lld -> %lld) out of range (%lld / %lld blocks)", fn,
                        (long long)i, (long long)s, (long long)d, (long long)src_num_blocks,
                        (long long)dst_num_blocks);
    }
    const int64_t bb = int64_t(layer->block_size) * layer->num_kv_heads * layer->head_size * cache_elt_bytes(layer);
    const char *src = static_cast<const char *>(src_cache);
    char *dst = static_cast<char *>(dst_cache);
    hipStream_t s_ = static_cast<hipStream_t>(stream);
    // runs of pairs (s, d), (s + 1, d + 1), ... go out as one copy per plane
    for (int64_t i = 0; i < num_pairs;) {
        const int64_t s0 = block_pairs[2 * i], d0 = block_pairs[2 * i + 1];
        int64_t n = 1;
        while (i + n < num_pairs && block_pairs[2 * (i + n)] == s0 + n && block_pairs[2 * (i + n) + 1] == d0 + n) ++n;
        for (int pl = 0; pl < 2; ++pl) {
            hipError_t e = hipMemcpyAsync(dst + (pl * dst_num_blocks + d0) * bb, src + (pl * src_num_blocks + s0) * bb,
                                          size_t(n * bb), hipMemcpyDefault, s_);
            if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: hipMemcpyAsync failed: %s", fn, hipGetErrorString(e));
        }
        i += n;
    }
    return ok();
}

size_t pa_decode_workspace_size(const pa_layer *layer, int32_t num_seqs, int32_t max_seq_len) {
    return pa_decode_multi_workspace_size(layer, num_seqs, 1, max_seq_len);
}

size_t pa_decode_multi_workspace_size(const pa_layer *layer, int32_t num_seqs, int32_t query_len, int32_t max_seq_len) {
    if (check_layer(layer, "pa_decode_workspace_size") != PA_OK || num_seqs <= 0 || max_seq_len < 0 || query_len < 1 ||
        query_len > kMaxQueryLen)
        return 0;
    return pa::plan_decode(layer->num_heads, layer->num_kv_heads, layer->head_size, layer->block_size, kernel_dtype(layer),
                           num_seqs, max_seq_len, query_len)
        .workspace_bytes;
}

pa_status pa_decode(const pa_layer *layer, void *out, const void *query, int64_t q_row_stride, const void *kv_cache,
                    const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *seq_lens,
                    int32_t num_seqs, int32_t max_seq_len, void *workspace, size_t workspace_bytes, void *stream) {
    return decode_impl("pa_decode", layer, out, query, q_row_stride, kv_cache, block_tables, max_blocks_per_seq,
                       seq_lens, num_seqs, 1, max_seq_len, workspace, workspace_bytes, stream);
}

pa_status pa_decode_noalloc(const pa_layer *layer, void *out, const void *query, int64_t q_row_stride,
                            const void *kv_cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
                            const int32_t *seq_lens, int32_t num_seqs, int32_t max_seq_len, void *stream) {
    const char *fn = "pa_decode_noalloc";
    pa_status st = check_layer(layer, fn);
    if (st != PA_OK) return st;
    void *ws = nullptr;
    if (num_seqs > 0 && max_seq_len >= 0) {
        const size_t need = pa_decode_workspace_size(layer, num_seqs, max_seq_len);
        if (need > kScratchBytes)
            return fail(PA_ERR_WORKSPACE,
                        "%s: %d sequences need %zu bytes of decode scratch, more than the %zu-byte device array; "
                        "use pa_decode with a caller workspace",
                        fn, num_seqs, need, kScratchBytes);
        if (need > 0) {
            st = scratch_address(fn, &ws);
            if (st != PA_OK) return st;
        }
    }
    return decode_impl(fn, layer, out, query, q_row_stride, kv_cache, block_tables, max_blocks_per_seq, seq_lens,
                       num_seqs, 1, max_seq_len, ws, ws ? kScratchBytes : 0, stream);
}

pa_status pa_decode_multi(const pa_layer *layer, void *out, const void *query, int64_t q_row_stride,
                          const void *kv_cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
                          const int32_t *seq_lens, int32_t num_seqs, int32_t query_len, int32_t max_seq_len,
                          void *workspace, size_t workspace_bytes, void *stream) {
    return decode_impl("pa_decode_multi", layer, out, query, q_row_stride, kv_cache, block_tables, max_blocks_per_seq,
                       seq_lens, num_seqs, query_len, max_seq_len, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

pa_status decode_impl(const char *fn, const pa_layer *layer, void *out, const void *query, int64_t q_row_stride,
                      const void *kv_cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
                      const int32_t *seq_lens, int32_t num_seqs, int32_t query_len, int32_t max_seq_len,
                      void *workspace, size_t workspace_bytes, void *stream) {
    pa_status st = check_layer(layer, fn);
    if (st != PA_OK) return st;
    if (query_len < 1 || query_len > kMaxQueryLen)
        return fail(PA_ERR_INVALID_ARGUMENT, "%s: query_len %d outside [1, %d]", fn, query_len, kMaxQueryLen);
    if (fp8_cache(layer) && layer->dtype == PA_DTYPE_F32)
        return fail(PA_ERR_UNSUPPORTED, "%s: an fp8 cache needs a bf16 or fp16 layer", fn);
    if (num_seqs < 0 || max_seq_len < 0 || max_blocks_per_seq < 0)
        return fail(PA_ERR_INVALID_ARGUMENT, "%s: num_seqs, max_seq_len and max_blocks_per_seq must be >= 0", fn);
    if (num_seqs == 0) return ok();
    if (!out || !query || !kv_cache || !block_tables || !seq_lens)
        return fail(PA_ERR_INVALID_ARGUMENT, "%s: out, query, kv_cache, block_tables and seq_lens must be non-NULL",
                    fn);
    if (max_blocks_per_seq == 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: max_blocks_per_seq must be positive", fn);
    const int eb = elt_bytes(layer->dtype);
    const int64_t qrow = int64_t(layer->num_heads) * layer->head_size;
    if (q_row_stride < qrow)
        return fail(PA_ERR_INVALID_ARGUMENT, "%s: q_row_stride %lld < num_heads * head_size %lld", fn,
                    (long long)q_row_stride, (long long)qrow);
    if (!aligned16(out) || !aligned16(query) || !aligned16(kv_cache) || (q_row_stride * eb) % 16 != 0)
        return fail(PA_ERR_INVALID_ARGUMENT, "%s: out/query/kv_cache must be 16-byte aligned with 16-byte row strides",
                    fn);
    const pa::DecodePlan plan = pa::plan_decode(layer->num_heads, layer->num_kv_heads, layer->head_size,
                                                layer->block_size, kernel_dtype(layer), num_seqs, max_seq_len,
                                                query_len);
    if (plan.workspace_bytes > 0) {
        if (!workspace || workspace_bytes < plan.workspace_bytes)
            return fail(PA_ERR_WORKSPACE, "%s: needs %zu bytes of workspace, got %zu", fn, plan.workspace_bytes,
                        workspace ? workspace_bytes : size_t(0));
        if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
            return fail(PA_ERR_INVALID_ARGUMENT, "%s: workspace must be 256-byte aligned", fn);
    }
    // Multi-token decode whose query rows times the query heads of a KV head exceed one head group:
    // the decode kernels would read every K/V byte once per group, so the rows go to the MFMA
    // prefill kernel instead, as a chunked prefill whose keys all come from the cache.
    if (query_len > 1 && layer->dtype != PA_DTYPE_F32 && plan.head_groups > 1) {
        if (int64_t(num_seqs) * query_len > 0x7fffffff)
            return fail(PA_ERR_INVALID_ARGUMENT, "%s: num_seqs * query_len exceeds int32", fn);
        pa::PrefillParams q{};
        q.out = out;
        q.query = query;
        q.q_stride = q_row_stride;
        q.key = nullptr;
        q.value = nullptr;
        q.kv_stride = int64_t(layer->num_kv_heads) * layer->head_size;
        q.k_cache = kv_cache;
        q.v_cache = static_cast<const char *>(kv_cache) + layer->num_blocks * layer->block_size *
                                                              int64_t(layer->num_kv_heads) * layer->head_size *
                                                              cache_elt_bytes(layer);
        q.block_tables = block_tables;
        q.max_blocks = max_blocks_per_seq;
        q.context_lens = nullptr;
        q.cu_subquery = nullptr;
        q.num_seqs = num_seqs;
        q.num_tokens = int64_t(num_seqs) * query_len;
        q.num_heads = layer->num_heads;
        q.num_kv_heads = layer->num_kv_heads;
        q.block_shift = log2_exact(layer->block_size);
        q.num_blocks = layer->num_blocks;
        q.scale = layer->scale;
        q.alibi_slopes = layer->alibi_slopes;
        q.window = layer->sliding_window;
        q.softcap = layer->logits_soft_cap > 0.f ? layer->logits_soft_cap : 0.f;
        q.sinks = layer->sinks;
        q.max_subquery_len = query_len;
        q.max_context_len = max_seq_len;
        q.k_scale = layer->k_scale;
        q.v_scale = layer->v_scale;
        q.uniform_qlen = query_len;
        q.seq_lens = seq_lens;
        hipError_t e = pa::launch_prefill(q, kernel_dtype(layer), layer->head_size, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
        return ok();
    }
    pa::DecodeParams p;
    p.out = out;
    p.query = query;
    p.q_stride = q_row_stride;
    p.k_cache = kv_cache;
    p.v_cache = static_cast<const char *>(kv_cache) + layer->num_blocks * layer->block_size *
                                                          int64_t(layer->num_kv_heads) * layer->head_size *
                                                          cache_elt_bytes(layer);
    p.block_tables = block_tables;
    p.max_blocks = max_blocks_per_seq;
    p.seq_lens = seq_lens;
    p.num_seqs = num_seqs;
    p.num_heads = layer->num_heads;
    p.num_kv_heads = layer->num_kv_heads;
    p.block_shift = log2_exact(layer->block_size);
    p.num_blocks = layer->num_blocks;
    // an FP8 cache's k_scale folds into the score scale, its v_scale into the output
    p.scale = fp8_cache(layer) ? layer->scale * layer->k_scale : layer->scale;
    p.out_scale = fp8_cache(layer) ? layer->v_scale : 1.f;
    p.alibi_slopes = layer->alibi_slopes;
    p.window = layer->sliding_window;
    p.softcap = layer->logits_soft_cap > 0.f ? layer->logits_soft_cap : 0.f;
    p.sinks = layer->sinks;
    p.max_seq_len = max_seq_len;
    p.qlen = query_len;
    char *ws = static_cast<char *>(workspace);
    p.ws_prefix = reinterpret_cast<int64_t *>(ws + plan.ws_prefix_off);
    p.ws_wseq = reinterpret_cast<int32_t *>(ws + plan.ws_wseq_off);
    p.ws_acc = reinterpret_cast<float *>(ws + plan.ws_acc_off);
    p.ws_ml = reinterpret_cast<float *>(ws + plan.ws_ml_off);
    hipError_t e = pa::launch_decode(p, plan, kernel_dtype(layer), layer->head_size, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

pa_status pa_prefill_varlen(const pa_layer *layer, void *out, const void *query, int64_t q_row_stride,
                            const void *key, const void *value, int64_t kv_row_stride, const void *kv_cache,
                            const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
                            const int32_t *cu_subquery, int32_t num_seqs, int64_t num_tokens,
                            int32_t max_subquery_len, int32_t max_context_len, void *stream) {
    const char *fn = "pa_prefill_varlen";
    pa_status st = check_layer(layer, fn);
    if (st != PA_OK) return st;
    if (fp8_cache(layer) && layer->dtype == PA_DTYPE_F32)
        return fail(PA_ERR_UNSUPPORTED, "%s: an fp8 cache needs a bf16 or fp16 layer", fn);
    if (num_seqs < 0 || num_tokens < 0 || max_subquery_len < 0 || max_context_len < 0 || max_blocks_per_seq < 0)
        return fail(PA_ERR_INVALID_ARGUMENT, "%s: sizes must be >= 0", fn);
    if (num_seqs == 0 || num_tokens == 0) return ok();
    if (num_tokens > 0x7fffffff) return fail(PA_ERR_INVALID_ARGUMENT, "%s: num_tokens exceeds int32", fn);
    if (!out || !query || !key || !value || !cu_subquery)
        return fail(PA_ERR_INVALID_ARGUMENT, "%s: out, query, key, value and cu_subquery must be non-NULL", fn);
    if (max_context_len > 0 && (!kv_cache || !block_tables || !context_lens || max_blocks_per_seq == 0))
        return fail(PA_ERR_INVALID_ARGUMENT,
                    "%s: a cached context (max_context_len > 0) needs kv_cache, block_tables, context_lens and "
                    "max_blocks_per_seq > 0",
                    fn);
    const int eb = elt_bytes(layer->dtype);
    const int64_t qrow = int64_t(layer->num_heads) * layer->head_size;
    const int64_t kvrow = int64_t(layer->num_kv_heads) * layer->head_size;
    if (q_row_stride < qrow || kv_row_stride < kvrow)
        return fail(PA_ERR_INVALID_ARGUMENT, "%s: row strides smaller than the rows", fn);
    if (!aligned16(out) || !aligned16(query) || !aligned16(key) || !aligned16(value) ||
        (kv_cache && !aligned16(kv_cache)) || (q_row_stride * eb) % 16 != 0 || (kv_row_stride * eb) % 16 != 0)
        return fail(PA_ERR_INVALID_ARGUMENT, "%s: buffers must be 16-byte aligned with 16-byte row strides", fn);
    if (max_subquery_len == 0) return ok();
    pa::PrefillParams p;
    p.out = out;
    p.query = query;
    p.q_stride = q_row_stride;
    p.key = key;
    p.value = value;
    p.kv_stride = kv_row_stride;
    p.k_cache = kv_cache;
    p.v_cache = kv_cache ? static_cast<const char *>(kv_cache) +
                               layer->num_blocks * layer->block_size * kvrow * cache_elt_bytes(layer)
                         : nullptr;
    const bool has_ctx = max_context_len > 0;
    p.block_tables = has_ctx ? block_tables : nullptr;
    p.max_blocks = has_ctx ? max_blocks_per_seq : 0;
    p.context_lens = has_ctx ? context_lens : nullptr;
    p.cu_subquery = cu_subquery;
    p.num_seqs = num_seqs;
    p.num_tokens = num_tokens;
    p.num_heads = layer->num_heads;
    p.num_kv_heads = layer->num_kv_heads;
    p.block_shift = log2_exact(layer->block_size);
    p.num_blocks = layer->num_blocks;
    p.scale = layer->scale;
    p.alibi_slopes = layer->alibi_slopes;
    p.window = layer->sliding_window;
    p.softcap = layer->logits_soft_cap > 0.f ? layer->logits_soft_cap : 0.f;
    p.sinks = layer->sinks;
    p.max_subquery_len = max_subquery_len;
    p.max_context_len = max_context_len;
    p.k_scale = layer->k_scale;
    p.v_scale = layer->v_scale;
    p.uniform_qlen = 0;
    p.seq_lens = nullptr;
    hipError_t e = pa::launch_prefill(p, kernel_dtype(layer), layer->head_size, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

}  // extern "C"
