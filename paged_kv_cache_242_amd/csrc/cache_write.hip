// Cache write: scatter each token's K and V row into its cache slot.
//
// A token's slot s lives in block s / block_size at offset s % block_size (vLLM "cpu_attn",
// TorchSDPAMetadata.slot_mapping worked example).  Because a block is row-major
// [block_size][num_kv_heads][head_size], the destination of a whole token is the single
// contiguous row starting at element s * num_kv_heads * head_size of the plane, so the copy is
// a row-to-row move of 16-byte chunks: coalesced loads of the source row, coalesced stores into
// the slot.  Bits are moved unchanged; no arithmetic touches the values.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void cache_write_kernel(CacheWriteParams p, int tokens_per_block,
                                                                int chunks_per_row) {
    const int per_token = 2 * chunks_per_row;                  // K row then V row
    const int64_t first = int64_t(blockIdx.x) * tokens_per_block;
    const int total = tokens_per_block * per_token;
    for (int idx = threadIdx.x; idx < total; idx += kThreads) {
        const int local = idx / per_token;
        const int rem = idx - local * per_token;
        const int which = rem >= chunks_per_row;               // 0 = key, 1 = value
        const int chunk = rem - which * chunks_per_row;
        const int64_t t = first + local;
        if (t >= p.num_tokens) break;
        const int64_t s = p.slot_mapping[t];
        if (s < 0 || s >= p.num_slots) continue;               // padded token or out-of-range slot
        const char *src = (which ? p.value : p.key) + t * p.kv_stride_bytes + int64_t(chunk) * 16;
        char *dst = p.kv_cache + which * p.plane_bytes + s * p.row_bytes + int64_t(chunk) * 16;
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src));
        *reinterpret_cast<u32x4 *>(dst) = v;
    }
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteParams &p, hipStream_t stream) {
    const int chunks = p.row_bytes / 16;
    int tokens_per_block = kThreads / (2 * chunks);
    if (tokens_per_block < 1) tokens_per_block = 1;
    const int64_t blocks = (p.num_tokens + tokens_per_block - 1) / tokens_per_block;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(cache_write_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, stream, p, tokens_per_block,
                       chunks);
    return hipGetLastError();
}

}  // namespace pa
