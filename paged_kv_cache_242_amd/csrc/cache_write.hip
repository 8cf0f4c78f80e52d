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
constexpr int kUnroll = 4;      // 16-byte chunks in flight per thread

// A workgroup moves `tokens_per_block` whole tokens (K row then V row, 16-byte chunks, chunk
// index idx = token * 2 * chunks_per_row + which * chunks_per_row + chunk); thread x takes chunks
// x, x + 256, ...  Each thread first issues up to kUnroll source loads (they do not depend on the
// slot), then looks up the slots and stores, so several loads per thread are in flight instead of
// one load-store round trip at a time.
__global__ __launch_bounds__(kThreads) void cache_write_kernel(CacheWriteParams p, int tokens_per_block,
                                                                int chunks_per_row) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const int per_token = 2 * chunks_per_row;
    const int64_t first = int64_t(blockIdx.x) * tokens_per_block;
    const int total = tokens_per_block * per_token;
    for (int base = threadIdx.x; base < total; base += kThreads * kUnroll) {
        u32x4 v[kUnroll];
        int64_t slot[kUnroll];
        int64_t dst_off[kUnroll];   // destination byte offset of the chunk inside its plane row
        bool live[kUnroll];
        // loads are unconditional (a chunk past the end re-reads one of the last token) so that
        // they all stay in flight together
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int idx = base + u * kThreads;
            const int local = idx / per_token;
            const int rem = idx - local * per_token;
            const int which = rem >= chunks_per_row;           // 0 = key, 1 = value
            const int chunk = rem - which * chunks_per_row;
            const int64_t t = first + local;
            live[u] = idx < total && t < p.num_tokens;
            const int64_t tc = t < p.num_tokens ? t : p.num_tokens - 1;
            const char *src = (which ? p.value : p.key) + tc * p.kv_stride_bytes + int64_t(chunk) * 16;
            v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src));
            slot[u] = p.slot_mapping[tc];
            dst_off[u] = which * p.plane_bytes + int64_t(chunk) * 16;
        }
        __builtin_amdgcn_sched_barrier(0);      // every load issues before the first slot test
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t sl = slot[u];
            if (live[u] && sl >= 0 && sl < p.num_slots)          // else padded token or out-of-range slot
                *reinterpret_cast<u32x4 *>(p.kv_cache + dst_off[u] + sl * p.row_bytes) = v[u];
        }
    }
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteParams &p, hipStream_t stream) {
    const int chunks = p.row_bytes / 16;
    int tokens_per_block = kThreads * kUnroll / (2 * chunks);
    if (tokens_per_block < 1) tokens_per_block = 1;
    const int64_t blocks = (p.num_tokens + tokens_per_block - 1) / tokens_per_block;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(cache_write_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, stream, p, tokens_per_block,
                       chunks);
    return hipGetLastError();
}

}  // namespace pa
