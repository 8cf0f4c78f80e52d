// Block copy inside the caches of several layers (copy-on-write of shared blocks).
//
// aphrodite-engine "xformers.py", XFormersBackend.copy_blocks: a map from a source block to a
// list of destination blocks, applied to the cache of every layer.  The map arrives flattened to
// (src, dst) pairs.  One workgroup moves one pair of one layer, both planes, as 16-byte chunks;
// each thread issues kUnroll loads before its stores so several are in flight.  Bits move
// unchanged.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(CopyBlocksParams p) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const int64_t w = blockIdx.x;                         // w = layer * num_pairs + pair
    const int layer = int(w / p.num_pairs);
    const int64_t pair = w - int64_t(layer) * p.num_pairs;
    const int64_t src = p.pairs[2 * pair], dst = p.pairs[2 * pair + 1];
    if (src < 0 || src >= p.num_blocks || dst < 0 || dst >= p.num_blocks) return;   // skipped pair
    char *base = reinterpret_cast<char *>(p.caches[layer]);
    const char *from = base + src * p.block_bytes;
    char *to = base + dst * p.block_bytes;
    const int64_t chunks = p.block_bytes / 16;            // per plane
    const int64_t total = 2 * chunks;
    for (int64_t i0 = threadIdx.x; i0 < total; i0 += kThreads * kUnroll) {
        u32x4 v[kUnroll];
        int64_t off[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = min(i0 + int64_t(u) * kThreads, total - 1);   // past the end: re-read the last chunk
            const int64_t pl = i >= chunks;
            off[u] = pl * p.plane_bytes + (i - pl * chunks) * 16;
            v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(from + off[u]));
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            if (i0 + int64_t(u) * kThreads < total) *reinterpret_cast<u32x4 *>(to + off[u]) = v[u];
    }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyBlocksParams &p, int32_t num_layers, hipStream_t stream) {
    const int64_t blocks = int64_t(num_layers) * p.num_pairs;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace pa
