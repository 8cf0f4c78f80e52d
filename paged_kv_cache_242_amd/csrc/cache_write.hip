// Cache write: scatter each token's K and V row into its cache slot.
//
// A token's slot s lives in block s / block_size at offset s % block_size (vLLM "cpu_attn",
// TorchSDPAMetadata.slot_mapping worked example).  Because a block is row-major
// [block_size][num_kv_heads][head_size], the destination of a whole token is the single
// contiguous row starting at element s * num_kv_heads * head_size of the plane, so the copy is
// a row-to-row move of 16-byte chunks: coalesced loads of the source row, coalesced stores into
// the slot.  Bits are moved unchanged; no arithmetic touches the values -- except for an FP8
// E4M3 cache, where each element is quantized on the way (x / scale to the nearest code, ties to
// even, saturating at 448; the pages pass a kv_cache_dtype and scales to the cache write but do
// not define the encoding, this is the library's reading).
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

// FP8 E4M3 code of an fp32 value: nearest code, ties to the even code, magnitudes of 448 and
// above saturate to 448, NaN gives the NaN code.  Integer rounding of the fp32 bit pattern, so
// the result does not depend on a conversion instruction's rounding mode or overflow behaviour.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
    const uint32_t b = __float_as_uint(x);
    const uint32_t sign = (b >> 24) & 0x80u;
    const uint32_t a = b & 0x7fffffffu;
    if (a > 0x7f800000u) return sign | 0x7fu;                    // NaN
    if (a >= 0x43e00000u) return sign | 0x7eu;                   // |x| >= 448 (infinity included)
    if (a >= 0x3c800000u) {                                      // |x| >= 2^-6: normal codes
        // keep 3 fraction bits, round half to even; the exponent rebias is -120 (127 - 7)
        const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
        return sign | (r - (120u << 3));
    }
    // subnormal codes: multiples of 2^-9 (exact scaling, then round half to even)
    return sign | uint32_t(__builtin_rintf(__uint_as_float(a) * 512.f));
}

// Quantizing cache write: each thread turns groups of 8 consecutive elements of a K or V row
// into 8 E4M3 codes (one 8-byte store).  The quotient x / scale is an IEEE-rounded fp32
// division, as the codes must not depend on how the reciprocal is formed.
template <typename T>
__device__ __forceinline__ void load8(const char *src, float (&x)[8]) {
    if constexpr (sizeof(T) == 4) {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(src));
        const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(src) + 1);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[k] = a[k];
            x[4 + k] = b[k];
        }
    } else {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t w = v[k];
            if constexpr (kIsF16<T>) {
                x[2 * k] = f16_to_f32(f16_t(w & 0xffffu));
                x[2 * k + 1] = f16_to_f32(f16_t(w >> 16));
            } else {
                x[2 * k] = bf16_lo(w);
                x[2 * k + 1] = bf16_hi(w);
            }
        }
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void cache_write_fp8_kernel(CacheWriteParams p, int tokens_per_block,
                                                                    int groups_per_row) {
    const int per_token = 2 * groups_per_row;
    const int64_t first = int64_t(blockIdx.x) * tokens_per_block;
    const int total = tokens_per_block * per_token;
    for (int base = threadIdx.x; base < total; base += kThreads * kUnroll) {
        float x[kUnroll][8];
        int64_t slot[kUnroll];
        int64_t dst_off[kUnroll];
        bool live[kUnroll];
        int which[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int idx = base + u * kThreads;
            const int local = idx / per_token;
            const int rem = idx - local * per_token;
            which[u] = rem >= groups_per_row;
            const int grp = rem - which[u] * groups_per_row;
            const int64_t t = first + local;
            live[u] = idx < total && t < p.num_tokens;
            const int64_t tc = t < p.num_tokens ? t : p.num_tokens - 1;
            load8<T>((which[u] ? p.value : p.key) + tc * p.kv_stride_bytes + int64_t(grp) * 8 * sizeof(T), x[u]);
            slot[u] = p.slot_mapping[tc];
            dst_off[u] = which[u] * p.plane_bytes + int64_t(grp) * 8;
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const float s = which[u] ? p.v_scale : p.k_scale;
            uint32_t c[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) c[e] = e4m3_code(x[u][e] / s);
            const uint2 w = make_uint2(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                                       c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24));
            const int64_t sl = slot[u];
            if (live[u] && sl >= 0 && sl < p.num_slots)
                *reinterpret_cast<uint2 *>(p.kv_cache + dst_off[u] + sl * p.row_bytes) = w;
        }
    }
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteParams &p, hipStream_t stream) {
    if (p.fp8) {
        const int groups = p.row_bytes / 8;
        int tokens_per_block = kThreads * kUnroll / (2 * groups);
        if (tokens_per_block < 1) tokens_per_block = 1;
        const int64_t blocks = (p.num_tokens + tokens_per_block - 1) / tokens_per_block;
        if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
        const dim3 nb = dim3(unsigned(blocks)), nt = dim3(kThreads);
        if (p.src_dtype == 0)
            hipLaunchKernelGGL(cache_write_fp8_kernel<float>, nb, nt, 0, stream, p, tokens_per_block, groups);
        else if (p.src_dtype == 2)
            hipLaunchKernelGGL(cache_write_fp8_kernel<f16_t>, nb, nt, 0, stream, p, tokens_per_block, groups);
        else
            hipLaunchKernelGGL(cache_write_fp8_kernel<bf16_t>, nb, nt, 0, stream, p, tokens_per_block, groups);
        return hipGetLastError();
    }
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
