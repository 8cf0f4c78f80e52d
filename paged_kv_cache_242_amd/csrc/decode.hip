// Single-token decode over the paged KV cache: split-KV partition kernel + merge kernel.
//
// What is computed (aphrodite-engine "xformers.py", XFormersImpl.forward / forward_decode and the
// XFormersMetadata note on context_len; vLLM "cpu_attn", TorchSDPAMetadata.decode_seq_lens and
// decode_block_tables): query row i, at position L_i - 1, attends to keys 0 .. L_i - 1 of its
// sequence (restricted to the last W with a sliding window), which are read through block-table
// row i; scores scale * <q, k_j> (+ slope_h * (j - pos) with ALiBi); softmax; weighted sum of V.
//
// Work decomposition.  One workgroup of 4 wavefronts handles one (sequence, KV head, group of up
// to 8 query heads, partition of part_size keys).  The query heads of a group share every K/V
// byte, so each byte read from HBM feeds all of them.  Wavefronts take 32-key tiles of the
// partition in turn and keep their own running (max, sum, weighted V); the four are merged in
// LDS at the end.  With more than one partition per sequence the merged partial triple goes to
// the workspace and decode_merge_kernel combines partitions with the log-sum-exp rule.
//
// Lane layout.  A head row of K or V is D elements = D*elt bytes, read as 16-byte chunks by C
// consecutive lanes; one load instruction covers R = 64 / C rows (4 rows of 256 B for bf16 at
// D = 128), so each instruction reads whole rows.  For Q.K every lane forms the partial dot
// products of its 8 elements with all GP query heads, then a butterfly over the C lanes of the
// row sums them.  The butterfly is "head-permuted": lane c keeps in register slot s the partial
// for head s ^ A(c), where A is the linear map that makes every exchange step a pure halving
// (lane keeps half of its values, adds the partner's matching half), so the reduction of GP
// dot products costs GP - 1 DPP adds instead of GP * log2(C); lane c ends with the full score of
// head A(c).  P.V runs in the same layout: each lane accumulates its 8 output elements for all
// GP heads over the rows it loaded (pairs of rows feed v_dot2_f32_bf16), reading the softmax
// weights that the score lanes left in LDS; row groups are summed once at the end.
//
// Numerics: fp32 dot products (bf16 pairs through v_dot2_f32_bf16), softmax in the base-2
// domain with fp32 exp2, weights rounded to bf16 before they multiply V, fp32 accumulation,
// output rounded to nearest even.
#include <math.h>

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kTile = 32;          // keys per wavefront tile
constexpr int kMaxGroup = 8;       // query heads per workgroup

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x >> 1); }
constexpr int cmin(int a, int b) { return a < b ? a : b; }

template <typename T, int D>
struct Geo {
    static constexpr int kC = D * int(sizeof(T)) / 16;   // lanes per head row
    static constexpr int kR = 64 / kC;                   // rows per load instruction
    static constexpr int kEpl = 16 / int(sizeof(T));     // elements per lane per row
    static constexpr int kNi = kTile / kR;               // load instructions per tile
    static constexpr int kSteps = ilog2(kC);
    static_assert(kC >= 8 && kC <= 64 && kR * kC == 64, "unsupported head geometry");
    static_assert(kNi % 2 == 0, "rows are paired for v_dot2");
};

// Head held by lane c after the head-permuted butterfly over C lanes with GP heads.  The
// exchange masks are m_k = C/2^k - 1 (k = 0 .. log2 C - 1); A(m_k) = GP / 2^(k+1) for the first
// log2 GP steps (halving) and 0 afterwards (plain all-reduce steps).  Since
// 2^i = m_{n-1-i} ^ m_{n-i} (with m_n = 0), A(c) is the xor of a_{n-1-i} ^ a_{n-i} over the set
// bits i of c.
template <int C, int GP>
__host__ __device__ constexpr int head_of_lane(int c) {
    constexpr int n = ilog2(C);
    constexpr int hs = cmin(ilog2(GP), n);
    int a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int k = 0; k < hs; ++k) a[k] = GP >> (k + 1);
    int r = 0;
    for (int i = 0; i < n; ++i)
        if ((c >> i) & 1) r ^= a[n - 1 - i] ^ a[n - i];
    return r;
}

// Lanes whose bits along the plain (non-halving) steps are zero hold one copy of each head.
template <int C, int GP>
__host__ __device__ constexpr int writer_mask() {
    constexpr int n = ilog2(C);
    constexpr int hs = cmin(ilog2(GP), n);
    return (1 << (n - hs)) - 1;
}

template <int C, int GP>
__host__ __device__ constexpr int lane_of_head(int h) {
    for (int c = 0; c < C; ++c)
        if ((c & writer_mask<C, GP>()) == 0 && head_of_lane<C, GP>(c) == h) return c;
    return -1;
}

template <int C, int GP, int K>
__device__ __forceinline__ void butterfly(float (&v)[GP]) {
    constexpr int n = ilog2(C);
    if constexpr (K < n) {
        constexpr int mask = (C >> K) - 1;
        constexpr int hs = cmin(ilog2(GP), n);
        if constexpr (K < hs) {
            constexpr int half = GP >> (K + 1);
#pragma unroll
            for (int s = 0; s < half; ++s) v[s] += lane_xor<mask>(v[s + half]);
        } else {
            v[0] += lane_xor<mask>(v[0]);
        }
        butterfly<C, GP, K + 1>(v);
    }
}

// Sum / max over the row groups (lanes c, c + C, c + 2C, ...).
template <int C>
__device__ __forceinline__ float sum_row_groups(float x) { return xor_sum_from<C>(x); }
template <int C>
__device__ __forceinline__ float max_row_groups(float x) { return xor_max_from<C>(x); }

struct DecodeShape {
    int part_size;
    int num_parts;
    int head_groups;
    int heads_per_group;
};

template <typename T>
__device__ __forceinline__ void store_out(T *dst, float v);
template <>
__device__ __forceinline__ void store_out<float>(float *dst, float v) { *dst = v; }
template <>
__device__ __forceinline__ void store_out<bf16_t>(bf16_t *dst, float v) { *dst = f32_to_bf16(v); }

// Partial dot products of one 16-byte row chunk with GP query chunks.
template <typename T, int GP>
__device__ __forceinline__ void chunk_dots(const uint4 &k, const uint32_t (&q)[GP][4], float (&part)[GP]) {
    const uint32_t kw[4] = {k.x, k.y, k.z, k.w};
#pragma unroll
    for (int s = 0; s < GP; ++s) {
        float acc = 0.f;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int w = 0; w < 4; ++w) acc = dot2_bf16(kw[w], q[s][w], acc);
        } else {
#pragma unroll
            for (int w = 0; w < 4; ++w) acc = fmaf(__uint_as_float(kw[w]), __uint_as_float(q[s][w]), acc);
        }
        part[s] = acc;
    }
}

template <typename T, int D, int GP>
__global__ __launch_bounds__(kThreads) void decode_partition_kernel(DecodeParams p, DecodeShape shape) {
    using Gm = Geo<T, D>;
    constexpr int C = Gm::kC, R = Gm::kR, EPL = Gm::kEpl, NI = Gm::kNi;
    constexpr int WMASK = writer_mask<C, GP>();

    // LDS: softmax weights of the current tile, per wavefront, [head][row group][instruction];
    // then the cross-wavefront merge buffers.
    __shared__ __align__(16) T p_lds[kWaves][GP][R][NI];
    __shared__ float red_acc[kWaves][GP][D];
    __shared__ float red_m[kWaves][GP];
    __shared__ float red_l[kWaves][GP];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane % C;
    const int r = lane / C;
    const int my_head = head_of_lane<C, GP>(c);

    int bid = blockIdx.x;
    const int part = bid % shape.num_parts;
    bid /= shape.num_parts;
    const int hgrp = bid % shape.head_groups;
    bid /= shape.head_groups;
    const int g = bid % p.num_kv_heads;
    const int seq = bid / p.num_kv_heads;

    const int group = p.num_heads / p.num_kv_heads;
    const int head0 = g * group + hgrp * shape.heads_per_group;
    const int nh = shape.heads_per_group;

    int L = p.seq_lens[seq];
    L = max(0, min(L, min(p.max_blocks << p.block_shift, shape.num_parts * shape.part_size)));
    const int lo = p.window > 0 ? max(0, L - p.window) : 0;
    const int pstart = part * shape.part_size;
    const int pend = min(pstart + shape.part_size, L);
    const int kb = max(pstart, lo);
    T *out_row = reinterpret_cast<T *>(p.out) + (int64_t(seq) * p.num_heads + head0) * D;

    if (kb >= pend) {
        if (L == 0 && shape.num_parts == 1)
            for (int idx = threadIdx.x; idx < nh * D; idx += kThreads) store_out<T>(out_row + idx, 0.f);
        return;
    }

    // Query chunks, head-permuted: slot s holds head s ^ my_head.
    uint32_t q[GP][4];
    {
        const T *qrow = reinterpret_cast<const T *>(p.query) + int64_t(seq) * p.q_stride + int64_t(head0) * D + c * EPL;
#pragma unroll
        for (int s = 0; s < GP; ++s) {
            const int hs = s ^ my_head;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (hs < nh) v = *reinterpret_cast<const uint4 *>(qrow + int64_t(hs) * D);
            q[s][0] = v.x; q[s][1] = v.y; q[s][2] = v.z; q[s][3] = v.w;
        }
    }

    const float qk_scale = p.scale * kLog2e;
    const float slope2 = (p.alibi_slopes != nullptr && my_head < nh) ? p.alibi_slopes[head0 + my_head] * kLog2e : 0.f;
    const int pos = L - 1;
    const int32_t *table = p.block_tables + int64_t(seq) * p.max_blocks;
    const int64_t row_elems = int64_t(p.num_kv_heads) * D;
    const int bmask = (1 << p.block_shift) - 1;
    const T *kbase = reinterpret_cast<const T *>(p.k_cache) + int64_t(g) * D + c * EPL;
    const T *vbase = reinterpret_cast<const T *>(p.v_cache) + int64_t(g) * D + c * EPL;

    float m_run = -INFINITY;   // base-2 running max of head my_head
    float l_run = 0.f;         // running sum of (rounded) weights of head my_head, this row group
    float acc[GP][EPL];
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;

    for (int tb = (kb / kTile) * kTile + wave * kTile; tb < pend; tb += kWaves * kTile) {
        // ---- gather K and V rows of this tile (16-byte loads, whole rows per instruction)
        uint4 kr[NI], vr[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int row0 = min(max(tb + i * R, lo), pos);            // uniform: block of this instruction
            int64_t blk = table[row0 >> p.block_shift];
            blk = blk < 0 ? 0 : (blk >= p.num_blocks ? p.num_blocks - 1 : blk);
            const int jl = min(max(tb + i * R + r, lo), pos);         // clamped row: always a written slot
            const int64_t off = ((blk << p.block_shift) + (jl & bmask)) * row_elems;
            kr[i] = *reinterpret_cast<const uint4 *>(kbase + off);
            vr[i] = *reinterpret_cast<const uint4 *>(vbase + off);
        }

        // ---- scores (base-2 domain) of head my_head for rows tb + i*R + r
        float sc[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            float part_dot[GP];
            chunk_dots<T, GP>(kr[i], q, part_dot);
            butterfly<C, GP, 0>(part_dot);
            const int j = tb + i * R + r;
            const float s2 = part_dot[0] * qk_scale + slope2 * float(j - pos);
            sc[i] = (j >= lo && j <= pos) ? s2 : -INFINITY;
        }

        // ---- online softmax
        float tmax = sc[0];
#pragma unroll
        for (int i = 1; i < NI; ++i) tmax = fmaxf(tmax, sc[i]);
        tmax = max_row_groups<C>(tmax);
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
        float psum = 0.f;
        T pv[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const float pf = (sc[i] == -INFINITY) ? 0.f : fast_exp2(sc[i] - m_new);
            if constexpr (sizeof(T) == 2) {
                pv[i] = f32_to_bf16(pf);
                psum += bf16_to_f32(pv[i]);
            } else {
                pv[i] = pf;
                psum += pf;
            }
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        if ((c & WMASK) == 0) {
#pragma unroll
            for (int i = 0; i < NI; ++i) p_lds[wave][my_head][r][i] = pv[i];
        }
        wave_lds_sync();

        // ---- rescale and P.V
#pragma unroll
        for (int h = 0; h < GP; ++h) {
            const float a = readlane_f(alpha, lane_of_head<C, GP>(h));
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] *= a;
        }
        if constexpr (sizeof(T) == 2) {
            // row pairs (i, i+1) -> per element e the bf16 pair (v_i[e], v_{i+1}[e])
            uint32_t vp[NI / 2][EPL];
#pragma unroll
            for (int ip = 0; ip < NI / 2; ++ip) {
                const uint4 a = vr[2 * ip], b = vr[2 * ip + 1];
                const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
                const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    vp[ip][2 * w] = interleave_lo(aw[w], bw[w]);
                    vp[ip][2 * w + 1] = interleave_hi(aw[w], bw[w]);
                }
            }
#pragma unroll
            for (int h = 0; h < GP; ++h) {
                uint32_t pp[NI / 2];
                const uint32_t *src = reinterpret_cast<const uint32_t *>(&p_lds[wave][h][r][0]);
#pragma unroll
                for (int ip = 0; ip < NI / 2; ++ip) pp[ip] = src[ip];
#pragma unroll
                for (int ip = 0; ip < NI / 2; ++ip)
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[h][e] = dot2_bf16(pp[ip], vp[ip][e], acc[h][e]);
            }
        } else {
#pragma unroll
            for (int h = 0; h < GP; ++h) {
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    const float pw = p_lds[wave][h][r][i];
                    const uint32_t vw[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pw, __uint_as_float(vw[e]), acc[h][e]);
                }
            }
        }
        wave_lds_sync();
    }

    // ---- merge row groups inside the wavefront, then wavefronts through LDS
    l_run = sum_row_groups<C>(l_run);
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = sum_row_groups<C>(acc[h][e]);
    if (r == 0) {
#pragma unroll
        for (int h = 0; h < GP; ++h)
#pragma unroll
            for (int e = 0; e < EPL; ++e) red_acc[wave][h][c * EPL + e] = acc[h][e];
        if ((c & WMASK) == 0) {
            red_m[wave][my_head] = m_run;
            red_l[wave][my_head] = l_run;
        }
    }
    __syncthreads();

    for (int idx = threadIdx.x; idx < nh * D; idx += kThreads) {
        const int h = idx / D;
        const int d = idx - h * D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_m[w][h]);
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = red_m[w][h];
            const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
            num += f * red_acc[w][h][d];
            den += f * red_l[w][h];
        }
        if (shape.num_parts == 1) {
            store_out<T>(out_row + idx, num / den);
        } else {
            const int64_t slot = (int64_t(seq) * p.num_heads + head0 + h) * shape.num_parts + part;
            p.ws_acc[slot * D + d] = num;
            if (d == 0) {
                p.ws_ml[slot * 2] = M;
                p.ws_ml[slot * 2 + 1] = den;
            }
        }
    }
}

// Merge of split-KV partials: out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeParams p, DecodeShape shape) {
    constexpr int PER = D / 64;
    const int lane = threadIdx.x;
    const int h = blockIdx.x % p.num_heads;
    const int seq = blockIdx.x / p.num_heads;
    T *out_row = reinterpret_cast<T *>(p.out) + (int64_t(seq) * p.num_heads + h) * D;
    int L = p.seq_lens[seq];
    L = max(0, min(L, min(p.max_blocks << p.block_shift, shape.num_parts * shape.part_size)));
    if (L == 0) {
#pragma unroll
        for (int k = 0; k < PER; ++k) store_out<T>(out_row + lane + 64 * k, 0.f);
        return;
    }
    const int lo = p.window > 0 ? max(0, L - p.window) : 0;
    const int p0 = lo / shape.part_size;
    const int p1 = (L + shape.part_size - 1) / shape.part_size;
    const int64_t base = (int64_t(seq) * p.num_heads + h) * shape.num_parts;
    float M = -INFINITY;
    for (int pp = p0; pp < p1; ++pp) M = fmaxf(M, p.ws_ml[(base + pp) * 2]);
    float num[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) num[k] = 0.f;
    float den = 0.f;
    for (int pp = p0; pp < p1; ++pp) {
        const float f = fast_exp2(p.ws_ml[(base + pp) * 2] - M);
        den += f * p.ws_ml[(base + pp) * 2 + 1];
        const float *a = p.ws_acc + (base + pp) * D;
#pragma unroll
        for (int k = 0; k < PER; ++k) num[k] += f * a[lane + 64 * k];
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) store_out<T>(out_row + lane + 64 * k, num[k] / den);
}

template <typename T, int D, int GP>
hipError_t launch_typed(const DecodeParams &p, const DecodeShape &s, hipStream_t stream) {
    const int64_t blocks = int64_t(p.num_seqs) * p.num_kv_heads * s.head_groups * s.num_parts;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_partition_kernel<T, D, GP>), dim3(unsigned(blocks)), dim3(kThreads), 0, stream, p, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || s.num_parts == 1) return e;
    hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(unsigned(p.num_seqs * p.num_heads)), dim3(64), 0, stream, p,
                       s);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_group(const DecodeParams &p, const DecodeShape &s, int padded_group, hipStream_t stream) {
    switch (padded_group) {
        case 1: return launch_typed<T, D, 1>(p, s, stream);
        case 2: return launch_typed<T, D, 2>(p, s, stream);
        case 4: return launch_typed<T, D, 4>(p, s, stream);
        case 8: return launch_typed<T, D, 8>(p, s, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

DecodePlan plan_decode(int32_t num_heads, int32_t num_kv_heads, int32_t head_size, int32_t num_seqs,
                       int32_t max_seq_len) {
    DecodePlan plan{};
    const int group = num_heads / num_kv_heads;
    plan.head_groups = (group + kMaxGroup - 1) / kMaxGroup;
    plan.heads_per_group = (group + plan.head_groups - 1) / plan.head_groups;
    plan.padded_group = 1;
    while (plan.padded_group < plan.heads_per_group) plan.padded_group <<= 1;
    const int64_t units = int64_t(num_seqs) * num_kv_heads * plan.head_groups;
    const int64_t len = max_seq_len > 0 ? max_seq_len : 1;
    // Partitions of 512 keys, or 1024 when that still gives >= 8192 workgroups (halves the
    // partial-result traffic on long contexts).
    int part = 512;
    if (units * ((len + 1023) / 1024) >= 8192) part = 1024;
    plan.part_size = part;
    plan.num_parts = int((len + part - 1) / part);
    plan.workspace_bytes = 0;
    if (plan.num_parts > 1) {
        const size_t slots = size_t(num_seqs) * num_heads * plan.num_parts;
        const size_t acc = slots * head_size * sizeof(float);
        const size_t acc_aligned = (acc + 255) / 256 * 256;
        plan.workspace_bytes = acc_aligned + slots * 2 * sizeof(float);
    }
    return plan;
}

hipError_t launch_decode(const DecodeParams &p, const DecodePlan &plan, int dtype, int head_size,
                         hipStream_t stream) {
    DecodeShape s{plan.part_size, plan.num_parts, plan.head_groups, plan.heads_per_group};
    if (dtype == 1) {
        if (head_size == 128) return launch_group<bf16_t, 128>(p, s, plan.padded_group, stream);
        if (head_size == 64) return launch_group<bf16_t, 64>(p, s, plan.padded_group, stream);
    } else {
        if (head_size == 128) return launch_group<float, 128>(p, s, plan.padded_group, stream);
        if (head_size == 64) return launch_group<float, 64>(p, s, plan.padded_group, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace pa
