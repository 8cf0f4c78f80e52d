// Variable-length causal prefill with a paged cached context (chunked prefill).
//
// What is computed (aphrodite-engine "xformers.py": XFormersMetadata note on context_len /
// subquery_len / seqlen, subquery_start_loc, XFormersImpl.forward with forward_prefix and
// _run_memory_efficient_xformers_forward; vLLM "cpu_attn": flash_attn_varlen_func call): the
// subquery token t of sequence i sits at position c_i + t and attends causally to keys
// 0 .. c_i + t, the first c_i of which are read from the paged cache through the block table and
// the rest from the key/value rows of the call; sliding window and ALiBi as in decode.
//
// bf16 kernel (MFMA).  A workgroup of 4 wavefronts owns 128 consecutive query rows of one
// (sequence, query head); each wavefront owns 32 rows (two 16-row MFMA blocks).  It walks the
// needed keys in 64-key tiles that are staged in LDS:
//   * K tile row-major [64][D] (16-byte chunks xor-swizzled by row, so the 16 rows an MFMA
//     operand read touches hit distinct banks);
//   * V tile transposed [D][64] (keys contiguous per d, in a key order matched to the P
//     operand below, 16-byte units xor-swizzled by d).
// Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_16x16x32_bf16: the accumulator
// layout then gives every lane 4 consecutive keys of ONE query row, so the row's max and sum
// need only two cross-lane steps, and two key blocks of those lanes are exactly the 8-key
// slice a lane must supply as the B operand of O^T = V^T P^T (the k index of A and B uses the
// same slot->key assignment, so the pairing is exact).  O^T accumulates in fp32 registers, with
// the lane's query row fixed, so rescaling by the running max is lane-local.
//
// fp32 kernel: a plain wavefront-per-(row, head) VALU loop (no MFMA for fp32 here).
#include <math.h>

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kBM = 128;       // query rows per workgroup
constexpr int kBN = 64;        // keys per tile
constexpr int kThreads = 256;

struct SeqInfo {
    int start;      // first query/key row of the sequence
    int n;          // subquery rows
    int c;          // cached context tokens
};

__device__ __forceinline__ SeqInfo seq_info(const PrefillParams &p, int seq) {
    SeqInfo s;
    int a = p.cu_subquery[seq];
    int b = p.cu_subquery[seq + 1];
    a = max(0, min(a, int(p.num_tokens)));
    b = max(a, min(b, int(p.num_tokens)));
    s.start = a;
    s.n = b - a;
    int c = p.context_lens ? p.context_lens[seq] : 0;
    c = max(0, min(c, p.block_tables ? (p.max_blocks << p.block_shift) : 0));
    s.c = c;
    return s;
}

// Element offset of key/value row j of a sequence, and which source it comes from.
struct RowSrc {
    const bf16_t *k;
    const bf16_t *v;
};

template <typename T>
__device__ __forceinline__ void row_ptrs(const PrefillParams &p, const SeqInfo &s, int seq, int g, int D, int j,
                                         const T *&kptr, const T *&vptr) {
    if (j < s.c) {
        int64_t blk = p.block_tables[int64_t(seq) * p.max_blocks + (j >> p.block_shift)];
        blk = blk < 0 ? 0 : (blk >= p.num_blocks ? p.num_blocks - 1 : blk);
        const int64_t off = ((blk << p.block_shift) + (j & ((1 << p.block_shift) - 1))) *
                                (int64_t(p.num_kv_heads) * D) + int64_t(g) * D;
        kptr = reinterpret_cast<const T *>(p.k_cache) + off;
        vptr = reinterpret_cast<const T *>(p.v_cache) + off;
    } else {
        const int64_t off = int64_t(s.start + (j - s.c)) * p.kv_stride + int64_t(g) * D;
        kptr = reinterpret_cast<const T *>(p.key) + off;
        vptr = reinterpret_cast<const T *>(p.value) + off;
    }
}

// Position of key kp' (0..63) of a tile in the transposed V tile, for key index k (0..63):
// k = 32 kc + 16 hh + 4 g + ii  ->  32 kc + 8 g + 4 hh + ii.
__device__ __forceinline__ int vt_key_pos(int k) {
    const int kc = k >> 5, hh = (k >> 4) & 1, g = (k >> 2) & 3, ii = k & 3;
    return 32 * kc + 8 * g + 4 * hh + ii;
}
// Element index inside Vt[D][64] of (d, permuted key position kp), with 16-byte units swizzled.
__device__ __forceinline__ int vt_index(int d, int kp) {
    const int f = (d ^ (d >> 3)) & 7;
    return d * kBN + (((kp >> 3) ^ f) << 3) + (kp & 7);
}

template <int D>
__global__ __launch_bounds__(kThreads) void prefill_bf16_kernel(PrefillParams p, int num_qtiles) {
    constexpr int CH = D / 8;       // 16-byte chunks per row
    constexpr int DC = D / 32;      // k-chunks of S^T
    constexpr int DB = D / 16;      // d-blocks of O^T
    __shared__ __align__(16) bf16_t Ks[kBN * D];
    __shared__ __align__(16) bf16_t Vt[D * kBN];

    int bid = blockIdx.x;
    const int h = bid % p.num_heads;
    bid /= p.num_heads;
    const int seq = bid % p.num_seqs;
    const int qt = num_qtiles - 1 - bid / p.num_seqs;      // heavy (late) tiles first
    const SeqInfo si = seq_info(p, seq);
    if (qt * kBM >= si.n) return;

    const int group = p.num_heads / p.num_kv_heads;
    const int g = h / group;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15;
    const int lg = lane >> 4;
    const int t0 = qt * kBM + wave * 32;

    // Q as the B operand of S^T = K Q^T: lane holds row (t0 + 16 qb + l16), d = 32 dc + 8 lg .. +7.
    bf16x8_v qf[2][DC];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int trow = min(t0 + 16 * qb + l16, si.n - 1);
        const bf16_t *qrow = reinterpret_cast<const bf16_t *>(p.query) + int64_t(si.start + trow) * p.q_stride +
                             int64_t(h) * D + 8 * lg;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) qf[qb][dc] = *reinterpret_cast<const bf16x8_v *>(qrow + 32 * dc);
    }

    const int row_hi = min(qt * kBM + kBM, si.n) - 1;
    const int pos_lo = si.c + qt * kBM;
    const int key_hi = si.c + row_hi;
    const int key_lo = p.window > 0 ? max(0, pos_lo - p.window + 1) : 0;
    const float qk_scale = p.scale * kLog2e;
    const float slope2 = p.alibi_slopes ? p.alibi_slopes[h] * kLog2e : 0.f;

    float m_run[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.f, 0.f};
    floatx4_v o[2][DB];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int db = 0; db < DB; ++db) o[qb][db] = floatx4_v{0.f, 0.f, 0.f, 0.f};

    for (int kt = key_lo / kBN; kt <= key_hi / kBN; ++kt) {
        __syncthreads();
        // ---- K tile -> LDS (row-major, chunk swizzle)
#pragma unroll
        for (int k = 0; k < (kBN * CH) / kThreads; ++k) {
            const int idx = tid + kThreads * k;
            const int row = idx / CH, ch = idx % CH;
            const int key = min(max(kt * kBN + row, key_lo), key_hi);
            const bf16_t *kp, *vp;
            row_ptrs<bf16_t>(p, si, seq, g, D, key, kp, vp);
            const uint4 v = *reinterpret_cast<const uint4 *>(kp + 8 * ch);
            *reinterpret_cast<uint4 *>(&Ks[row * D + ((ch ^ (row % CH)) << 3)]) = v;
        }
        // ---- V tile -> LDS transposed: thread = (key quad, 16-byte chunk)
        if (tid < 16 * CH) {
            const int quad = tid & 15, ch = tid >> 4;
            uint4 vv[4];
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int key = min(max(kt * kBN + 4 * quad + ii, key_lo), key_hi);
                const bf16_t *kp, *vp;
                row_ptrs<bf16_t>(p, si, seq, g, D, key, kp, vp);
                vv[ii] = *reinterpret_cast<const uint4 *>(vp + 8 * ch);
            }
            const int kp0 = vt_key_pos(4 * quad);
            const uint32_t w0[4] = {vv[0].x, vv[0].y, vv[0].z, vv[0].w};
            const uint32_t w1[4] = {vv[1].x, vv[1].y, vv[1].z, vv[1].w};
            const uint32_t w2[4] = {vv[2].x, vv[2].y, vv[2].z, vv[2].w};
            const uint32_t w3[4] = {vv[3].x, vv[3].y, vv[3].z, vv[3].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int w = e >> 1;
                uint2 pk;
                if (e & 1) {
                    pk.x = interleave_hi(w0[w], w1[w]);
                    pk.y = interleave_hi(w2[w], w3[w]);
                } else {
                    pk.x = interleave_lo(w0[w], w1[w]);
                    pk.y = interleave_lo(w2[w], w3[w]);
                }
                *reinterpret_cast<uint2 *>(&Vt[vt_index(8 * ch + e, kp0)]) = pk;
            }
        }
        __syncthreads();

        // ---- S^T = K Q^T: s[kb][qb] holds keys 16 kb + 4 lg + i of row 16 qb + l16
        floatx4_v s[4][2];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) s[kb][qb] = floatx4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int row = 16 * kb + l16;
                const bf16x8_v a =
                    *reinterpret_cast<const bf16x8_v *>(&Ks[row * D + (((4 * dc + lg) ^ (row % CH)) << 3)]);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
                    s[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[qb][dc], s[kb][qb], 0, 0, 0);
            }
        }

        // ---- mask, bias, online softmax; P^T operand
        bf16x8_v pb[2][2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int pos = si.c + t0 + 16 * qb + l16;
            float rmax = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = kt * kBN + 16 * kb + 4 * lg + i;
                    const bool vis = key <= pos && (p.window <= 0 || pos - key < p.window);
                    const float v = s[kb][qb][i] * qk_scale + slope2 * float(key - pos);
                    s[kb][qb][i] = vis ? v : -INFINITY;
                    rmax = fmaxf(rmax, s[kb][qb][i]);
                }
            rmax = fmaxf(rmax, lane_xor<16>(rmax));
            rmax = fmaxf(rmax, lane_xor<32>(rmax));
            const float m_new = fmaxf(m_run[qb], rmax);
            const float alpha = (m_run[qb] == -INFINITY) ? 0.f : fast_exp2(m_run[qb] - m_new);
            float psum = 0.f;
            bf16_t pv[4][4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x = s[kb][qb][i];
                    const float pf = (x == -INFINITY) ? 0.f : fast_exp2(x - m_new);
                    pv[kb][i] = f32_to_bf16(pf);
                    psum += bf16_to_f32(pv[kb][i]);
                }
            l_run[qb] = l_run[qb] * alpha + psum;
            m_run[qb] = m_new;
#pragma unroll
            for (int db = 0; db < DB; ++db) o[qb][db] *= alpha;
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                uint4 w;
                w.x = uint32_t(pv[2 * kc][0]) | (uint32_t(pv[2 * kc][1]) << 16);
                w.y = uint32_t(pv[2 * kc][2]) | (uint32_t(pv[2 * kc][3]) << 16);
                w.z = uint32_t(pv[2 * kc + 1][0]) | (uint32_t(pv[2 * kc + 1][1]) << 16);
                w.w = uint32_t(pv[2 * kc + 1][2]) | (uint32_t(pv[2 * kc + 1][3]) << 16);
                pb[qb][kc] = __builtin_bit_cast(bf16x8_v, w);
            }
        }

        // ---- O^T += V^T P^T
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int d = 16 * db + l16;
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                const bf16x8_v a = *reinterpret_cast<const bf16x8_v *>(&Vt[vt_index(d, 32 * kc + 8 * lg)]);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
                    o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[qb][kc], o[qb][db], 0, 0, 0);
            }
        }
    }

    // ---- epilogue: O = O^T / l, rounded to bf16; lane holds d = 16 db + 4 lg + i of its row
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        float l = l_run[qb];
        l += lane_xor<16>(l);
        l += lane_xor<32>(l);
        const int trow = t0 + 16 * qb + l16;
        if (trow < si.n) {
            const float inv = 1.f / l;
            bf16_t *orow = reinterpret_cast<bf16_t *>(p.out) + int64_t(si.start + trow) * p.num_heads * D +
                           int64_t(h) * D + 4 * lg;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                uint2 w;
                w.x = pack_bf16x2(o[qb][db][0] * inv, o[qb][db][1] * inv);
                w.y = pack_bf16x2(o[qb][db][2] * inv, o[qb][db][3] * inv);
                *reinterpret_cast<uint2 *>(orow + 16 * db) = w;
            }
        }
    }
}

// fp32: one wavefront per (query row, head).  Keys in 64-key tiles, lane = key for the scores,
// lane = output element for P.V.
template <int D>
__global__ __launch_bounds__(64) void prefill_f32_kernel(PrefillParams p) {
    constexpr int PER = D / 64;
    __shared__ float qs[D];
    const int lane = threadIdx.x;
    const int h = blockIdx.x % p.num_heads;
    const int64_t t = blockIdx.x / p.num_heads;
    // sequence of row t: last seq with cu[seq] <= t
    int lo_s = 0, hi_s = p.num_seqs - 1;
    while (lo_s < hi_s) {
        const int mid = (lo_s + hi_s + 1) >> 1;
        if (p.cu_subquery[mid] <= t) lo_s = mid; else hi_s = mid - 1;
    }
    const int seq = lo_s;
    const SeqInfo si = seq_info(p, seq);
    const int trow = int(t) - si.start;
    if (trow < 0 || trow >= si.n) return;
    const int g = h / (p.num_heads / p.num_kv_heads);
    const int pos = si.c + trow;
    const int klo = p.window > 0 ? max(0, pos - p.window + 1) : 0;
    const float *qrow = reinterpret_cast<const float *>(p.query) + t * p.q_stride + int64_t(h) * D;
    for (int d = lane; d < D; d += 64) qs[d] = qrow[d];
    __syncthreads();
    const float qk_scale = p.scale * kLog2e;
    const float slope2 = p.alibi_slopes ? p.alibi_slopes[h] * kLog2e : 0.f;
    float m = -INFINITY, l = 0.f, acc[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = 0.f;
    for (int kt = klo; kt <= pos; kt += 64) {
        const int key = kt + lane;
        const int keyc = min(key, pos);
        const float *kp, *vp;
        row_ptrs<float>(p, si, seq, g, D, keyc, kp, vp);
        float dot = 0.f;
        for (int d = 0; d < D; d += 4) {
            const float4 kv = *reinterpret_cast<const float4 *>(kp + d);
            dot = fmaf(kv.x, qs[d], dot);
            dot = fmaf(kv.y, qs[d + 1], dot);
            dot = fmaf(kv.z, qs[d + 2], dot);
            dot = fmaf(kv.w, qs[d + 3], dot);
        }
        const float sc = key <= pos ? dot * qk_scale + slope2 * float(key - pos) : -INFINITY;
        const float tmax = xor_max_from<1>(sc);
        const float m_new = fmaxf(m, tmax);
        const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - m_new);
        const float pw = (sc == -INFINITY) ? 0.f : fast_exp2(sc - m_new);
        l = l * alpha + xor_sum_from<1>(pw);
        m = m_new;
#pragma unroll
        for (int k = 0; k < PER; ++k) acc[k] *= alpha;
        const int nk = min(64, pos - kt + 1);
        for (int jj = 0; jj < nk; ++jj) {
            const float pj = __shfl(pw, jj, 64);
            const float *kq, *vq;
            row_ptrs<float>(p, si, seq, g, D, kt + jj, kq, vq);
#pragma unroll
            for (int k = 0; k < PER; ++k) acc[k] = fmaf(pj, vq[lane + 64 * k], acc[k]);
        }
    }
    float *orow = reinterpret_cast<float *>(p.out) + t * p.num_heads * D + int64_t(h) * D;
#pragma unroll
    for (int k = 0; k < PER; ++k) orow[lane + 64 * k] = acc[k] / l;
}

}  // namespace

hipError_t launch_prefill(const PrefillParams &p, int dtype, int head_size, hipStream_t stream) {
    if (dtype == 1) {
        const int num_qtiles = (p.max_subquery_len + kBM - 1) / kBM;
        const int64_t blocks = int64_t(num_qtiles) * p.num_seqs * p.num_heads;
        if (blocks == 0) return hipSuccess;
        if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
        if (head_size == 128)
            hipLaunchKernelGGL(prefill_bf16_kernel<128>, dim3(unsigned(blocks)), dim3(kThreads), 0, stream, p,
                               num_qtiles);
        else if (head_size == 64)
            hipLaunchKernelGGL(prefill_bf16_kernel<64>, dim3(unsigned(blocks)), dim3(kThreads), 0, stream, p,
                               num_qtiles);
        else
            return hipErrorInvalidValue;
        return hipGetLastError();
    }
    const int64_t blocks = p.num_tokens * p.num_heads;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (head_size == 128)
        hipLaunchKernelGGL(prefill_f32_kernel<128>, dim3(unsigned(blocks)), dim3(64), 0, stream, p);
    else if (head_size == 64)
        hipLaunchKernelGGL(prefill_f32_kernel<64>, dim3(unsigned(blocks)), dim3(64), 0, stream, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace pa
