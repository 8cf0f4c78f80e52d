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
// The running row max is raised only when a tile's max exceeds it by more than this (base-2
// units); until then weights are <= 2^8 and the O accumulators need no rescaling.
constexpr float kRescaleSlack = 8.0f;

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

// Grid of the bf16 kernel.  Workgroups that read the same K/V -- the G query heads of one KV head
// and `qtiles_per_group` neighbouring query tiles of one sequence -- form a group.  Workgroups
// are dealt to the 8 XCDs round-robin by index, so the index is built as
// ((group / 8) * group_size + member) * 8 + group % 8: the members of a group run back to back on
// one XCD and share its L2, and each XCD takes every 8th group in heavy-first order (late query
// tiles see the most keys).
struct PrefillGrid {
    int num_qtiles;        // ceil(max_subquery_len / kBM)
    int qtiles_per_group;  // query tiles in a group
    int num_qblocks;       // ceil(num_qtiles / qtiles_per_group)
    int group_size;        // G * qtiles_per_group workgroups
    int num_groups;        // num_qblocks * num_seqs * num_kv_heads
};

template <int D>
__global__ __launch_bounds__(kThreads, 2) void prefill_bf16_kernel(PrefillParams p, PrefillGrid grid) {
    constexpr int CH = D / 8;        // 16-byte chunks per row
    constexpr int DC = D / 32;       // k-chunks of S^T
    constexpr int DB = D / 16;       // d-blocks of O^T
    constexpr int KPT = CH / 4;      // K chunks per thread (one row per thread, 4 threads per row)
    constexpr int V_THREADS = 16 * CH;
    // two stages of K (row-major) and V (transposed)
    __shared__ __align__(16) bf16_t Ks[2][kBN * D];
    __shared__ __align__(16) bf16_t Vt[2][D * kBN];

    // ---- workgroup -> (sequence, KV head, query head, query tile)
    const int b = blockIdx.x;
    const int xcd = b & 7;
    const int qq = b >> 3;
    const int member = qq % grid.group_size;
    const int k = (qq / grid.group_size) * 8 + xcd;
    if (k >= grid.num_groups) return;
    const int group = p.num_heads / p.num_kv_heads;
    const int per_qb = p.num_seqs * p.num_kv_heads;
    const int qb = grid.num_qblocks - 1 - k / per_qb;
    const int seq = (k % per_qb) / p.num_kv_heads;
    const int g = k % p.num_kv_heads;
    const int h = g * group + member % group;
    const int qt = qb * grid.qtiles_per_group + member / group;
    const SeqInfo si = seq_info(p, seq);
    if (qt >= grid.num_qtiles || qt * kBM >= si.n) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15;
    const int lg = lane >> 4;
    const int t0 = qt * kBM + wave * 32;

    // Q as the B operand of S^T = K Q^T: lane holds row (t0 + 16 qb + l16), d = 32 dc + 8 lg .. +7.
    bf16x8_v qf[2][DC];
#pragma unroll
    for (int qbk = 0; qbk < 2; ++qbk) {
        const int trow = min(t0 + 16 * qbk + l16, si.n - 1);
        const bf16_t *qrow = reinterpret_cast<const bf16_t *>(p.query) + int64_t(si.start + trow) * p.q_stride +
                             int64_t(h) * D + 8 * lg;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) qf[qbk][dc] = *reinterpret_cast<const bf16x8_v *>(qrow + 32 * dc);
    }

    const int row_hi = min(qt * kBM + kBM, si.n) - 1;
    const int pos_lo = si.c + qt * kBM;
    const int key_hi = si.c + row_hi;
    const int key_lo = p.window > 0 ? max(0, pos_lo - p.window + 1) : 0;
    const int kt_lo = key_lo / kBN, kt_hi = key_hi / kBN;
    const float qk_scale = p.scale * kLog2e;
    const float slope2 = p.alibi_slopes ? p.alibi_slopes[h] * kLog2e : 0.f;
    const bool has_alibi = p.alibi_slopes != nullptr;

    // ---- tile loaders.  Each thread loads one K row (KPT chunks) and, if it is a V thread, four
    // consecutive keys of one 16-byte column; both lie in one cache block, whose id is fetched two
    // tiles ahead.
    const int k_row = tid >> 2;
    const int k_ch0 = (tid & 3) * KPT;
    const int v_quad = tid & 15, v_ch = tid >> 4;
    const int64_t kv_head_off = int64_t(g) * D;
    const int64_t cache_row_elems = int64_t(p.num_kv_heads) * D;
    auto block_id = [&](int key) -> int {
        if (key >= si.c) return 0;
        int64_t blk = p.block_tables[int64_t(seq) * p.max_blocks + (key >> p.block_shift)];
        return int(blk < 0 ? 0 : (blk >= p.num_blocks ? p.num_blocks - 1 : blk));
    };
    auto clampk = [&](int key) { return min(max(key, key_lo), key_hi); };
    auto row_ptr = [&](const void *cache, const void *rows, int key, int blk) -> const bf16_t * {
        if (key < si.c) {
            const int64_t off = ((int64_t(blk) << p.block_shift) + (key & ((1 << p.block_shift) - 1))) * cache_row_elems +
                                kv_head_off;
            return reinterpret_cast<const bf16_t *>(cache) + off;
        }
        return reinterpret_cast<const bf16_t *>(rows) + int64_t(si.start + (key - si.c)) * p.kv_stride + kv_head_off;
    };
    int kid_a = 0, vid_a = 0, kid_b = 0, vid_b = 0;   // block ids of tiles kt+1 (a) and kt+2 (b)
    auto fetch_ids = [&](int kt, int &kid, int &vid) {
        kid = block_id(clampk(kt * kBN + k_row));
        vid = block_id(clampk(kt * kBN + 4 * v_quad));
    };
    uint4 kreg[KPT], vreg[4];
    auto load_tile = [&](int kt, int kid, int vid) {
        const int kk = clampk(kt * kBN + k_row);
        const bf16_t *kp = row_ptr(p.k_cache, p.key, kk, kid);
#pragma unroll
        for (int c = 0; c < KPT; ++c) kreg[c] = *reinterpret_cast<const uint4 *>(kp + 8 * (k_ch0 + c));
        if (tid < V_THREADS) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                // the four keys of a quad share a block (block sizes are multiples of 8)
                const int kv = clampk(kt * kBN + 4 * v_quad + ii);
                const int vb = (kv >> p.block_shift) == ((kt * kBN + 4 * v_quad) >> p.block_shift) ? vid : block_id(kv);
                vreg[ii] = *reinterpret_cast<const uint4 *>(row_ptr(p.v_cache, p.value, kv, vb) + 8 * v_ch);
            }
        }
    };
    auto store_tile = [&](int stage) {
#pragma unroll
        for (int c = 0; c < KPT; ++c) {
            const int ch = k_ch0 + c;
            *reinterpret_cast<uint4 *>(&Ks[stage][k_row * D + ((ch ^ (k_row % CH)) << 3)]) = kreg[c];
        }
        if (tid < V_THREADS) {
            const int kp0 = vt_key_pos(4 * v_quad);
            const uint32_t w0[4] = {vreg[0].x, vreg[0].y, vreg[0].z, vreg[0].w};
            const uint32_t w1[4] = {vreg[1].x, vreg[1].y, vreg[1].z, vreg[1].w};
            const uint32_t w2[4] = {vreg[2].x, vreg[2].y, vreg[2].z, vreg[2].w};
            const uint32_t w3[4] = {vreg[3].x, vreg[3].y, vreg[3].z, vreg[3].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int wv = e >> 1;
                uint2 pk;
                if (e & 1) {
                    pk.x = interleave_hi(w0[wv], w1[wv]);
                    pk.y = interleave_hi(w2[wv], w3[wv]);
                } else {
                    pk.x = interleave_lo(w0[wv], w1[wv]);
                    pk.y = interleave_lo(w2[wv], w3[wv]);
                }
                *reinterpret_cast<uint2 *>(&Vt[stage][vt_index(8 * v_ch + e, kp0)]) = pk;
            }
        }
    };

    float m_run[2] = {-INFINITY, -INFINITY};   // row max (base 2), uniform over the row's 4 lanes
    float l_run[2] = {0.f, 0.f};               // this lane's part of the row sum
    floatx4_v o[2][DB];
#pragma unroll
    for (int qbk = 0; qbk < 2; ++qbk)
#pragma unroll
        for (int db = 0; db < DB; ++db) o[qbk][db] = floatx4_v{0.f, 0.f, 0.f, 0.f};

    // ---- prologue: tile kt_lo into stage 0; ids of the next two tiles in flight
    {
        int kid, vid;
        fetch_ids(kt_lo, kid, vid);
        load_tile(kt_lo, kid, vid);
        fetch_ids(kt_lo + 1, kid_a, vid_a);
        fetch_ids(kt_lo + 2, kid_b, vid_b);
        store_tile(0);
        __syncthreads();
    }

    int stage = 0;
    for (int kt = kt_lo; kt <= kt_hi; ++kt) {
        const bool more = kt < kt_hi;
        if (more) {
            load_tile(kt + 1, kid_a, vid_a);     // data of the next tile in flight during this one
            kid_a = kid_b;
            vid_a = vid_b;
            fetch_ids(kt + 3, kid_b, vid_b);
        }

        // ---- S^T = K Q^T: s[kb][qbk] holds keys 16 kb + 4 lg + i of row 16 qbk + l16
        floatx4_v s[4][2];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int qbk = 0; qbk < 2; ++qbk) s[kb][qbk] = floatx4_v{0.f, 0.f, 0.f, 0.f};
        const bf16_t *ks = Ks[stage];
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int row = 16 * kb + l16;
                const bf16x8_v a = *reinterpret_cast<const bf16x8_v *>(&ks[row * D + (((4 * dc + lg) ^ (row % CH)) << 3)]);
#pragma unroll
                for (int qbk = 0; qbk < 2; ++qbk)
                    s[kb][qbk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[qbk][dc], s[kb][qbk], 0, 0, 0);
            }
        }

        // ---- scale, bias, mask (edge tiles only), lazily raised row max
        const int kbase = kt * kBN + 4 * lg;
        const bool full = kt * kBN + kBN - 1 <= si.c + t0 && (p.window <= 0 || si.c + t0 + 31 - kt * kBN < p.window);
        float tmax[2];
#pragma unroll
        for (int qbk = 0; qbk < 2; ++qbk) {
            const int pos = si.c + t0 + 16 * qbk + l16;
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v = s[kb][qbk][i] * qk_scale;
                    if (has_alibi) v += slope2 * float(kbase + 16 * kb + i - pos);
                    if (!full) {
                        const int key = kbase + 16 * kb + i;
                        const bool vis = key <= pos && (p.window <= 0 || pos - key < p.window);
                        v = vis ? v : -INFINITY;
                    }
                    s[kb][qbk][i] = v;
                    mx = fmaxf(mx, v);
                }
            tmax[qbk] = mx;
        }
        const bool raise = tmax[0] > m_run[0] + kRescaleSlack || tmax[1] > m_run[1] + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {
#pragma unroll
            for (int qbk = 0; qbk < 2; ++qbk) {
                float r = fmaxf(tmax[qbk], lane_xor<16>(tmax[qbk]));
                r = fmaxf(r, lane_xor<32>(r));
                const float m_new = fmaxf(m_run[qbk], r);
                const float alpha = (m_run[qbk] == -INFINITY) ? 0.f : fast_exp2(m_run[qbk] - m_new);
                l_run[qbk] *= alpha;
                m_run[qbk] = m_new;
#pragma unroll
                for (int db = 0; db < DB; ++db) o[qbk][db] *= alpha;
            }
        }

        // ---- P (bf16) as the B operand of O^T = V^T P^T
        bf16x8_v pb[2][2];
#pragma unroll
        for (int qbk = 0; qbk < 2; ++qbk) {
            const float m = m_run[qbk];
            float psum = 0.f;
            uint32_t pk[4][2];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                float pf[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x = s[kb][qbk][i];
                    pf[i] = (x == -INFINITY) ? 0.f : fast_exp2(x - m);
                }
                pk[kb][0] = pack_bf16x2(pf[0], pf[1]);
                pk[kb][1] = pack_bf16x2(pf[2], pf[3]);
                psum += bf16_lo(pk[kb][0]) + bf16_hi(pk[kb][0]) + bf16_lo(pk[kb][1]) + bf16_hi(pk[kb][1]);
            }
            l_run[qbk] += psum;
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                const uint4 w = make_uint4(pk[2 * kc][0], pk[2 * kc][1], pk[2 * kc + 1][0], pk[2 * kc + 1][1]);
                pb[qbk][kc] = __builtin_bit_cast(bf16x8_v, w);
            }
        }

        // ---- O^T += V^T P^T
        const bf16_t *vt = Vt[stage];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int d = 16 * db + l16;
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                const bf16x8_v a = *reinterpret_cast<const bf16x8_v *>(&vt[vt_index(d, 32 * kc + 8 * lg)]);
#pragma unroll
                for (int qbk = 0; qbk < 2; ++qbk)
                    o[qbk][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[qbk][kc], o[qbk][db], 0, 0, 0);
            }
        }

        if (more) store_tile(stage ^ 1);
        __syncthreads();
        stage ^= 1;
    }

    // ---- epilogue: O = O^T / l, rounded to bf16; lane holds d = 16 db + 4 lg + i of its row
#pragma unroll
    for (int qbk = 0; qbk < 2; ++qbk) {
        float l = l_run[qbk];
        l += lane_xor<16>(l);
        l += lane_xor<32>(l);
        const int trow = t0 + 16 * qbk + l16;
        if (trow < si.n) {
            const float inv = 1.f / l;
            bf16_t *orow = reinterpret_cast<bf16_t *>(p.out) + int64_t(si.start + trow) * p.num_heads * D +
                           int64_t(h) * D + 4 * lg;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                uint2 w;
                w.x = pack_bf16x2(o[qbk][db][0] * inv, o[qbk][db][1] * inv);
                w.y = pack_bf16x2(o[qbk][db][2] * inv, o[qbk][db][3] * inv);
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
        PrefillGrid grid;
        grid.num_qtiles = (p.max_subquery_len + kBM - 1) / kBM;
        const int group = p.num_heads / p.num_kv_heads;
        grid.qtiles_per_group = group >= 8 ? 1 : min(8 / group, grid.num_qtiles);
        if (grid.qtiles_per_group < 1) grid.qtiles_per_group = 1;
        grid.num_qblocks = (grid.num_qtiles + grid.qtiles_per_group - 1) / grid.qtiles_per_group;
        grid.group_size = group * grid.qtiles_per_group;
        const int64_t groups = int64_t(grid.num_qblocks) * p.num_seqs * p.num_kv_heads;
        if (groups == 0) return hipSuccess;
        const int64_t blocks = (groups + 7) / 8 * 8 * grid.group_size;
        if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
        grid.num_groups = int(groups);
        if (head_size == 128)
            hipLaunchKernelGGL(prefill_bf16_kernel<128>, dim3(unsigned(blocks)), dim3(kThreads), 0, stream, p, grid);
        else if (head_size == 64)
            hipLaunchKernelGGL(prefill_bf16_kernel<64>, dim3(unsigned(blocks)), dim3(kThreads), 0, stream, p, grid);
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
