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

constexpr int kTile = 32;          // keys per wavefront tile
constexpr int kMaxGroup = 8;       // query heads per work unit
#ifndef PA_DECODE_MIN_UNITS
#define PA_DECODE_MIN_UNITS 8192
#endif
constexpr int64_t kMinUnits = PA_DECODE_MIN_UNITS;   // work units the partition size aims for

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

// Load instructions per wavefront tile.  Two tiles of K and V (4 * NI * 4 registers) are live at
// once, so wide head groups (more accumulators) and fp32 rows (more registers per key) use
// narrower tiles.
#ifndef PA_DECODE_NI_SMALL
#define PA_DECODE_NI_SMALL 8
#endif
#ifndef PA_DECODE_WAVES_SMALL
#define PA_DECODE_WAVES_SMALL 2
#endif
template <typename T, int GP>
constexpr int tile_loads() { return (GP >= 8 || sizeof(T) == 4) ? 4 : (GP <= 2 ? PA_DECODE_NI_SMALL : 8); }

// The running max is only raised when a tile's max exceeds it by more than this (base-2 units):
// until then weights are exp2(s - m) <= 2^8, exact enough in fp32 sums and bf16 weights, and the
// accumulators need no rescaling.
constexpr float kRescaleSlack = 8.0f;

// Per-wavefront state of the online softmax over the tiles of one work unit.
template <int GP, int EPL>
struct WaveAcc {
    float m_run;              // base-2 running max of the lane's score head
    float l_run;              // running sum of rounded weights, this row group
    float acc[GP][EPL];       // weighted V, this lane's elements, all heads, this row group
};

// Work unit u -> (sequence, KV head, head group, partition).  The partition index varies
// slowest: workgroups are dispatched in index order, so full partitions start first and the
// units past a sequence's end (which exit at once) come last.
struct Unit {
    int seq, g, hgrp, part;
};
__device__ __forceinline__ Unit unit_of(int u, const DecodeParams &p, const DecodeShape &s) {
    Unit w;
    const int per_part = p.num_seqs * p.num_kv_heads * s.head_groups;
    w.part = u / per_part;
    int rest = u - w.part * per_part;
    w.hgrp = rest % s.head_groups;
    rest /= s.head_groups;
    w.g = rest % p.num_kv_heads;
    w.seq = rest / p.num_kv_heads;
    return w;
}

__device__ __forceinline__ int clamp_len(int L, const DecodeParams &p, const DecodeShape &s) {
    return max(0, min(L, min(p.max_blocks << p.block_shift, s.num_parts * s.part_size)));
}

// Block ids of partition `part` of sequence `seq` (at most 128 blocks: lanes 0..63 and 64..127),
// clamped into the pool.  Read without knowing the sequence length: entries past the
// sequence's last block are read (within the table row) but never used.
__device__ __forceinline__ void load_ids(const DecodeParams &p, const DecodeShape &s, int seq, int part, int lane,
                                         int &ids0, int &ids1) {
    const int32_t *table = p.block_tables + int64_t(seq) * p.max_blocks;
    const int first = (part * s.part_size) >> p.block_shift;
    const int last = p.max_blocks - 1;
    const int64_t nbm1 = p.num_blocks - 1;
    int64_t b0 = table[min(first + lane, last)];
    ids0 = int(b0 < 0 ? 0 : (b0 > nbm1 ? nbm1 : b0));
    ids1 = ids0;
    if ((s.part_size >> p.block_shift) > 64) {
        int64_t b1 = table[min(first + 64 + lane, last)];
        ids1 = int(b1 < 0 ? 0 : (b1 > nbm1 ? nbm1 : b1));
    }
}

// Occupancy hint: the accumulators of a head group grow with its size.
template <int GP>
constexpr int waves_per_simd() { return GP <= 2 ? PA_DECODE_WAVES_SMALL : 2; }

// One work unit = one wavefront: partition `part` of (sequence, KV head, head group).
//   ONE_BLOCK: every tile lies inside one cache block (tile keys <= block size), so a tile needs
//              one block id; otherwise each load instruction looks up its own block.
template <typename T, int D, int GP, int NI, bool ONE_BLOCK>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(waves_per_simd<GP>(), 8)))
void decode_partition_kernel(DecodeParams p, DecodeShape shape) {
    constexpr int C = Geo<T, D>::kC, R = Geo<T, D>::kR, EPL = Geo<T, D>::kEpl;
    constexpr int TILE = NI * R;                       // keys per tile
    constexpr int WMASK = writer_mask<C, GP>();
    static_assert(NI % 2 == 0, "rows are paired for v_dot2");

    // Softmax weights of the current tile, [head][row group][instruction].
    __shared__ __align__(16) T p_lds[GP][R][NI];

    const int lane = threadIdx.x;
    const int c = lane % C;
    const int r = lane / C;
    const int my_head = head_of_lane<C, GP>(c);
    const int group = p.num_heads / p.num_kv_heads;
    const int nh = shape.heads_per_group;
    const int bmask = (1 << p.block_shift) - 1;
    const uint32_t row_bytes = uint32_t(p.num_kv_heads) * D * sizeof(T);           // one token, all heads
    const int64_t block_bytes = int64_t(row_bytes) << p.block_shift;
    const char *kcache = reinterpret_cast<const char *>(p.k_cache);
    const char *vcache = reinterpret_cast<const char *>(p.v_cache);
    const float qk_scale = p.scale * kLog2e;

    // Length, block ids and query are requested together; none waits for another.
    const Unit w = unit_of(blockIdx.x, p, shape);
    int ids0, ids1;
    load_ids(p, shape, w.seq, w.part, lane, ids0, ids1);
    const int L = clamp_len(p.seq_lens[w.seq], p, shape);
    const int head0 = w.g * group + w.hgrp * nh;
    // Query chunks, head-permuted: slot s holds head s ^ my_head.
    uint32_t q[GP][4];
    {
        const T *qrow =
            reinterpret_cast<const T *>(p.query) + int64_t(w.seq) * p.q_stride + int64_t(head0) * D + c * EPL;
#pragma unroll
        for (int s = 0; s < GP; ++s) {
            const int hs = s ^ my_head;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (hs < nh) v = *reinterpret_cast<const uint4 *>(qrow + int64_t(hs) * D);
            q[s][0] = v.x; q[s][1] = v.y; q[s][2] = v.z; q[s][3] = v.w;
        }
    }
    const int lo = p.window > 0 ? max(0, L - p.window) : 0;
    const int pstart = w.part * shape.part_size;
    const int pend = min(pstart + shape.part_size, L);
    const int kb = max(pstart, lo);
    const int p_first = lo / shape.part_size;
    const int p_count = L > 0 ? (L + shape.part_size - 1) / shape.part_size - p_first : 0;
    T *out_row = reinterpret_cast<T *>(p.out) + (int64_t(w.seq) * p.num_heads + head0) * D;
    if (kb >= pend) {
        if (L == 0 && w.part == 0)
            for (int idx = lane; idx < nh * D; idx += 64) store_out<T>(out_row + idx, 0.f);
        return;
    }

    const bool has_alibi = p.alibi_slopes != nullptr;
    const float slope2 = (has_alibi && my_head < nh) ? p.alibi_slopes[head0 + my_head] * kLog2e : 0.f;
    const int pos = L - 1;
    const int pblock0 = pstart >> p.block_shift;
    // Lane part of every K/V address: row group r's token inside the instruction, KV head g, chunk c.
    const uint32_t lane_off = uint32_t(r) * row_bytes + (uint32_t(w.g) * D + c * EPL) * sizeof(T);

    // Scalar (uniform) part of the address of instruction i of the tile starting at tb: block base
    // plus the instruction's first token inside the block.  Tokens past the sequence's end read
    // unwritten slots of in-pool blocks; their scores are masked and their V rows zeroed.
    auto inst_base = [&](int tb, int i, int blk_tile) -> int64_t {
        const int row0 = tb + i * R;
        int blk = blk_tile;
        if constexpr (!ONE_BLOCK) {
            const int bidx = (row0 >> p.block_shift) - pblock0;
            blk = __builtin_amdgcn_readlane(bidx < 64 ? ids0 : ids1, bidx & 63);
        }
        return int64_t(blk) * block_bytes + int64_t(row0 & bmask) * row_bytes;
    };
    auto tile_block = [&](int tb) -> int {
        if constexpr (ONE_BLOCK) {
            const int bidx = (tb >> p.block_shift) - pblock0;
            return __builtin_amdgcn_readlane(bidx < 64 ? ids0 : ids1, bidx & 63);
        } else {
            return 0;
        }
    };
    auto load_rows = [&](const char *cache, int tb, uint4 (&x)[NI]) {
        const int blk = tile_block(tb);
#pragma unroll
        for (int i = 0; i < NI; ++i)
            x[i] = *reinterpret_cast<const uint4 *>(cache + inst_base(tb, i, blk) + lane_off);
    };

    // Online softmax state.  Each row group keeps its own running max (base 2) per head, so no
    // tile needs a cross-row-group reduction; the groups are brought to a common max at the end.
    float m_run = -INFINITY;      // head my_head, this row group
    float l_run = 0.f;            // sum of rounded weights, head my_head, this row group
    float acc[GP][EPL];           // weighted V, all heads, this lane's elements, this row group
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;

    auto scores = [&](int tb, const uint4 (&kr)[NI], float (&sc)[NI]) {
        const bool edge = tb < lo || tb + TILE - 1 > pos;           // uniform
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            float part_dot[GP];
            chunk_dots<T, GP>(kr[i], q, part_dot);
            butterfly<C, GP, 0>(part_dot);
            sc[i] = part_dot[0] * qk_scale;
        }
        if (has_alibi) {
#pragma unroll
            for (int i = 0; i < NI; ++i) sc[i] += slope2 * float(tb + i * R + r - pos);
        }
        if (edge) {
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int j = tb + i * R + r;
                sc[i] = (j >= lo && j <= pos) ? sc[i] : -INFINITY;
            }
        }
    };
    auto softmax_pv = [&](int tb, const float (&sc)[NI], uint4 (&vr)[NI]) {
        // Lazily raised max: rescale only when some tile max exceeds the running max by more than
        // kRescaleSlack (always on the first tile, rarely afterwards); uniform over the wavefront.
        float tmax = sc[0];
#pragma unroll
        for (int i = 1; i < NI; ++i) tmax = fmaxf(tmax, sc[i]);
        const bool raise = tmax > m_run + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {
            const float m_new = fmaxf(m_run, tmax);
            const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
            l_run *= alpha;
            m_run = m_new;
#pragma unroll
            for (int h = 0; h < GP; ++h) {
                const float a = __shfl(alpha, r * C + lane_of_head<C, GP>(h), 64);
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[h][e] *= a;
            }
        }
        float psum = 0.f;
        T pv[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const float pf = (sc[i] == -INFINITY) ? 0.f : fast_exp2(sc[i] - m_run);
            if constexpr (sizeof(T) == 2) {
                pv[i] = f32_to_bf16(pf);
                psum += bf16_to_f32(pv[i]);
            } else {
                pv[i] = pf;
                psum += pf;
            }
        }
        l_run += psum;
        if ((c & WMASK) == 0) {
#pragma unroll
            for (int i = 0; i < NI; ++i) p_lds[my_head][r][i] = pv[i];
        }
        // Rows past the sequence's end hold unwritten cache bytes: zero them so that their zero
        // weights cannot meet a NaN.
        if (tb + TILE - 1 > pos) {
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const bool past = tb + i * R + r > pos;
                vr[i].x = past ? 0u : vr[i].x;
                vr[i].y = past ? 0u : vr[i].y;
                vr[i].z = past ? 0u : vr[i].z;
                vr[i].w = past ? 0u : vr[i].w;
            }
        }
        wave_lds_sync();

        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int ip = 0; ip < NI / 2; ++ip) {
                // row pair (2ip, 2ip+1) -> per element e the bf16 pair (v_2ip[e], v_2ip+1[e])
                const uint4 a = vr[2 * ip], b = vr[2 * ip + 1];
                const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
                const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
                uint32_t vp[EPL];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    vp[2 * k] = interleave_lo(aw[k], bw[k]);
                    vp[2 * k + 1] = interleave_hi(aw[k], bw[k]);
                }
#pragma unroll
                for (int h = 0; h < GP; ++h) {
                    const uint32_t pp = reinterpret_cast<const uint32_t *>(&p_lds[h][r][0])[ip];
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[h][e] = dot2_bf16(pp, vp[e], acc[h][e]);
                }
            }
        } else {
#pragma unroll
            for (int h = 0; h < GP; ++h) {
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    const float pw = p_lds[h][r][i];
                    const uint32_t vw[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pw, __uint_as_float(vw[e]), acc[h][e]);
                }
            }
        }
        wave_lds_sync();
    };

    // Tiles of the partition in order, two register sets in turn: the next tile's K rows are
    // requested once this tile's scores have consumed K, its V rows once P.V has consumed V.  At
    // the last tile the loads re-read it (cache hits), keeping them unconditional.
    {
        int tb = (kb / TILE) * TILE;
        uint4 ka[NI], va[NI], kb2[NI], vb2[NI];
        load_rows(kcache, tb, ka);
        load_rows(vcache, tb, va);
        while (true) {
            int tn = tb + TILE;
            bool more = tn < pend;
            float sc[NI];
            scores(tb, ka, sc);
            load_rows(kcache, more ? tn : tb, kb2);
            softmax_pv(tb, sc, va);
            load_rows(vcache, more ? tn : tb, vb2);
            if (!more) break;
            tb = tn;
            tn = tb + TILE;
            more = tn < pend;
            scores(tb, kb2, sc);
            load_rows(kcache, more ? tn : tb, ka);
            softmax_pv(tb, sc, vb2);
            load_rows(vcache, more ? tn : tb, va);
            if (!more) break;
            tb = tn;
        }
    }

    // Bring the row groups to a common max per head, then sum them; lanes of row group 0 end
    // with the unit's weighted V for all heads.
    const float m_all = max_row_groups<C>(m_run);
    const float f_own = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_all);
#pragma unroll
    for (int h = 0; h < GP; ++h) {
        const float f = __shfl(f_own, r * C + lane_of_head<C, GP>(h), 64);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = sum_row_groups<C>(acc[h][e] * f);
    }
    const float l_sum = sum_row_groups<C>(l_run * f_own);
    if (p_count == 1) {
        // The whole (windowed) sequence is this partition: write the normalized output.
#pragma unroll
        for (int h = 0; h < GP; ++h) {
            const float lh = __shfl(l_sum, lane_of_head<C, GP>(h), 64);
            if (r == 0 && h < nh) {
                const float inv = 1.f / lh;
#pragma unroll
                for (int e = 0; e < EPL; ++e) store_out<T>(out_row + h * D + c * EPL + e, acc[h][e] * inv);
            }
        }
    } else {
        const int64_t slot0 = (int64_t(w.seq) * p.num_heads + head0) * shape.num_parts + w.part;
#pragma unroll
        for (int h = 0; h < GP; ++h) {
            const float lh = __shfl(l_sum, lane_of_head<C, GP>(h), 64);
            const float mh = __shfl(m_all, lane_of_head<C, GP>(h), 64);
            if (r == 0 && h < nh) {
                const int64_t slot = slot0 + int64_t(h) * shape.num_parts;
                float4 *dst = reinterpret_cast<float4 *>(p.ws_acc + slot * D + c * EPL);
#pragma unroll
                for (int e = 0; e < EPL; e += 4)
                    dst[e / 4] = make_float4(acc[h][e], acc[h][e + 1], acc[h][e + 2], acc[h][e + 3]);
                if (c == 0) {
                    p.ws_ml[slot * 2] = mh;
                    p.ws_ml[slot * 2 + 1] = lh;
                }
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
    if (L == 0) return;                       // padded row: written by its first unit
    const int lo = p.window > 0 ? max(0, L - p.window) : 0;
    const int p0 = lo / shape.part_size;
    const int p1 = (L + shape.part_size - 1) / shape.part_size;
    if (p1 - p0 <= 1) return;                 // one partition: its unit wrote the output
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

template <typename T, int D, int GP, int NI, bool ONE>
hipError_t launch_units(const DecodeParams &p, const DecodeShape &s, int64_t units, hipStream_t stream) {
    hipLaunchKernelGGL((decode_partition_kernel<T, D, GP, NI, ONE>), dim3(unsigned(units)), dim3(64), 0, stream, p, s);
    return hipGetLastError();
}

template <typename T, int D, int GP>
hipError_t launch_typed(const DecodeParams &p, const DecodeShape &s, hipStream_t stream) {
    const int64_t units = int64_t(p.num_seqs) * p.num_kv_heads * s.head_groups * s.num_parts;
    if (units > 0x7fffffff) return hipErrorInvalidConfiguration;
    constexpr int NI = tile_loads<T, GP>();
    constexpr int TILE = NI * Geo<T, D>::kR;
    const bool one_block = (1 << p.block_shift) >= TILE;
    hipError_t e = one_block ? launch_units<T, D, GP, NI, true>(p, s, units, stream)
                             : launch_units<T, D, GP, NI, false>(p, s, units, stream);
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

DecodePlan plan_decode(int32_t num_heads, int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                       int32_t num_seqs, int32_t max_seq_len) {
    int block_shift = 0;
    while ((1 << block_shift) < block_size) ++block_shift;
    DecodePlan plan{};
    const int group = num_heads / num_kv_heads;
    plan.head_groups = (group + kMaxGroup - 1) / kMaxGroup;
    plan.heads_per_group = (group + plan.head_groups - 1) / plan.head_groups;
    plan.padded_group = 1;
    while (plan.padded_group < plan.heads_per_group) plan.padded_group <<= 1;
    const int64_t units = int64_t(num_seqs) * num_kv_heads * plan.head_groups;
    const int64_t len = max_seq_len > 0 ? max_seq_len : 1;
    // Partition size: the largest of 4096 / 2048 / 1024 / 512 / 256 keys that still gives >= 8192
    // work units (one single-wavefront workgroup each; 256 CUs hold ~2048-4096 at once) for the
    // longest sequence: long partitions amortize the per-unit start and the partial-result
    // traffic, enough units keep every CU fed to the end.  At most 128 blocks per partition
    // (two id registers per lane).
    int part = 256;
    for (int cand : {4096, 2048, 1024, 512}) {
        if ((cand >> block_shift) <= 128 && units * ((len + cand - 1) / cand) >= kMinUnits) {
            part = cand;
            break;
        }
    }
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
