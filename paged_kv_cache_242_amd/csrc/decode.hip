// Single-token decode over the paged KV cache: split-KV partition kernel + merge kernel.
//
// What is computed (aphrodite-engine "xformers.py", XFormersImpl.forward / forward_decode and the
// XFormersMetadata note on context_len; vLLM "cpu_attn", TorchSDPAMetadata.decode_seq_lens and
// decode_block_tables): query row i, at position L_i - 1, attends to keys 0 .. L_i - 1 of its
// sequence (restricted to the last W with a sliding window), which are read through block-table
// row i; scores scale * <q, k_j> (+ slope_h * (j - pos) with ALiBi); softmax; weighted sum of V.
// Optional soft-cap (c tanh(x / c) of the scaled dot product, before the bias) and per-head sink
// logits (added to the softmax denominator only) follow the readings stated in pa.h.
//
// Work decomposition.  A work unit is one (sequence, KV head, group of up to 8 query heads); the
// query heads of a group share every K/V byte, so each byte read from HBM feeds all of them.  The
// key tiles of all units are laid end to end and split evenly over as many single-wavefront
// workgroups as the device holds at once (decode_plan_kernel computes the per-sequence tile
// prefix and each wavefront's first sequence on the device, from seq_lens), so every wavefront
// streams the same number of bytes and no tail of long units is left at the end.  A wavefront
// walks its tiles in order, keeping a running (max, sum, weighted V); a unit cut between
// wavefronts leaves partials that decode_merge_kernel combines with the log-sum-exp rule.
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
// GP heads over the rows it loaded (pairs of rows feed v_dot2), reading the softmax
// weights that the score lanes left in LDS; row groups are summed once at the end.
//
// Numerics: fp32 dot products (bf16 or fp16 pairs through v_dot2_f32_bf16 / v_dot2_f32_f16),
// softmax in the base-2 domain with fp32 exp2, weights rounded to the element type before they
// multiply V, fp32 accumulation, output rounded to nearest even.
#include <math.h>

#include <atomic>
#include <type_traits>

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kTile = 32;          // keys per wavefront tile
constexpr int kMaxGroup = 8;       // query heads per work unit
// Up to this many sequences the split kernel's wavefronts plan their own share (a scan of the
// sequences' tile counts each); beyond it a planning kernel does it once.
#ifndef PA_DECODE_INWAVE_MAX
#define PA_DECODE_INWAVE_MAX 2048
#endif
constexpr int kInWavePlanMax = PA_DECODE_INWAVE_MAX;

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
    int chunk;              // keys per block-id chunk (<= 128 blocks, multiple of the tile)
    int head_groups;        // query heads of one KV head are processed in this many groups
    int heads_per_group;    // real heads per group
    int units_per_seq;      // num_kv_heads * head_groups
    int num_waves;          // wavefronts of the split kernel
    int tile;               // keys per tile of the split kernel instance
    int max_len;            // bound on every sequence length
    int kvh;                // KV heads per work unit
    int inwave;             // 1: every split wavefront finds its own first tile (no planning kernel)
};

template <typename T>
__device__ __forceinline__ void store_out(T *dst, float v);
template <>
__device__ __forceinline__ void store_out<float>(float *dst, float v) { *dst = v; }
template <>
__device__ __forceinline__ void store_out<bf16_t>(bf16_t *dst, float v) { *dst = f32_to_bf16(v); }
template <>
__device__ __forceinline__ void store_out<f16_t>(f16_t *dst, float v) { *dst = f32_to_f16(v); }
template <>
__device__ __forceinline__ void store_out<bf16_c8_t>(bf16_c8_t *dst, float v) { *dst = to_elt<bf16_c8_t>(v); }
template <>
__device__ __forceinline__ void store_out<f16_c8_t>(f16_c8_t *dst, float v) { *dst = to_elt<f16_c8_t>(v); }

// Partial dot products of one 16-byte row chunk with GP query chunks.
template <typename T, int GP>
__device__ __forceinline__ void chunk_dots(const uint4 &k, const uint32_t (&q)[GP][4], float (&part)[GP]) {
    const uint32_t kw[4] = {k.x, k.y, k.z, k.w};
#pragma unroll
    for (int s = 0; s < GP; ++s) {
        float acc = 0.f;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int w = 0; w < 4; ++w) acc = dot2<T>(kw[w], q[s][w], acc);
        } else {
#pragma unroll
            for (int w = 0; w < 4; ++w) acc = fmaf(__uint_as_float(kw[w]), __uint_as_float(q[s][w]), acc);
        }
        part[s] = acc;
    }
}

// Tile shape per instance: NI load instructions per tile (R rows each), DEPTH register sets in
// flight, OCC wavefronts per SIMD.  DEPTH sets of K and V take 2 * DEPTH * NI * 4 registers;
// wide head groups (more accumulators) and fp32 rows (more registers per key) use fewer.
// Bytes in flight per CU = waves per CU * (DEPTH - 1) * 2 * NI KB (for 16-byte lanes).
#ifndef PA_DECODE_NI_S
#define PA_DECODE_NI_S 8        // 16-bit elements, head groups of 1 or 2
#endif
#ifndef PA_DECODE_DEPTH_S
#define PA_DECODE_DEPTH_S 2
#endif
#ifndef PA_DECODE_OCC_S
#define PA_DECODE_OCC_S 2
#endif
#ifndef PA_DECODE_NI_M
#define PA_DECODE_NI_M 8        // 16-bit elements, head groups of 4
#endif
#ifndef PA_DECODE_DEPTH_M
#define PA_DECODE_DEPTH_M 2
#endif
#ifndef PA_DECODE_OCC_M
#define PA_DECODE_OCC_M 1       // one wavefront per SIMD: ~2% faster than two for groups of 4
#endif
#ifndef PA_DECODE_NI_B
#define PA_DECODE_NI_B 4        // 16-bit elements, head groups of 8
#endif
#ifndef PA_DECODE_DEPTH_B
#define PA_DECODE_DEPTH_B 2
#endif
#ifndef PA_DECODE_OCC_B
#define PA_DECODE_OCC_B 1
#endif
// FP8 caches: each load instruction carries half the bytes (8 codes per lane), so the tile
// shapes are set separately to keep enough bytes in flight.
#ifndef PA_DECODE_NI_S8
#define PA_DECODE_NI_S8 8
#endif
#ifndef PA_DECODE_NI_M8
#define PA_DECODE_NI_M8 8
#endif
#ifndef PA_DECODE_NI_B8
#define PA_DECODE_NI_B8 4
#endif
#ifndef PA_DECODE_DEPTH_S8
#define PA_DECODE_DEPTH_S8 3
#endif
#ifndef PA_DECODE_DEPTH_M8
#define PA_DECODE_DEPTH_M8 3
#endif
#ifndef PA_DECODE_DEPTH_B8
#define PA_DECODE_DEPTH_B8 3
#endif
template <typename T, int GP>
constexpr int tile_loads() {
    if constexpr (kFp8Cache<T>) return GP <= 2 ? PA_DECODE_NI_S8 : (GP == 4 ? PA_DECODE_NI_M8 : PA_DECODE_NI_B8);
    return sizeof(T) == 4 ? 4 : (GP <= 2 ? PA_DECODE_NI_S : (GP == 4 ? PA_DECODE_NI_M : PA_DECODE_NI_B));
}
template <typename T, int GP>
constexpr int tile_depth() {
    if constexpr (kFp8Cache<T>)
        return GP <= 2 ? PA_DECODE_DEPTH_S8 : (GP == 4 ? PA_DECODE_DEPTH_M8 : PA_DECODE_DEPTH_B8);
    return sizeof(T) == 4 ? 2 : (GP <= 2 ? PA_DECODE_DEPTH_S : (GP == 4 ? PA_DECODE_DEPTH_M : PA_DECODE_DEPTH_B));
}
#ifndef PA_DECODE_OCC_M8
#define PA_DECODE_OCC_M8 2
#endif
#ifndef PA_DECODE_OCC_B8
#define PA_DECODE_OCC_B8 2
#endif
template <typename T, int GP>
constexpr int tile_occ() {
    if constexpr (kFp8Cache<T>) return GP <= 2 ? PA_DECODE_OCC_S : (GP == 4 ? PA_DECODE_OCC_M8 : PA_DECODE_OCC_B8);
    return sizeof(T) == 4 ? 2 : (GP <= 2 ? PA_DECODE_OCC_S : (GP == 4 ? PA_DECODE_OCC_M : PA_DECODE_OCC_B));
}

// The running max is only raised when a tile's max exceeds it by more than this (base-2 units):
// until then weights are exp2(s - m) <= 2^8, exact enough in fp32 sums and 16-bit weights, and the
// accumulators need no rescaling.
constexpr float kRescaleSlack = 8.0f;

// Per-wavefront state of the online softmax over the tiles of one work unit.
template <int GP, int EPL>
struct WaveAcc {
    float m_run;              // base-2 running max of the lane's score head
    float l_run;              // running sum of rounded weights, this row group
    float acc[GP][EPL];       // weighted V, this lane's elements, all heads, this row group
};

__device__ __forceinline__ int clamp_len(int L, const DecodeParams &p, const DecodeShape &s) {
    return max(0, min(L, min(p.max_blocks << p.block_shift, s.max_len)));
}

// Tiles (of s.tile keys, absolute alignment) that one work unit of sequence seq covers: keys
// lo .. L - 1, with a sliding window lo = L - qlen + 1 - W (the first query row's window start).
__device__ __forceinline__ int seq_tiles(const DecodeParams &p, const DecodeShape &s, int seq, int &L, int &lo) {
    L = clamp_len(p.seq_lens[seq], p, s);
    lo = p.window > 0 ? max(0, L - p.qlen + 1 - p.window) : 0;
    return L > 0 ? (L + s.tile - 1) / s.tile - lo / s.tile : 0;
}

// Wavefront that owns tile t of the concatenated tile space (T tiles over N wavefronts,
// wavefront i owning tiles floor(i T / N) .. floor((i + 1) T / N) - 1).
__device__ __forceinline__ int wave_of_tile(int64_t t, int64_t T, int N) {
    const int64_t i = ((t + 1) * N + T - 1) / T - 1;
    return int(i < N - 1 ? i : N - 1);
}

// Plan of the even split (one workgroup of 1024 threads): prefix[q] = tiles of the work units of
// sequences 0 .. q - 1 (prefix[num_seqs] = total T), and for every wavefront the sequence that
// holds its first tile (-1: no tiles).
__global__ __launch_bounds__(1024) void decode_plan_kernel(DecodeParams p, DecodeShape s) {
    __shared__ int64_t part[1024];
    const int tid = threadIdx.x;
    const int per = (p.num_seqs + 1023) / 1024;
    const int a = min(tid * per, p.num_seqs), b = min(a + per, p.num_seqs);
    const int64_t ups = s.units_per_seq;
    int L, lo;
    int64_t sum = 0;
    // with one sequence per thread (up to 1024 sequences) its tile count stays in a register
    const int own = per == 1 && a < b ? seq_tiles(p, s, a, L, lo) : 0;
    if (per == 1) sum = own;
    else
        for (int q = a; q < b; ++q) sum += seq_tiles(p, s, q, L, lo);
    part[tid] = sum;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {           // inclusive scan of the chunk sums
        const int64_t v = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int64_t run = tid > 0 ? part[tid - 1] : 0;
    if (per == 1) {
        if (a < b) p.ws_prefix[a] = run * ups;
    } else {
        for (int q = a; q < b; ++q) {
            p.ws_prefix[q] = run * ups;
            run += seq_tiles(p, s, q, L, lo);
        }
    }
    const int64_t T = part[1023] * ups;
    if (tid == 0) p.ws_prefix[p.num_seqs] = T;
    if (per == 1 && T > 0) {
        // Wavefront i starts at tile floor(i T / N), inside sequence q iff it lies in
        // [P_q, P_q+1): the wavefronts ceil(P_q N / T) .. ceil(P_q+1 N / T) - 1, which this
        // sequence's thread writes (the ranges cover 0 .. N - 1 exactly).
        if (a < b) {
            const int64_t N = s.num_waves;
            const int64_t p0 = (tid > 0 ? part[tid - 1] : 0) * ups, p1 = part[tid] * ups;
            const int64_t lo = (p0 * N + T - 1) / T;
            const int64_t hi = min((p1 * N + T - 1) / T, N);
            for (int64_t i = lo; i < hi; ++i) p.ws_wseq[i] = a;
        }
        return;
    }
    for (int i = tid; i < s.num_waves; i += 1024) {
        const int64_t t = int64_t(i) * T / s.num_waves;
        int seq = -1;
        if (t < T) {
            int c0 = 0, c1 = 1023;                       // first chunk whose inclusive sum exceeds t
            while (c0 < c1) {
                const int mid = (c0 + c1) / 2;
                if (part[mid] * ups > t) c1 = mid; else c0 = mid + 1;
            }
            int q = min(c0 * per, p.num_seqs - 1);
            if (per > 1) {                               // the sequence inside the chunk
                int64_t r = c0 > 0 ? part[c0 - 1] * ups : 0;
                for (; q < p.num_seqs - 1; ++q) {
                    const int64_t ts = int64_t(seq_tiles(p, s, q, L, lo)) * ups;
                    if (r + ts > t) break;
                    r += ts;
                }
            }
            seq = q;
        }
        p.ws_wseq[i] = seq;
    }
}

// Block ids of key chunk ch of sequence seq (at most 128 blocks: lanes 0..63 and 64..127),
// clamped into the pool.  Entries past the sequence's last block are read (within the table row)
// but never used.
__device__ __forceinline__ void load_ids(const DecodeParams &p, const DecodeShape &s, int seq, int ch, int lane,
                                         int &ids0, int &ids1) {
    const int32_t *table = p.block_tables + int64_t(seq) * p.max_blocks;
    const int first = (ch * s.chunk) >> p.block_shift;
    const int last = p.max_blocks - 1;
    const int64_t nbm1 = p.num_blocks - 1;
    int64_t b0 = table[min(first + lane, last)];
    ids0 = int(b0 < 0 ? 0 : (b0 > nbm1 ? nbm1 : b0));
    ids1 = ids0;
    if ((s.chunk >> p.block_shift) > 64) {
        int64_t b1 = table[min(first + 64 + lane, last)];
        ids1 = int(b1 < 0 ? 0 : (b1 > nbm1 ? nbm1 : b1));
    }
}

// Up to a few thousand sequences a split wavefront plans its own share: it scans the tile counts of
// all sequences, 64 at a time -- their total, then the sequence holding its first tile and that
// sequence's prefix -- instead of a planning kernel running first.  Wavefront 0 stores the total for
// the merge kernel (which also reads the prefixes the split wavefronts store as they enter
// sequences; every sequence with tiles is entered by some wavefront).  Counts are 32-bit (the host
// enables this only while num_seqs * tiles per sequence stays below 2^30); the results are
// wave-uniform and returned through readfirstlane, so they live in scalar registers.
struct InWavePlan {
    int64_t total;      // tiles of all work units
    int seq;            // sequence holding the wavefront's first tile
    int64_t pre;        // tiles of the work units of the sequences before it
};
__device__ __forceinline__ InWavePlan plan_in_wave(const DecodeParams &p, const DecodeShape &shape, int wave,
                                                   int lane) {
    const int B = p.num_seqs;
    const int ups = shape.units_per_seq;
    auto tiles_of = [&](int q) -> int {
        int L_, lo_;
        return q < B ? seq_tiles(p, shape, q, L_, lo_) : 0;
    };
    InWavePlan ip{0, 0, 0};
    int tot = 0;
    for (int c0 = 0; c0 < B; c0 += 64) {
        int x = tiles_of(c0 + lane);
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) x += __shfl_xor(x, d, 64);
        tot += __builtin_amdgcn_readfirstlane(x);
    }
    ip.total = int64_t(tot) * ups;
    if (wave == 0 && lane == 0) p.ws_prefix[B] = ip.total;
    const int64_t tb = int64_t(wave) * ip.total / shape.num_waves;
    if (tb >= int64_t(wave + 1) * ip.total / shape.num_waves) return ip;     // no tiles
    const int tbu = int(tb / ups);           // its sequence is the first whose inclusive count exceeds tbu
    int base = 0;
    for (int c0 = 0; c0 < B; c0 += 64) {
        const int own = tiles_of(c0 + lane);
        int incl = own;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(incl, d, 64);
            if (lane >= d) incl += y;
        }
        const int chunk = __builtin_amdgcn_readlane(incl, 63);
        if (base + chunk > tbu) {
            const uint64_t hit = __builtin_amdgcn_ballot_w64(base + incl > tbu);
            const int l = int(__builtin_ctzll(hit));
            ip.seq = c0 + l;
            ip.pre = int64_t(base + __builtin_amdgcn_readlane(incl - own, l)) * ups;
            break;
        }
        base += chunk;
    }
    return ip;
}

// Even split: wavefront i takes tiles floor(i T / N) .. floor((i + 1) T / N) - 1 of the
// concatenated tiles of all work units (sequence-major, then KV head, then head group), i.e. a
// run of segments each inside one work unit.  A segment that is a whole unit writes the output;
// any other writes a partial (max, sum, weighted V) to slot i + u (unique: along a unit the
// wavefronts are consecutive and along a wavefront the units are), merged afterwards.
//   ONE_BLOCK: every tile lies inside one cache block (tile keys <= block size), so a tile needs
//              one block id; otherwise each load instruction looks up its own block.
//   KVH: KV heads per work unit (1, or 2 for small head groups): the R row groups of a load
//        instruction are then KVH adjacent head rows of R / KVH tokens, so one instruction reads
//        KVH * 16 * C contiguous bytes per token instead of one head's slice.
template <typename T, int D, int GP, int NI, bool ONE_BLOCK, int DEPTH, int OCC, int KVH>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void decode_split_kernel(DecodeParams p, DecodeShape shape) {
    constexpr int C = Geo<T, D>::kC, R = Geo<T, D>::kR, EPL = Geo<T, D>::kEpl;
    constexpr int TR = R / KVH;                        // tokens per load instruction
    constexpr int TILE = NI * TR;                      // keys per tile
    static_assert(R % KVH == 0, "row groups split evenly over the unit's KV heads");
    constexpr int WMASK = writer_mask<C, GP>();
    static_assert(NI % 2 == 0, "rows are paired for v_dot2");

    // Softmax weights of the current tile, [head][row group][instruction].
    __shared__ __align__(16) T p_lds[GP][R][NI];

    const int wave = blockIdx.x;
    const int lane = threadIdx.x;
    const int c = lane % C;
    const int r = lane / C;
    const int hk = r % KVH;                  // KV head of this row group within the unit
    const int tr = r / KVH;                  // token of this row group within an instruction
    const int my_head = head_of_lane<C, GP>(c);
    // A unit's query heads are "virtual heads" v = t * G + h of its KV head: query row t of the
    // sequence (t < qlen, position L - qlen + t), query head g * G + h.  With one query row they
    // are simply the group's query heads.
    const int group = p.num_heads / p.num_kv_heads;
    const int nh = shape.heads_per_group;
    const int ups = shape.units_per_seq;
    const int bmask = (1 << p.block_shift) - 1;
    // cache bytes per element: one for an FP8 cache (each lane then loads 8 codes, 8 bytes, and
    // widens them to the same four 16-bit pairs a bf16 / fp16 cache delivers)
    constexpr int CB = kFp8Cache<T> ? 1 : int(sizeof(T));
    typedef typename std::conditional<kFp8Cache<T>, uint2, uint4>::type LoadT;
    auto widen = [](const LoadT &x) -> uint4 {
        if constexpr (kFp8Cache<T>) return widen_e4m3<T>(x);
        else return x;
    };
    const uint32_t row_bytes = uint32_t(p.num_kv_heads) * D * CB;                   // one token, all heads
    const int64_t block_bytes = int64_t(row_bytes) << p.block_shift;
    const char *kcache = reinterpret_cast<const char *>(p.k_cache);
    const char *vcache = reinterpret_cast<const char *>(p.v_cache);
    const bool has_cap = p.softcap > 0.f;
    // scores in base-2 units: dot * scale * log2(e), or with a soft-cap c,
    // c log2(e) * tanh(dot * scale / c)
    const float qk_scale = has_cap ? p.scale / p.softcap : p.scale * kLog2e;
    const float cap2 = p.softcap * kLog2e;
    const bool has_alibi = p.alibi_slopes != nullptr;

    int64_t Ttot, pre = 0;
    int seq = 0;
    if (shape.inwave) {
        const InWavePlan ip = plan_in_wave(p, shape, wave, lane);
        Ttot = ip.total;
        seq = ip.seq;
        pre = ip.pre;
    } else {
        Ttot = p.ws_prefix[p.num_seqs];
        seq = p.ws_wseq[wave];
        pre = p.ws_prefix[seq];
    }
    const int64_t t_begin = int64_t(wave) * Ttot / shape.num_waves;
    const int64_t t_end = int64_t(wave + 1) * Ttot / shape.num_waves;
    if (t_begin >= t_end) return;

    int64_t t = t_begin;
    while (t < t_end) {
        int L, lo;
        const int ts = seq_tiles(p, shape, seq, L, lo);
        if (t >= pre + int64_t(ts) * ups) {               // (sequence without tiles, or exhausted)
            pre += int64_t(ts) * ups;
            ++seq;
            continue;
        }
        if (shape.inwave && lane == 0) p.ws_prefix[seq] = pre;
        const int64_t local = t - pre;
        const int u_in = int(local / ts);
        const int tile0 = int(local - int64_t(u_in) * ts);
        const int tile1 = int(min(int64_t(ts), int64_t(tile0) + (t_end - t)));
        const int gu = u_in / shape.head_groups;
        const int hgrp = u_in - gu * shape.head_groups;
        const int g = gu * KVH + hk;                       // this lane's KV head
        const int v0 = hgrp * nh;                          // first virtual head of the unit
        // virtual heads of the unit that exist: the last group of a split is short when the
        // virtual heads per KV head (group * qlen) are not a multiple of heads_per_group
        const int nreal = min(nh, group * p.qlen - v0);
        // query row (sequence row seq * qlen + t) and query head of virtual head v0 + h
        auto vrow = [&](int h) -> int64_t { return int64_t(seq) * p.qlen + (v0 + h) / group; };
        auto vhead = [&](int h) -> int { return g * group + (v0 + h) % group; };

        // ---- one segment: tiles tile0 .. tile1 - 1 of unit (seq, KV heads gu KVH.., hgrp)
        uint32_t q[GP][4];      // query chunks, head-permuted: slot s holds head s ^ my_head
        {
            const T *qbase = reinterpret_cast<const T *>(p.query) + c * EPL;
#pragma unroll
            for (int s = 0; s < GP; ++s) {
                const int hs = s ^ my_head;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (hs < nreal)
                    v = *reinterpret_cast<const uint4 *>(qbase + vrow(hs) * p.q_stride + int64_t(vhead(hs)) * D);
                q[s][0] = v.x; q[s][1] = v.y; q[s][2] = v.z; q[s][3] = v.w;
            }
        }
        const float slope2 = (has_alibi && my_head < nreal) ? p.alibi_slopes[vhead(my_head)] * kLog2e : 0.f;
        // positions: this lane's score head (row t) sits at L - qlen + t; the unit's rows span
        // pos_min .. L - 1, and the window start of the last row is lo_max
        const int pos = L - p.qlen + (my_head < nreal ? (v0 + my_head) / group : 0);
        const int pos_min = L - p.qlen;
        const int lo_lane = p.window > 0 ? max(0, pos - p.window + 1) : 0;
        const int lo_max = p.window > 0 ? max(0, L - p.window) : 0;
        const int kfirst = (lo / TILE + tile0) * TILE;
        const int kend = min(L, (lo / TILE + tile1) * TILE);
        // Lane part of every K/V address: row group r's token inside the instruction, KV head g, chunk c.
        const uint32_t lane_off = uint32_t(tr) * row_bytes + (uint32_t(g) * D + c * EPL) * CB;

        float m_run = -INFINITY;      // head my_head, this row group
        float l_run = 0.f;            // sum of rounded weights, head my_head, this row group
        float acc[GP][EPL];           // weighted V, all heads, this lane's elements, this row group
#pragma unroll
        for (int h = 0; h < GP; ++h)
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;

        auto scores = [&](int tb, const LoadT (&kr)[NI], float (&sc)[NI]) {
            const bool edge = tb < lo_max || tb + TILE - 1 > pos_min;   // uniform
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                float part_dot[GP];
                chunk_dots<T, GP>(widen(kr[i]), q, part_dot);
                butterfly<C, GP, 0>(part_dot);
                sc[i] = part_dot[0] * qk_scale;
            }
            if (has_cap) {
#pragma unroll
                for (int i = 0; i < NI; ++i) sc[i] = cap2 * tanh_fast(sc[i]);
            }
            if (has_alibi) {
#pragma unroll
                for (int i = 0; i < NI; ++i) sc[i] += slope2 * float(tb + i * TR + tr - pos);
            }
            if (edge) {
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    const int j = tb + i * TR + tr;
                    sc[i] = (j >= lo_lane && j <= pos) ? sc[i] : -INFINITY;
                }
            }
        };
        auto softmax_pv = [&](int tb, const float (&sc)[NI], const LoadT (&vraw)[NI]) {
            uint4 vr[NI];
#pragma unroll
            for (int i = 0; i < NI; ++i) vr[i] = widen(vraw[i]);
            // Lazily raised max: rescale only when some tile max exceeds the running max by more
            // than kRescaleSlack (always on the first tile, rarely afterwards); uniform over the wave.
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
                    pv[i] = to_elt<T>(pf);
                    psum += elt_to_f32(pv[i]);
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
            // Rows past the sequence's end hold unwritten cache bytes: zero them so that their
            // zero weights cannot meet a NaN.
            if (tb + TILE - 1 > L - 1) {
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    const bool past = tb + i * TR + tr > L - 1;
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
                    // row pair (2ip, 2ip+1) -> per element e the pair (v_2ip[e], v_2ip+1[e])
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
                        for (int e = 0; e < EPL; ++e) acc[h][e] = dot2<T>(pp, vp[e], acc[h][e]);
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

        // Key chunks of the segment (chunk boundaries are absolute multiples of shape.chunk, so a
        // chunk's block ids are one row of the table): ids per chunk, then its tiles in order with
        // two register sets in turn -- the next tile's K rows are requested once this tile's
        // scores have consumed K, its V rows once P.V has consumed V.  At a chunk's last tile the
        // loads re-read it (cache hits), keeping them unconditional.
        for (int ch = kfirst / shape.chunk; ch * shape.chunk < kend; ++ch) {
            int ids0, ids1;
            load_ids(p, shape, seq, ch, lane, ids0, ids1);
            const int cend = min(kend, (ch + 1) * shape.chunk);
            const int pblock0 = (ch * shape.chunk) >> p.block_shift;
            // Scalar part of the address of instruction i of the tile starting at tb: block base
            // plus the instruction's first token inside the block.  Tokens past the sequence's end
            // read unwritten slots of in-pool blocks; their scores are masked, their V rows zeroed.
            auto inst_base = [&](int tb, int i, int blk_tile) -> int64_t {
                const int row0 = tb + i * TR;
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
            auto load_rows = [&](const char *cache, int tb, LoadT (&x)[NI]) {
                const int blk = tile_block(tb);
#pragma unroll
                for (int i = 0; i < NI; ++i)
                    x[i] = *reinterpret_cast<const LoadT *>(cache + inst_base(tb, i, blk) + lane_off);
            };
            // DEPTH register sets in a ring: while tile t is scored and summed from set t % DEPTH,
            // tiles t + 1 .. t + DEPTH - 1 are in flight.  Loads past the chunk's last tile
            // re-read it (cache hits), keeping every load unconditional.
            const int tfirst = max(kfirst, ch * shape.chunk);
            const int tlast = ((cend - 1) / TILE) * TILE;
            LoadT kr[DEPTH][NI], vr[DEPTH][NI];
#pragma unroll
            for (int d = 0; d < DEPTH - 1; ++d) {
                const int tt = min(tfirst + d * TILE, tlast);
                load_rows(kcache, tt, kr[d]);
                load_rows(vcache, tt, vr[d]);
            }
            int tb = tfirst;
            bool done = false;
            while (!done) {
#pragma unroll
                for (int d = 0; d < DEPTH; ++d) {
                    if (!done) {
                        const int nd = (d + DEPTH - 1) % DEPTH;          // set of the previous tile: free
                        const int ahead = min(tb + (DEPTH - 1) * TILE, tlast);
                        load_rows(kcache, ahead, kr[nd]);
                        float sc[NI];
                        scores(tb, kr[d], sc);
                        load_rows(vcache, ahead, vr[nd]);
                        softmax_pv(tb, sc, vr[d]);
                        done = tb >= tlast;
                        tb += TILE;
                    }
                }
            }
        }

        // Bring the row groups of each KV head to a common max per head, then sum them; lanes of
        // row groups 0 .. KVH - 1 end with the segment's weighted V for all heads of their KV head.
        const float m_all = max_row_groups<C * KVH>(m_run);
        const float f_own = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_all);
#pragma unroll
        for (int h = 0; h < GP; ++h) {
            const float f = __shfl(f_own, r * C + lane_of_head<C, GP>(h), 64);
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] = sum_row_groups<C * KVH>(acc[h][e] * f);
        }
        const float l_sum = sum_row_groups<C * KVH>(l_run * f_own);
        if (tile0 == 0 && tile1 == ts) {
            // The whole (windowed) unit is this segment: write the normalized output.
#pragma unroll
            for (int h = 0; h < GP; ++h) {
                float lh = __shfl(l_sum, r * C + lane_of_head<C, GP>(h), 64);
                const float mh = __shfl(m_all, r * C + lane_of_head<C, GP>(h), 64);
                if (tr == 0 && h < nreal) {
                    T *out_row = reinterpret_cast<T *>(p.out) + (vrow(h) * p.num_heads + vhead(h)) * D;
                    // a sink logit joins the denominator only
                    if (p.sinks) lh += fast_exp2(p.sinks[vhead(h)] * kLog2e - mh);
                    const float inv = p.out_scale / lh;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) store_out<T>(out_row + c * EPL + e, acc[h][e] * inv);
                }
            }
        } else {
            const int64_t slot0 = (int64_t(wave) + int64_t(seq) * ups + u_in) * (KVH * nh) + hk * nh;
#pragma unroll
            for (int h = 0; h < GP; ++h) {
                const float lh = __shfl(l_sum, r * C + lane_of_head<C, GP>(h), 64);
                const float mh = __shfl(m_all, r * C + lane_of_head<C, GP>(h), 64);
                if (tr == 0 && h < nreal) {
                    const int64_t slot = slot0 + h;
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

        t += tile1 - tile0;
        if (tile1 == ts && u_in == ups - 1) {
            pre += int64_t(ts) * ups;
            ++seq;
        }
    }
}

// ---- MFMA variant for wide head groups ------------------------------------------------------
// With many virtual heads per KV head the dot products of the VALU kernel above cost more issue
// time than the bytes take to arrive: an FP8 cache with a group of 8 query heads (the bytes halve,
// the products do not), or 9 to 32 query rows x heads (wide groups, multi-token decode), which the
// VALU kernel could only split over units of 8 that each read K/V.  This kernel forms the products on
// the matrix unit instead, with the same work split, partial slots and merge:
//   * a work unit is one (sequence, KV head) with its nh <= 32 virtual heads as the columns of
//     v_mfma_f32_16x16x32_{bf16,f16}, in NB = 1 or 2 blocks of 16 that share every K and V
//     operand;
//   * a 32-key tile is two 16-key blocks; lane (k = lane % 16, g = lane / 16) loads 16 bytes at
//     byte 64 j + 16 g of key k's head row for j = 0 .. NL - 1, which for 16-bit rows is exactly
//     the A operand of S^T = K Q^T (d = 32 j + 8 g .. + 7 for MFMA j).  For an FP8 row a load
//     holds 16 codes (d = 64 j + 16 g .. + 15) that widen to the operands of MFMAs 2 j and
//     2 j + 1; the query chunks are gathered in the same d order, so each MFMA still pairs
//     equal d;
//   * S^T leaves lane (head k, g) the scores of keys 16 kk + 4 g + i; the weights, rounded to the
//     element type, are the B operand of O^T = V^T P^T as in the prefill kernel;
//   * V passes through per-wavefront LDS tiles (row-major, 32-byte units xor-swizzled by key) and
//     is read back transposed with ds_read_b64_tr_b16.  16-bit rows go there by load-to-LDS
//     copies into two stages: before any LDS read the compiler waits for every copy in flight,
//     so the next tile's loads are issued after this tile's reads and a deeper ring would gain
//     nothing.  FP8 codes are loaded into a ring of registers, widened and written;
//   * row sums come from an all-ones MFMA on the same rounded weights; the running max is raised
//     lazily as in the VALU kernel.
// 16-key blocks must lie inside one cache block (block size >= 16).  With up to 8 virtual heads
// of 16-bit rows the VALU kernel is as fast or faster (its products still hide behind the bytes),
// so it keeps them.
constexpr int kMfmaTile = 32;
constexpr int kMfmaMaxHeads = 32;          // two blocks of 16 MFMA columns
// Smallest group (query heads x query rows per KV head) that takes the MFMA kernel: 16-bit rows
// past the VALU kernel's 8 heads per unit; FP8 rows from 5 (at 4 the two kernels are level).
#ifndef PA_DECODE_MFMA_MIN_GROUP
#define PA_DECODE_MFMA_MIN_GROUP 9
#endif
#ifndef PA_DECODE_MFMA_MIN_GROUP8
#define PA_DECODE_MFMA_MIN_GROUP8 5
#endif

#ifndef PA_DECODE_MFMA_DEPTH
#define PA_DECODE_MFMA_DEPTH 2
#endif
#ifndef PA_DECODE_MFMA_OCC
#define PA_DECODE_MFMA_OCC 2
#endif
#ifndef PA_DECODE_MFMA_DEPTH8
#define PA_DECODE_MFMA_DEPTH8 3
#endif
#ifndef PA_DECODE_MFMA_OCC8
#define PA_DECODE_MFMA_OCC8 2
#endif
// With two column blocks (17 to 32 virtual heads) the second set of Q operands and accumulators
// leaves room for one wavefront per SIMD.
#ifndef PA_DECODE_MFMA_OCC_NB2
#define PA_DECODE_MFMA_OCC_NB2 1
#endif
template <typename T>
constexpr int mfma_depth() { return kFp8Cache<T> ? PA_DECODE_MFMA_DEPTH8 : PA_DECODE_MFMA_DEPTH; }
template <typename T, int NB>
constexpr int mfma_occ() {
    return NB > 1 ? PA_DECODE_MFMA_OCC_NB2 : (kFp8Cache<T> ? PA_DECODE_MFMA_OCC8 : PA_DECODE_MFMA_OCC);
}

// V tile swizzle: the 32-byte unit u of key r sits at unit u ^ (r & 7), so the 8 keys a
// transposing read touches at one d fall in distinct 32-byte units.
__device__ __forceinline__ int mfma_vswz(int r) { return r & 7; }

template <typename T, int D, int NB, int DEPTH, int OCC>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void decode_mfma_kernel(DecodeParams p, DecodeShape shape) {
    typedef typename Operand8<T>::type V8;
    constexpr int TILE = kMfmaTile;
    constexpr int CB = kFp8Cache<T> ? 1 : 2;      // cache bytes per element
    constexpr int DC = D / 32;                      // score MFMAs per 16-key block
    constexpr int DB = D / 16;                      // d-blocks of O^T
    constexpr int NL = D * CB / 64;                 // 16-byte loads per lane per 16-key block and row kind
    static_assert(D == 128, "the MFMA decode kernel is built for head size 128");
    constexpr bool VDMA = CB == 2;                  // V rows copied straight into LDS
    constexpr int VST = VDMA ? DEPTH : 1;           // V stages in LDS
    constexpr int NVR = VDMA ? 1 : NL;              // V register loads per 16-key block (unused with VDMA)
    __shared__ __align__(16) bf16_t vt[VST][TILE * D];

    const int wave = blockIdx.x;
    const int lane = threadIdx.x;
    const int l16 = lane & 15;
    const int lg = lane >> 4;
    const int group = p.num_heads / p.num_kv_heads;
    const int nh = shape.heads_per_group;
    const int ups = shape.units_per_seq;
    const int bmask = (1 << p.block_shift) - 1;
    const uint32_t row_bytes = uint32_t(p.num_kv_heads) * D * CB;
    const int64_t block_bytes = int64_t(row_bytes) << p.block_shift;
    const char *kcache = reinterpret_cast<const char *>(p.k_cache);
    const char *vcache = reinterpret_cast<const char *>(p.v_cache);
    const bool has_cap = p.softcap > 0.f;
    const float qk_scale = has_cap ? p.scale / p.softcap : p.scale * kLog2e;
    const float cap2 = p.softcap * kLog2e;
    const bool has_alibi = p.alibi_slopes != nullptr;
    const uint32_t one2 = uint32_t(__builtin_bit_cast(uint16_t, to_elt<T>(1.f))) * 0x10001u;
    const V8 ones = __builtin_bit_cast(V8, make_uint4(one2, one2, one2, one2));
    // element offset of the 8 query elements that lane group lg supplies to score MFMA n
    auto q_d = [&](int n) -> int { return CB == 1 ? 64 * (n >> 1) + 16 * lg + 8 * (n & 1) : 32 * n + 8 * lg; };
    // V^T operand reads (elements): lane l16 = 4 a + c of group lg reads key 4 lg + a (and 16 more)
    // at d = 16 db + 4 c
    int v_off[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
        v_off[db] = (4 * lg + (l16 >> 2)) * D + ((db ^ mfma_vswz(4 * lg + (l16 >> 2))) << 4) + 4 * (l16 & 3);
    // V copies: copy q (0..3) of a 16-key block fills its rows 4 q .. 4 q + 3, lane l the 16-byte
    // place l16 of row 4 q + lg; it fetches the source chunk that the swizzle puts there.  The
    // swizzle of row 4 q + lg depends on q only through q & 1.
    uint32_t v_chunk[2] = {0u, 0u};
    if constexpr (VDMA) {
#pragma unroll
        for (int par = 0; par < 2; ++par)
            v_chunk[par] = uint32_t((((l16 >> 1) ^ mfma_vswz(4 * par + lg)) << 1) | (l16 & 1)) * 16u;
    }

    int64_t Ttot, pre = 0;
    int seq = 0;
    if (shape.inwave) {
        const InWavePlan ip = plan_in_wave(p, shape, wave, lane);
        Ttot = ip.total;
        seq = ip.seq;
        pre = ip.pre;
    } else {
        Ttot = p.ws_prefix[p.num_seqs];
        seq = p.ws_wseq[wave];
        pre = p.ws_prefix[seq];
    }
    const int64_t t_begin = int64_t(wave) * Ttot / shape.num_waves;
    const int64_t t_end = int64_t(wave + 1) * Ttot / shape.num_waves;
    if (t_begin >= t_end) return;

    int64_t t = t_begin;
    while (t < t_end) {
        int L, lo;
        const int ts = seq_tiles(p, shape, seq, L, lo);
        if (t >= pre + int64_t(ts) * ups) {
            pre += int64_t(ts) * ups;
            ++seq;
            continue;
        }
        if (shape.inwave && lane == 0) p.ws_prefix[seq] = pre;
        const int64_t local = t - pre;
        const int u_in = int(local / ts);               // the KV head (one head group per KV head)
        const int tile0 = int(local - int64_t(u_in) * ts);
        const int tile1 = int(min(int64_t(ts), int64_t(tile0) + (t_end - t)));
        const int g = u_in;
        // this lane's columns: virtual head h = 16 b + l16 of column block b = query row h / G,
        // query head g G + h % G
        bool live[NB];
        int64_t my_row[NB];
        int my_head[NB], pos[NB], lo_h[NB];
        float slope2[NB];
        V8 qf[NB][DC];          // Q^T operands (zero for padding columns)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int h = 16 * b + l16;
            live[b] = h < nh;
            my_row[b] = int64_t(seq) * p.qlen + (live[b] ? h / group : 0);
            my_head[b] = g * group + (live[b] ? h % group : 0);
            const T *qrow = reinterpret_cast<const T *>(p.query) + my_row[b] * p.q_stride + int64_t(my_head[b]) * D;
#pragma unroll
            for (int n = 0; n < DC; ++n) {
                uint4 v = make_uint4(0u, 0u, 0u, 0u);
                if (live[b]) v = *reinterpret_cast<const uint4 *>(qrow + q_d(n));
                qf[b][n] = __builtin_bit_cast(V8, v);
            }
            slope2[b] = (has_alibi && live[b]) ? p.alibi_slopes[my_head[b]] * kLog2e : 0.f;
            pos[b] = L - p.qlen + (live[b] ? h / group : 0);
            lo_h[b] = p.window > 0 ? max(0, pos[b] - p.window + 1) : 0;
        }
        const int pos_min = L - p.qlen;
        const int lo_max = p.window > 0 ? max(0, L - p.window) : 0;
        const int kfirst = (lo / TILE + tile0) * TILE;
        const int kend = min(L, (lo / TILE + tile1) * TILE);
        const uint32_t head_off = uint32_t(g) * D * CB;
        const uint32_t lane_off = uint32_t(l16) * row_bytes + head_off + 16u * uint32_t(lg);
        const uint32_t v_lane0 = uint32_t(lg) * row_bytes + head_off + v_chunk[0];
        const uint32_t v_lane1 = uint32_t(lg) * row_bytes + head_off + v_chunk[1];

        float m_run[NB];
        floatx4_v o[NB][DB], lsum[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            m_run[b] = -INFINITY;
            lsum[b] = floatx4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int db = 0; db < DB; ++db) o[b][db] = floatx4_v{0.f, 0.f, 0.f, 0.f};
        }

        // One tile in two phases.  A: scores from the K registers kr, the V tile into LDS (FP8: from
        // the V registers vr; 16-bit rows were copied into stage vs), and the V^T operands read
        // back.  B: mask, softmax and the P.V and row-sum MFMAs.  The compiler waits for every
        // outstanding load-to-LDS copy before an LDS read, so with copies the next tile's loads
        // are issued between the two phases, after this tile's reads.
        floatx4_v s[NB][2];
        V8 vop[DB];
        auto tile_a = [&](int tb, const uint4 (&kr)[2][NL], const uint4 (&vr)[2][NVR], bf16_t *vs) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
                for (int b = 0; b < NB; ++b) s[b][kk] = floatx4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int n = 0; n < DC; ++n) {
                    V8 ka;
                    if constexpr (CB == 1) {
                        const uint4 c = kr[kk][n >> 1];
                        ka = __builtin_bit_cast(V8, widen_e4m3<T>((n & 1) ? make_uint2(c.z, c.w) : make_uint2(c.x, c.y)));
                    } else {
                        ka = __builtin_bit_cast(V8, kr[kk][n]);
                    }
#pragma unroll
                    for (int b = 0; b < NB; ++b) s[b][kk] = mfma16(ka, qf[b][n], s[b][kk]);
                }
            }
            const bool tail = tb + TILE > L;
            if constexpr (!VDMA) {
                // FP8: widened V rows into the LDS tile (rows past the sequence's end zeroed: their
                // zero weights must not meet unwritten cache bytes)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int key = 16 * kk + l16;
                    const bool past = tail && tb + key >= L;
                    bf16_t *row = vs + key * D;
#pragma unroll
                    for (int j = 0; j < NL; ++j) {
                        const uint4 c = vr[kk][j];
                        uint4 lo8 = widen_e4m3<T>(make_uint2(c.x, c.y));
                        uint4 hi8 = widen_e4m3<T>(make_uint2(c.z, c.w));
                        if (past) lo8 = hi8 = make_uint4(0u, 0u, 0u, 0u);
                        const int u = 4 * j + lg;                 // 32-byte unit of d = 64 j + 16 lg
                        uint4 *dst = reinterpret_cast<uint4 *>(row + ((u ^ mfma_vswz(key)) << 4));
                        dst[0] = lo8;
                        dst[1] = hi8;
                    }
                }
            }
            wave_lds_sync();
            // copied V rows past the sequence's end hold unwritten cache bytes: their weights are
            // zero, but 0 * NaN would poison O, so the tail tile's operands of those keys are zeroed
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const bf16_t *vb = vs + v_off[db];
                v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)vb);
                v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vb + 16 * D));
                if (VDMA && tail) {
                    // lane holds keys 4 lg + i (a) and 16 + 4 lg + i (b) of the tile
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        a[i] = tb + 4 * lg + i < L ? a[i] : short(0);
                        b[i] = tb + 16 + 4 * lg + i < L ? b[i] : short(0);
                    }
                }
                const v4i16 both[2] = {a, b};
                vop[db] = __builtin_bit_cast(V8, both);
            }
            wave_lds_sync();
        };
        auto tile_b = [&](int tb) {
            // scores in base-2 units, bias and mask: key tb + 16 kk + 4 lg + i
            const bool edge = tb < lo_max || tb + TILE - 1 > pos_min;
            bool raise = false;
            float tmax[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float x = s[b][kk][i] * qk_scale;
                        if (has_cap) x = cap2 * tanh_fast(x);
                        const int key = tb + 16 * kk + 4 * lg + i;
                        if (has_alibi) x += slope2[b] * float(key - pos[b]);
                        if (edge) x = (key >= lo_h[b] && key <= pos[b]) ? x : -INFINITY;
                        s[b][kk][i] = x;
                    }
                float mx = fmaxf(fmaxf(s[b][0][0], s[b][0][1]), s[b][0][2]);
                mx = fmaxf(fmaxf(mx, s[b][0][3]), s[b][1][0]);
                mx = fmaxf(fmaxf(mx, s[b][1][1]), s[b][1][2]);
                tmax[b] = max_xor32(max_xor16(fmaxf(mx, s[b][1][3])));
                raise |= tmax[b] > m_run[b] + kRescaleSlack;
            }
            if (__builtin_amdgcn_ballot_w64(raise) != 0) {
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const float m_new = fmaxf(m_run[b], tmax[b]);
                    const float alpha = (m_run[b] == -INFINITY) ? 0.f : fast_exp2(m_run[b] - m_new);
                    m_run[b] = m_new;
                    lsum[b] *= alpha;
#pragma unroll
                    for (int db = 0; db < DB; ++db) o[b][db] *= alpha;
                }
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                uint32_t pk[2][2];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    float pf[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        pf[i] = (s[b][kk][i] == -INFINITY) ? 0.f : fast_exp2(s[b][kk][i] - m_run[b]);
                    pk[kk][0] = pack_x2<T>(pf[0], pf[1]);
                    pk[kk][1] = pack_x2<T>(pf[2], pf[3]);
                }
                const V8 pb = __builtin_bit_cast(V8, make_uint4(pk[0][0], pk[0][1], pk[1][0], pk[1][1]));
#pragma unroll
                for (int db = 0; db < DB; ++db) o[b][db] = mfma16(vop[db], pb, o[b][db]);
                lsum[b] = mfma16(ones, pb, lsum[b]);
            }
        };

        for (int ch = kfirst / shape.chunk; ch * shape.chunk < kend; ++ch) {
            int ids0, ids1;
            load_ids(p, shape, seq, ch, lane, ids0, ids1);
            const int cend = min(kend, (ch + 1) * shape.chunk);
            const int pblock0 = (ch * shape.chunk) >> p.block_shift;
            // base of 16-key block kk of the tile at tb (one cache block holds all 16 keys)
            auto block_base = [&](int tb, int kk) -> int64_t {
                const int row0 = tb + 16 * kk;
                const int bidx = (row0 >> p.block_shift) - pblock0;
                const int blk = __builtin_amdgcn_readlane(bidx < 64 ? ids0 : ids1, bidx & 63);
                return int64_t(blk) * block_bytes + int64_t(row0 & bmask) * row_bytes;
            };
            auto load_k = [&](int tb, uint4 (&x)[2][NL]) {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const char *base = kcache + block_base(tb, kk) + lane_off;
#pragma unroll
                    for (int j = 0; j < NL; ++j) x[kk][j] = *reinterpret_cast<const uint4 *>(base + 64 * j);
                }
            };
            // V of the tile at tb: copies into stage vs (16-bit) or loads into registers (FP8)
            auto load_v = [&](int tb, uint4 (&x)[2][NVR], bf16_t *vs) {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    if constexpr (VDMA) {
                        const char *base = vcache + block_base(tb, kk);
                        const uint32_t lds0 = lds_address(vs + 16 * kk * D);
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            dma16_at(base, (q & 1) ? v_lane1 : v_lane0, uint32_t(4 * q) * row_bytes,
                                     lds0 + uint32_t(4 * q * D * 2));
                    } else {
                        const char *base = vcache + block_base(tb, kk) + lane_off;
#pragma unroll
                        for (int j = 0; j < NL; ++j) x[kk][j] = *reinterpret_cast<const uint4 *>(base + 64 * j);
                    }
                }
            };
            const int tfirst = max(kfirst, ch * shape.chunk);
            const int tlast = ((cend - 1) / TILE) * TILE;
            uint4 kr[DEPTH][2][NL], vr[DEPTH][2][NVR];
#pragma unroll
            for (int d = 0; d < DEPTH - 1; ++d) {
                const int tt = min(tfirst + d * TILE, tlast);
                load_k(tt, kr[d]);
                load_v(tt, vr[d], vt[VDMA ? d : 0]);
            }
            int tb = tfirst;
            bool done = false;
            while (!done) {
#pragma unroll
                for (int d = 0; d < DEPTH; ++d) {
                    if (!done) {
                        const int nd = (d + DEPTH - 1) % DEPTH;
                        const int ahead = min(tb + (DEPTH - 1) * TILE, tlast);
                        if constexpr (VDMA) {
                            tile_a(tb, kr[d], vr[d], vt[d]);
                            load_k(ahead, kr[nd]);
                            load_v(ahead, vr[nd], vt[nd]);
                        } else {
                            load_k(ahead, kr[nd]);
                            load_v(ahead, vr[nd], vt[0]);
                            tile_a(tb, kr[d], vr[d], vt[0]);
                        }
                        tile_b(tb);
                        done = tb >= tlast;
                        tb += TILE;
                    }
                }
            }
            if constexpr (VDMA) {
                // no copy may still be writing a stage when the next chunk or unit reuses it
                __builtin_amdgcn_s_waitcnt(0x0F70);
                wave_lds_sync();
            }
        }

#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (!live[b]) continue;
            const float l_sum = lsum[b][0];
            if (tile0 == 0 && tile1 == ts) {
                float lh = l_sum;
                if (p.sinks) lh += fast_exp2(p.sinks[my_head[b]] * kLog2e - m_run[b]);
                const float inv = p.out_scale / lh;
                T *out_row = reinterpret_cast<T *>(p.out) + (my_row[b] * p.num_heads + my_head[b]) * D + 4 * lg;
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const uint2 w = make_uint2(pack_x2<T>(o[b][db][0] * inv, o[b][db][1] * inv),
                                               pack_x2<T>(o[b][db][2] * inv, o[b][db][3] * inv));
                    *reinterpret_cast<uint2 *>(out_row + 16 * db) = w;
                }
            } else {
                const int64_t slot = (int64_t(wave) + int64_t(seq) * ups + u_in) * nh + 16 * b + l16;
                float *dst = p.ws_acc + slot * D + 4 * lg;
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    *reinterpret_cast<float4 *>(dst + 16 * db) =
                        make_float4(o[b][db][0], o[b][db][1], o[b][db][2], o[b][db][3]);
                if (lg == 0) {
                    p.ws_ml[slot * 2] = m_run[b];
                    p.ws_ml[slot * 2 + 1] = l_sum;
                }
            }
        }

        t += tile1 - tile0;
        if (tile1 == ts && u_in == ups - 1) {
            pre += int64_t(ts) * ups;
            ++seq;
        }
    }
}

// Merge, one wavefront per (work unit, head of its group): zero rows of empty sequences, and for
// units split over several wavefronts out = sum_i 2^(m_i - M) acc_i / sum_i 2^(m_i - M) l_i over
// their partials.  Lane j takes partial i0 + j (+ 64 k) for the (max, sum) step, so the step
// costs a few dependent loads however many partials there are.
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeParams p, DecodeShape shape) {
    constexpr int PER = D / 64;
    const int lane = threadIdx.x;
    const int nh = shape.heads_per_group;
    const int nhu = nh * shape.kvh;          // heads of a work unit
    const int u = blockIdx.x / nhu;
    const int hh = blockIdx.x - u * nhu;
    const int ups = shape.units_per_seq;
    const int seq = u / ups;
    const int u_in = u - seq * ups;
    const int gu = u_in / shape.head_groups;
    const int hgrp = u_in - gu * shape.head_groups;
    const int g = gu * shape.kvh + hh / nh;
    const int group = p.num_heads / p.num_kv_heads;
    const int v = hgrp * nh + hh % nh;                     // virtual head: query row v / G, head v % G
    if (v >= group * p.qlen) return;                       // past the last virtual head (a short last group)
    const int head = g * group + v % group;
    T *out_row = reinterpret_cast<T *>(p.out) + ((int64_t(seq) * p.qlen + v / group) * p.num_heads + head) * D;
    int L, lo;
    const int ts = seq_tiles(p, shape, seq, L, lo);
    if (ts == 0) {                          // empty sequence: zero output
#pragma unroll
        for (int k = 0; k < PER; ++k) store_out<T>(out_row + lane + 64 * k, 0.f);
        return;
    }
    const int64_t Ttot = p.ws_prefix[p.num_seqs];
    const int64_t U = p.ws_prefix[seq] + int64_t(u_in) * ts;
    const int i0 = wave_of_tile(U, Ttot, shape.num_waves);
    const int i1 = wave_of_tile(U + ts - 1, Ttot, shape.num_waves);
    if (i0 == i1) return;                   // one segment: its wavefront wrote the output
    const int n = i1 - i0 + 1;
    // Wavefronts between i0 and i1 with no tiles at all (only when there are fewer tiles than
    // wavefronts) wrote nothing and are skipped.
    auto has_tiles = [&](int i) {
        return int64_t(i) * Ttot / shape.num_waves < int64_t(i + 1) * Ttot / shape.num_waves;
    };
    auto slot_of = [&](int j) { return (int64_t(i0 + j) + u) * nhu + hh; };
    // (m, l) of partial j in lane j (chunks of 64), maximum over all of them
    float M = -INFINITY;
    for (int j = lane; j < n; j += 64)
        if (has_tiles(i0 + j)) M = fmaxf(M, p.ws_ml[slot_of(j) * 2]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    float den = 0.f;
    float num[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) num[k] = 0.f;
    for (int j0 = 0; j0 < n; j0 += 64) {
        const int j = j0 + lane;
        float f = 0.f;
        if (j < n && has_tiles(i0 + j)) {
            const float2 ml = *reinterpret_cast<const float2 *>(p.ws_ml + slot_of(j) * 2);
            f = fast_exp2(ml.x - M);
            den += f * ml.y;
        }
        const int cnt = min(64, n - j0);
        // partials four at a time: their accumulator rows are loaded together (a slot of a
        // wavefront that wrote nothing holds stale bits; the select drops them, NaN included)
        for (int jb = 0; jb < cnt; jb += 4) {
            float a[4][PER];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int jj = min(jb + q, cnt - 1);
                const float *row = p.ws_acc + slot_of(j0 + jj) * D;
#pragma unroll
                for (int k = 0; k < PER; ++k) a[q][k] = row[lane + 64 * k];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float fj = jb + q < cnt ? __shfl(f, jb + q, 64) : 0.f;
#pragma unroll
                for (int k = 0; k < PER; ++k) num[k] += fj != 0.f ? fj * a[q][k] : 0.f;
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off, 64);
    if (p.sinks) den += fast_exp2(p.sinks[head] * kLog2e - M);
    const float inv = p.out_scale / den;
#pragma unroll
    for (int k = 0; k < PER; ++k) store_out<T>(out_row + lane + 64 * k, num[k] * inv);
}

// KV heads per work unit: 2 for head groups of 1, 2 or 8 (whole 512-byte runs of two adjacent head
// rows per token instead of 256-byte slices; 2.7% faster for the 8 virtual heads of a two-row
// decode over 256 bf16 sequences of 512-8192 tokens with 32/8 heads), 4 for 16-bit head groups of 4
// (1 KB runs: one token's four head rows per load instruction, 1.3-2.8% faster than two on that
// single-row decode), when the KV head count divides by it;
// never more than the rows of one load instruction.
#ifndef PA_DECODE_KVH_S
#define PA_DECODE_KVH_S 2
#endif
#ifndef PA_DECODE_KVH_M
#define PA_DECODE_KVH_M 4
#endif
#ifndef PA_DECODE_KVH_M8
#define PA_DECODE_KVH_M8 2
#endif
#ifndef PA_DECODE_KVH_B
#define PA_DECODE_KVH_B 2
#endif
template <typename T, int GP, int D>
constexpr int kvh_max() {
    constexpr int k = sizeof(T) == 4 ? 1
                      : GP <= 2 ? PA_DECODE_KVH_S
                      : GP == 4 ? (kFp8Cache<T> ? PA_DECODE_KVH_M8 : PA_DECODE_KVH_M)
                                : PA_DECODE_KVH_B;
    return k <= Geo<T, D>::kR ? k : Geo<T, D>::kR;
}

template <typename T, int D, int GP, int KVH>
constexpr int tile_keys() { return tile_loads<T, GP>() * Geo<T, D>::kR / KVH; }

template <typename T, int D, int GP, bool ONE, int KVH>
const void *split_kernel_fn() {
    return reinterpret_cast<const void *>(
        &decode_split_kernel<T, D, GP, tile_loads<T, GP>(), ONE, tile_depth<T, GP>(), tile_occ<T, GP>(), KVH>);
}

// Resident wavefronts of the split kernel instance on the current device (occupancy x CUs),
// cached per device and instance.  Host threads may race to fill an entry; they compute the same
// value, and the atomic makes the race well defined.
template <typename T, int D, int GP, int KVH>
int split_waves(int block_shift) {
    constexpr int TILE = tile_keys<T, D, GP, KVH>();
    const bool one = (1 << block_shift) >= TILE;
    static std::atomic<int> cache[64][2];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    std::atomic<int> &slot = cache[dev][one ? 1 : 0];
    const int known = slot.load(std::memory_order_relaxed);
    if (known > 0) return known;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    const void *fn = one ? split_kernel_fn<T, D, GP, true, KVH>() : split_kernel_fn<T, D, GP, false, KVH>();
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 64, 0) != hipSuccess || per_cu <= 0) per_cu = 8;
    slot.store(cus * per_cu, std::memory_order_relaxed);
    return cus * per_cu;
}

template <typename T, int D, int GP, bool ONE, int KVH>
hipError_t launch_split(const DecodeParams &p, const DecodeShape &s, hipStream_t stream) {
    hipLaunchKernelGGL(
        (decode_split_kernel<T, D, GP, tile_loads<T, GP>(), ONE, tile_depth<T, GP>(), tile_occ<T, GP>(), KVH>),
        dim3(unsigned(s.num_waves)), dim3(64), 0, stream, p, s);
    return hipGetLastError();
}

template <typename T, int D, int GP, int KVH>
hipError_t launch_typed(const DecodeParams &p, const DecodeShape &s, hipStream_t stream) {
    constexpr int TILE = tile_keys<T, D, GP, KVH>();
    const int64_t units = int64_t(p.num_seqs) * s.units_per_seq;
    if (units > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipError_t e = hipSuccess;
    if (!s.inwave) {
        hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, stream, p, s);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const bool one_block = (1 << p.block_shift) >= TILE;
    e = one_block ? launch_split<T, D, GP, true, KVH>(p, s, stream) : launch_split<T, D, GP, false, KVH>(p, s, stream);
    if (e != hipSuccess) return e;
    const int64_t merges = units * s.heads_per_group * KVH;
    if (merges > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(unsigned(merges)), dim3(64), 0, stream, p, s);
    return hipGetLastError();
}

// Resident wavefronts of the MFMA instance for element type T and NB column blocks (cached per
// device, as split_waves).
template <typename T, int NB>
int mfma_waves() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    const int known = cache[dev].load(std::memory_order_relaxed);
    if (known > 0) return known;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    const void *fn =
        reinterpret_cast<const void *>(&decode_mfma_kernel<T, 128, NB, mfma_depth<T>(), mfma_occ<T, NB>()>);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 64, 0) != hipSuccess || per_cu <= 0) per_cu = 8;
    cache[dev].store(cus * per_cu, std::memory_order_relaxed);
    return cus * per_cu;
}

template <typename T, int NB>
hipError_t launch_mfma(const DecodeParams &p, const DecodeShape &s, hipStream_t stream) {
    const int64_t units = int64_t(p.num_seqs) * s.units_per_seq;
    if (units > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (!s.inwave) {
        hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, stream, p, s);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((decode_mfma_kernel<T, 128, NB, mfma_depth<T>(), mfma_occ<T, NB>()>),
                       dim3(unsigned(s.num_waves)), dim3(64), 0, stream, p, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t merges = units * s.heads_per_group;
    if (merges > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_merge_kernel<T, 128>), dim3(unsigned(merges)), dim3(64), 0, stream, p, s);
    return hipGetLastError();
}

// KV heads per unit actually used: kvh_max when the KV head count divides by it, else 2 (when
// kvh_max is 4 and the count is even), else 1.
template <typename T, int GP, int D>
constexpr int kvh_mid() { return kvh_max<T, GP, D>() >= 4 ? 2 : 1; }

template <typename T, int D, int GP>
hipError_t launch_kvh(const DecodeParams &p, const DecodeShape &s, hipStream_t stream) {
    constexpr int K1 = kvh_max<T, GP, D>(), K2 = kvh_mid<T, GP, D>();
    if constexpr (K1 > 1) {
        if (s.kvh == K1) return launch_typed<T, D, GP, K1>(p, s, stream);
    }
    if constexpr (K2 > 1) {
        if (s.kvh == K2) return launch_typed<T, D, GP, K2>(p, s, stream);
    }
    return launch_typed<T, D, GP, 1>(p, s, stream);
}

template <typename T, int D>
hipError_t launch_group(const DecodeParams &p, const DecodeShape &s, int padded_group, hipStream_t stream) {
    switch (padded_group) {
        case 1: return launch_kvh<T, D, 1>(p, s, stream);
        case 2: return launch_kvh<T, D, 2>(p, s, stream);
        case 4: return launch_kvh<T, D, 4>(p, s, stream);
        case 8: return launch_kvh<T, D, 8>(p, s, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename T, int D, int GP>
void instance_info_gp(int num_kv_heads, int block_shift, int &kvh, int &tile, int &waves) {
    constexpr int K1 = kvh_max<T, GP, D>(), K2 = kvh_mid<T, GP, D>();
    if (K1 > 1 && num_kv_heads % K1 == 0) {
        kvh = K1;
        tile = tile_keys<T, D, GP, K1>();
        waves = split_waves<T, D, GP, K1>(block_shift);
    } else if (K2 > 1 && num_kv_heads % K2 == 0) {
        kvh = K2;
        tile = tile_keys<T, D, GP, K2>();
        waves = split_waves<T, D, GP, K2>(block_shift);
    } else {
        kvh = 1;
        tile = tile_keys<T, D, GP, 1>();
        waves = split_waves<T, D, GP, 1>(block_shift);
    }
}

template <typename T, int D>
void instance_info(int padded_group, int num_kv_heads, int block_shift, int &kvh, int &tile, int &waves) {
    switch (padded_group) {
        case 1: instance_info_gp<T, D, 1>(num_kv_heads, block_shift, kvh, tile, waves); break;
        case 2: instance_info_gp<T, D, 2>(num_kv_heads, block_shift, kvh, tile, waves); break;
        case 4: instance_info_gp<T, D, 4>(num_kv_heads, block_shift, kvh, tile, waves); break;
        default: instance_info_gp<T, D, 8>(num_kv_heads, block_shift, kvh, tile, waves); break;
    }
}

template <typename T>
struct TypeTag { typedef T type; };

// Calls f(TypeTag<element type>, integral_constant<head size>) for a kernel element code and a
// head size of 64, 128 or 256.
template <typename F>
auto dispatch_type_size(int dtype, int head_size, F &&f) {
    auto by_size = [&](auto t) {
        if (head_size == 64) return f(t, std::integral_constant<int, 64>());
        if (head_size == 128) return f(t, std::integral_constant<int, 128>());
        return f(t, std::integral_constant<int, 256>());
    };
    switch (dtype) {
        case 1: return by_size(TypeTag<bf16_t>());
        case 2: return by_size(TypeTag<f16_t>());
        case 3: return by_size(TypeTag<bf16_c8_t>());
        case 4: return by_size(TypeTag<f16_c8_t>());
        default: return by_size(TypeTag<float>());
    }
}

}  // namespace

DecodePlan plan_decode(int32_t num_heads, int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                       int32_t dtype, int32_t num_seqs, int32_t max_seq_len, int32_t query_len) {
    int block_shift = 0;
    while ((1 << block_shift) < block_size) ++block_shift;
    DecodePlan plan{};
    // the query heads of one KV head times the query rows per sequence share its K/V bytes
    const int group = num_heads / num_kv_heads * (query_len > 1 ? query_len : 1);
    plan.head_groups = (group + kMaxGroup - 1) / kMaxGroup;
    plan.heads_per_group = (group + plan.head_groups - 1) / plan.head_groups;
    plan.padded_group = 1;
    while (plan.padded_group < plan.heads_per_group) plan.padded_group <<= 1;
    // Block-id chunk: 128 blocks (two id registers per lane), at most 4096 keys.
    plan.chunk = (128 << block_shift) < 4096 ? (128 << block_shift) : 4096;
    int kvh = 1, tile = 32, waves = 2048;
    // Wide groups of 16-bit (or FP8-cache) rows at head size 128 take the MFMA kernel: one work
    // unit per (sequence, KV head) with all its virtual heads as MFMA columns.
    const int mfma_min = (dtype == 3 || dtype == 4) ? PA_DECODE_MFMA_MIN_GROUP8 : PA_DECODE_MFMA_MIN_GROUP;
    plan.mfma = dtype >= 1 && dtype <= 4 && head_size == 128 && block_shift >= 4 && group >= mfma_min &&
                group <= kMfmaMaxHeads;
    if (plan.mfma) {
        plan.head_groups = 1;
        plan.heads_per_group = group;
        plan.padded_group = group > 16 ? 32 : 16;
        tile = kMfmaTile;
        const bool two = group > 16;
        switch (dtype) {
            case 1: waves = two ? mfma_waves<bf16_t, 2>() : mfma_waves<bf16_t, 1>(); break;
            case 2: waves = two ? mfma_waves<f16_t, 2>() : mfma_waves<f16_t, 1>(); break;
            case 3: waves = two ? mfma_waves<bf16_c8_t, 2>() : mfma_waves<bf16_c8_t, 1>(); break;
            default: waves = two ? mfma_waves<f16_c8_t, 2>() : mfma_waves<f16_c8_t, 1>(); break;
        }
    } else {
        dispatch_type_size(dtype, head_size, [&](auto t, auto d) {
            instance_info<typename decltype(t)::type, decltype(d)::value>(plan.padded_group, num_kv_heads, block_shift,
                                                                          kvh, tile, waves);
            return 0;
        });
    }
    plan.kv_per_unit = kvh;
    plan.units_per_seq = num_kv_heads / kvh * plan.head_groups;
    plan.tile = tile;
    plan.num_waves = waves;
    // Workspace: tile prefix per sequence, first sequence per wavefront, then the partial slots
    // (one per (wavefront, unit) pair that can meet: at most num_waves + units) of nh heads.
    const size_t units = size_t(num_seqs) * plan.units_per_seq;
    const size_t slots = (size_t(waves) + units) * plan.heads_per_group * kvh;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    plan.ws_prefix_off = 0;
    plan.ws_wseq_off = up(size_t(num_seqs + 1) * sizeof(int64_t));
    plan.ws_acc_off = plan.ws_wseq_off + up(size_t(waves) * sizeof(int32_t));
    plan.ws_ml_off = plan.ws_acc_off + up(slots * head_size * sizeof(float));
    plan.workspace_bytes = plan.ws_ml_off + up(slots * 2 * sizeof(float));
    (void)max_seq_len;
    return plan;
}

hipError_t launch_decode(const DecodeParams &p, const DecodePlan &plan, int dtype, int head_size,
                         hipStream_t stream) {
    DecodeShape s;
    s.chunk = plan.chunk;
    s.head_groups = plan.head_groups;
    s.heads_per_group = plan.heads_per_group;
    s.units_per_seq = plan.units_per_seq;
    s.num_waves = plan.num_waves;
    s.tile = plan.tile;
    s.max_len = p.max_seq_len;
    s.kvh = plan.kv_per_unit;
    s.inwave = p.num_seqs <= kInWavePlanMax &&
                       int64_t(p.num_seqs) * ((int64_t(p.max_seq_len) + s.tile - 1) / s.tile + 1) < (int64_t(1) << 30)
                   ? 1 : 0;
    if (plan.mfma) {
        const bool two = s.heads_per_group > 16;
        switch (dtype) {
            case 1: return two ? launch_mfma<bf16_t, 2>(p, s, stream) : launch_mfma<bf16_t, 1>(p, s, stream);
            case 2: return two ? launch_mfma<f16_t, 2>(p, s, stream) : launch_mfma<f16_t, 1>(p, s, stream);
            case 3: return two ? launch_mfma<bf16_c8_t, 2>(p, s, stream) : launch_mfma<bf16_c8_t, 1>(p, s, stream);
            default: return two ? launch_mfma<f16_c8_t, 2>(p, s, stream) : launch_mfma<f16_c8_t, 1>(p, s, stream);
        }
    }
    return dispatch_type_size(dtype, head_size, [&](auto t, auto d) {
        return launch_group<typename decltype(t)::type, decltype(d)::value>(p, s, plan.padded_group, stream);
    });
}

}  // namespace pa
