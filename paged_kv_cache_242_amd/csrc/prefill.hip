// Variable-length causal prefill with a paged cached context (chunked prefill).
//
// What is computed (aphrodite-engine "xformers.py": XFormersMetadata note on context_len /
// subquery_len / seqlen, subquery_start_loc, XFormersImpl.forward with forward_prefix and
// _run_memory_efficient_xformers_forward; vLLM "cpu_attn": flash_attn_varlen_func call): the
// subquery token t of sequence i sits at position c_i + t and attends causally to keys
// 0 .. c_i + t, the first c_i of which are read from the paged cache through the block table and
// the rest from the key/value rows of the call; sliding window, ALiBi, soft-cap and sinks as in
// decode.
//
// 16-bit kernel (MFMA; bf16 or fp16 elements).  A workgroup of 4 wavefronts owns 128 (query row, head) pairs of one
// sequence and KV head: 32 consecutive rows of 4 query heads of the group when the group size is
// a multiple of 4 (all four wavefronts then share one diagonal), 64 rows of 2 heads, or 128 rows
// of one head.  Each wavefront owns 32 rows of one head (two 16-row MFMA blocks).  The workgroup
// walks the needed keys in 64-key tiles that are staged in LDS:
//   * K tile row-major [64][D] (16-byte chunks xor-swizzled by row, so the 16 rows an MFMA
//     operand read touches hit distinct banks);
//   * V tile row-major [64][D] (32-byte units xor-swizzled by row), read transposed by
//     ds_read_b64_tr_b16.
// Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_16x16x32_{bf16,f16}: the accumulator
// layout then gives every lane 4 consecutive keys of ONE query row, so the row's max and sum
// need only two cross-lane steps, and two key blocks of those lanes are exactly the 8-key
// slice a lane must supply as the B operand of O^T = V^T P^T (the k index of A and B uses the
// same slot->key assignment, so the pairing is exact).  O^T accumulates in fp32 registers, with
// the lane's query row fixed, so rescaling by the running max is lane-local.
//
// fp32 kernel: a plain wavefront-per-(row, head) VALU loop (no MFMA for fp32 here).
#include <math.h>

#include <type_traits>

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kRowsPerBlock = 128;   // (query row, head) pairs per workgroup: 4 wavefronts x 32 rows
constexpr int kBN = 64;        // keys per tile
constexpr int kThreads = 256;
// The running row max is raised only when a tile's max exceeds it by more than this (base-2
// units); until then weights are <= 2^8 and the O accumulators need no rescaling.
constexpr float kRescaleSlack = 8.0f;

struct SeqInfo {
    int start;      // first query/key row of the sequence
    int n;          // subquery rows
    int c;          // keys read from the cache (those below c); keys from c on are the call's new rows
    int q0;         // position of subquery row 0 (c, except in the uniform multi-token mode)
    bool empty;     // uniform mode: a padded (or too short) sequence, whose rows are written as zeros
};

__device__ __forceinline__ SeqInfo seq_info(const PrefillParams &p, int seq) {
    SeqInfo s;
    if (p.uniform_qlen > 0) {
        // multi-token decode: query_len rows per sequence at seq * query_len, at positions
        // L - query_len .. L - 1, every key (0 .. L - 1) already in the cache
        const int L = max(0, min(p.seq_lens[seq], min(p.max_blocks << p.block_shift, p.max_context_len)));
        s.start = seq * p.uniform_qlen;
        s.n = p.uniform_qlen;
        s.c = L;
        s.q0 = L - p.uniform_qlen;
        s.empty = L < p.uniform_qlen;
        return s;
    }
    int a = p.cu_subquery[seq];
    int b = p.cu_subquery[seq + 1];
    a = max(0, min(a, int(p.num_tokens)));
    b = max(a, min(b, int(p.num_tokens)));
    s.start = a;
    s.n = b - a;
    int c = p.context_lens ? p.context_lens[seq] : 0;
    c = max(0, min(c, p.block_tables ? (p.max_blocks << p.block_shift) : 0));
    s.c = c;
    s.q0 = c;
    s.empty = false;
    return s;
}

// Key and value rows j of a sequence: cached (through the block table) or new.
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

// Grid of the MFMA kernel.  Workgroups that read the same K/V -- the G query heads of one KV head
// and `qtiles_per_group` neighbouring query tiles of one sequence -- form a group.  Workgroups
// are dealt to the 8 XCDs round-robin by index, so the index is built as
// ((group / 8) * group_size + member) * 8 + group % 8: the members of a group run back to back on
// one XCD and share its L2, and each XCD takes every 8th group in heavy-first order (late query
// tiles see the most keys).  Groups are enumerated by query-tile level (latest first), then
// sequence, then KV head.  In compact mode (up to 64 sequences and 64 query-tile levels, one query
// tile per group) a level lists only the sequences long enough to have that tile, so no workgroup
// of the grid stands for a tile past a sequence's end; the grid is sized from num_tokens (at most
// num_tokens / rows + num_seqs tiles per KV head), and workgroups past the last group exit at once.
struct PrefillGrid {
    int heads;             // query heads per workgroup (hp = 4, 2 or 1; divides G)
    int rows;              // query rows per workgroup (128 / hp)
    int num_qtiles;        // ceil(max_subquery_len / rows)
    int qtiles_per_group;  // query tiles in a group
    int num_qblocks;       // ceil(num_qtiles / qtiles_per_group)
    int group_size;        // (G / hp) * qtiles_per_group workgroups
    int num_groups;        // num_qblocks * num_seqs * num_kv_heads, or its bound in compact mode
    int compact;           // 1: only groups of existing query tiles are enumerated (qtiles_per_group 1)
};

// V tile swizzle of row r: spreads the 8 rows read together by 32 lanes of the transposing load
// (4 rows at 8 bytes per lane in each 16-lane group) over distinct 32-byte units of a 256-byte
// bank window.
template <int D>
__device__ __forceinline__ int vswz(int r) {
    return D >= 128 ? (r & 7) : ((r >> 1) & 3);
}

// Tile staging.  K and V tiles (64 keys x D) are copied global -> LDS by the load-to-LDS path
// (buffer/global_load_lds_dwordx4: lane l of an instruction fills 16-byte unit l of a 1 KB LDS
// stretch), so they never pass through registers.  Swizzles are applied by choosing, per lane,
// which 16-byte chunk of the source row to fetch:
//   K: row-major [64][D], chunk c of row r stored at chunk c ^ ((r mod 16) mod CH); the S^T operand read
//      (16 rows, same chunk) then hits distinct banks.
//   V: row-major [64][D], 32-byte unit u of key k stored at unit u ^ vswz(k); the transposing
//      operand read (ds_read_b64_tr_b16: 4 keys x 32 bytes per 16 lanes, 8 keys per 32 lanes)
//      then hits distinct banks.
// Each wavefront copies 16 keys (rows 16 w .. 16 w + 15) of each tile, which lie in one cache
// block (two for 8-token blocks), so one descriptor per block and tile serves all its copies.
//
// Scores.  A wavefront's 32 rows meet a tile in two 32-key halves.  The score MFMAs take Q as it
// is stored, and one fp32 FMA per score turns their result into the exponent of its weight:
// scale log2(e) times the product plus c_row - m + b_key, where c_row is the row's ALiBi term for
// the half's first key (0 without ALiBi), m the finite stand-in of the row's running max and b_key
// the key's ALiBi offset from the half's first key times slope log2(e) (a per-lane constant, which
// enters through the accumulators' start values or the FMA's addend).  A half is
//   * empty for the wavefront when every (row, key) pair is masked -- skipped entirely;
//   * full when none is -- no per-score work besides the max and the exponent;
//   * partial otherwise -- masked scores are set to -inf.
//
// With a logits soft-cap c (SOFTCAP) the raw dot product must reach tanh, so Q keeps its values
// (a negative scale folded into a sign flip of Q, exact in both 16-bit formats; a zero scale into
// Q = 0); the raw scores become c log2(e) tanh(s |scale| / c) right after the score MFMAs, the
// ALiBi key term is added to them in fp32 (it must stay outside the cap), and the exponent
// subtracts the running max.  Sink logits (p.sinks) join the row sums in the epilogue.

// Head size 256 doubles the O accumulators and the operands per wavefront and the LDS stages
// (128 KB): one workgroup per CU then, with the register file of a single wavefront per SIMD.
template <typename T, int D, bool ALIBI, bool SOFTCAP>
__global__ __launch_bounds__(kThreads, D > 128 ? 1 : 2) void prefill_mfma_kernel(PrefillParams p, PrefillGrid grid) {
    typedef typename Operand8<T>::type V8;
    auto elt_bits = [](T x) -> uint32_t { return uint32_t(__builtin_bit_cast(uint16_t, x)); };
    constexpr int CH = D / 8;        // 16-byte chunks per row
    constexpr int DC = D / 32;       // k-chunks of S^T
    constexpr int DB = D / 16;       // d-blocks of O^T
    constexpr int RPI = 64 / CH;     // tile rows per copy instruction (4 or 8)
    constexpr int NJ = 16 / RPI;     // copy instructions per wavefront per operand per tile
    constexpr int ROWB = D * 2;      // bytes per tile row
    __shared__ __align__(16) bf16_t Ks0[kBN * D];
    __shared__ __align__(16) bf16_t Vs0[kBN * D];
    __shared__ __align__(16) bf16_t Ks1[kBN * D];
    __shared__ __align__(16) bf16_t Vs1[kBN * D];

    // ---- workgroup -> (sequence, KV head, query head, query tile)
    const int b = blockIdx.x;
    const int xcd = b & 7;
    const int qq = b >> 3;
    const int member = qq % grid.group_size;
    const int k = (qq / grid.group_size) * 8 + xcd;
    if (k >= grid.num_groups) return;
    const int group = p.num_heads / p.num_kv_heads;
    int qb, seq, g;
    SeqInfo si;
    if (grid.compact) {
        // lane i < num_seqs holds sequence i's bounds (loaded once: the workgroup's sequence is then
        // read out of its lane, with no second round trip) and query tiles; level l holds the
        // sequences with more than l query tiles
        const int lane_id = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0));
        SeqInfo ls{0, 0, 0, 0, false};
        if (lane_id < p.num_seqs) ls = seq_info(p, lane_id);
        const int nq = (ls.n + grid.rows - 1) / grid.rows;
        int rem = k, lvl = grid.num_qtiles - 1;
        uint64_t m = 0;
        for (; lvl >= 0; --lvl) {
            m = __builtin_amdgcn_ballot_w64(nq > lvl);
            const int cnt = __builtin_popcountll(m) * p.num_kv_heads;
            if (rem < cnt) break;
            rem -= cnt;
        }
        if (lvl < 0) return;
        // the (rem / Hkv)-th sequence of the level: the lane whose bit is set with that many set bits below it
        const int r = rem / p.num_kv_heads;
        const int below = __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0));
        const uint64_t hit = __builtin_amdgcn_ballot_w64(((m >> lane_id) & 1) && below == r);
        seq = __builtin_ctzll(hit);
        g = rem % p.num_kv_heads;
        qb = lvl;
        si.start = __builtin_amdgcn_readlane(ls.start, seq);
        si.n = __builtin_amdgcn_readlane(ls.n, seq);
        si.c = __builtin_amdgcn_readlane(ls.c, seq);
        si.q0 = __builtin_amdgcn_readlane(ls.q0, seq);
        si.empty = __builtin_amdgcn_readlane(int(ls.empty), seq) != 0;
    } else {
        const int per_qb = p.num_seqs * p.num_kv_heads;
        qb = grid.num_qblocks - 1 - k / per_qb;
        seq = (k % per_qb) / p.num_kv_heads;
        g = k % p.num_kv_heads;
        si = seq_info(p, seq);
    }
    const int hblocks = group / grid.heads;
    const int qt = qb * grid.qtiles_per_group + member / hblocks;
    if (qt >= grid.num_qtiles || qt * grid.rows >= si.n) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15;
    const int lg = lane >> 4;
    // wavefront -> (head, 32-row strip): with hp heads per workgroup the wavefronts share strips,
    // so for hp = 4 all four see the same diagonal and reach every tile with equal work
    const int h = g * group + (member % hblocks) * grid.heads + wave % grid.heads;
    const int t0 = qt * grid.rows + (wave / grid.heads) * 32;   // first subquery row of this wavefront
    const int p0 = si.q0 + t0;                                 // its position
    if (si.empty) {
        // uniform mode, a padded sequence: zero rows (uniform over the workgroup, before any barrier)
#pragma unroll
        for (int qbk = 0; qbk < 2; ++qbk) {
            const int trow = t0 + 16 * qbk + l16;
            if (trow < si.n) {
                bf16_t *orow = reinterpret_cast<bf16_t *>(p.out) + int64_t(si.start + trow) * p.num_heads * D +
                               int64_t(h) * D + 4 * lg;
#pragma unroll
                for (int db = 0; db < D / 16; ++db) *reinterpret_cast<uint2 *>(orow + 16 * db) = make_uint2(0u, 0u);
            }
        }
        return;
    }

    const float qk_scale = p.scale * kLog2e;
    // Without a soft-cap (PRE) the score MFMAs take Q as it is and one fp32 FMA per score turns the
    // result into the base-2 logit relative to the running max: s = m (dot + b_key / m) + (c_row -
    // m_fin), with m = scale log2(e), b_key the key's ALiBi offset from the half's first key times
    // slope log2(e) (b_key / m, a per-lane constant, is where the accumulators start), c_row the
    // row's ALiBi term and m_fin the finite stand-in of the running max (both per row).  An FP8
    // cache has two multipliers (cached keys carry k_scale); there the accumulators start at zero
    // and b_key joins the FMA's addend instead, which keeps one set of per-lane constants.
    // (Pre-scaling Q in the element type instead saves the FMA but rounds scale * q to 8 bits, which
    // doubled the bf16 error at 2.5 times the default scale.)  With start values a zero scale
    // zeroes Q and takes m = 1.  With a soft-cap the raw dot product must reach tanh, so Q keeps
    // its values there too (a negative scale as a sign flip, exact; a zero scale as Q = 0).
    constexpr bool PRE = !SOFTCAP;
    constexpr bool C8 = kFp8Cache<T>;
    constexpr bool KB_INIT = PRE && ALIBI && !C8;         // ALiBi start values in the accumulators
    const uint32_t qxor = !PRE && qk_scale < 0.f ? 0x80008000u : 0u;      // sign flips of both halves
    const uint32_t qand = (!PRE || KB_INIT) && qk_scale == 0.f ? 0u : 0xffffffffu;
    // The ALiBi key term (the key's offset from the half's first key times slope log2(e)) joins the
    // accumulators' start values or the FMA's addend; with a soft-cap it must stay outside the cap,
    // so there it is added after the cap (the capped scores are base-2 logits already).
    const float cap_in = SOFTCAP ? fabsf(p.scale) / p.softcap : 0.f;
    const float cap2 = SOFTCAP ? p.softcap * kLog2e : 0.f;

    // FP8 cache: cached K rows sit in the tile as exact code values (k_scale not applied); the
    // score FMA (or the soft-cap's input scale) of a cached key multiplies by k_scale as well.
    const float qk_scale_c = C8 ? qk_scale * p.k_scale : qk_scale;     // cached keys
    // FP8 cache (EXACT_V): cached V rows sit in the tile as exact code values too; a cached key's
    // weight carries v_scale instead (log2 v_scale joins its exponent, so the weight is rounded
    // once, as any weight is) and its row-sum share, kept apart, is divided by v_scale at the end.
    // At head size 256 with both ALiBi and a soft-cap, V rows are staged as code * v_scale rounded
    // to the element type: there this form came out of the compiler wrong (its outputs differed
    // from the identical arithmetic of the rounded form even with no cached key).
    constexpr bool EXACT_V = C8 && (D <= 128 || !(ALIBI && SOFTCAP));
    const float lvs = EXACT_V ? __log2f(p.v_scale) : 0.f;
    // PRE multipliers of new and cached keys (with start values and a zero scale, 1: Q is zero)
    const float mul_n = KB_INIT && qk_scale == 0.f ? 1.f : qk_scale;
    const float mul_c = qk_scale_c;

    // Q as the B operand of S^T = K Q^T: lane holds row (t0 + 16 qbk + l16), d = 32 dc + 8 lg .. +7.
    V8 qf[2][DC];
#pragma unroll
    for (int qbk = 0; qbk < 2; ++qbk) {
        const int trow = min(t0 + 16 * qbk + l16, si.n - 1);
        const bf16_t *qrow = reinterpret_cast<const bf16_t *>(p.query) + int64_t(si.start + trow) * p.q_stride +
                             int64_t(h) * D + 8 * lg;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
            uint4 w = *reinterpret_cast<const uint4 *>(qrow + 32 * dc);
            {
                w.x = (w.x ^ qxor) & qand;
                w.y = (w.y ^ qxor) & qand;
                w.z = (w.z ^ qxor) & qand;
                w.w = (w.w ^ qxor) & qand;
            }
            qf[qbk][dc] = __builtin_bit_cast(V8, w);
        }
    }

    const int row_hi = min(qt * grid.rows + grid.rows, si.n) - 1;
    const int pos_lo = si.q0 + qt * grid.rows;
    const int key_hi = si.q0 + row_hi;
    const int key_lo = p.window > 0 ? max(0, pos_lo - p.window + 1) : 0;
    const int kt_lo = key_lo / kBN, kt_hi = key_hi / kBN;

    // ALiBi: slope in base-2 units; kbias[kk][i] is the key term of accumulator slot (kk, i), the key
    // k0h + 16 kk + 4 lg + i, relative to the half's first key k0h.
    float slope2 = 0.f;
    if constexpr (ALIBI) slope2 = p.alibi_slopes[h] * kLog2e;
    float kbias[2][4] = {};
    if constexpr (ALIBI) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int i = 0; i < 4; ++i) kbias[kk][i] = slope2 * float(16 * kk + 4 * lg + i);
    }
    // PRE with ALiBi over a 16-bit cache: the score accumulators' starting values b_key / m
    floatx4_v kb_n[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        kb_n[kk] = floatx4_v{0.f, 0.f, 0.f, 0.f};
        if constexpr (KB_INIT) {
#pragma unroll
            for (int i = 0; i < 4; ++i) kb_n[kk][i] = kbias[kk][i] / mul_n;
        }
    }

    // ---- copies
    const char *kc_bytes = reinterpret_cast<const char *>(p.k_cache);
    const char *vc_bytes = reinterpret_cast<const char *>(p.v_cache);
    const char *kn_bytes = reinterpret_cast<const char *>(p.key);
    const char *vn_bytes = reinterpret_cast<const char *>(p.value);
    const int64_t head_off = int64_t(g) * ROWB;
    const int64_t cache_row_bytes = int64_t(p.num_kv_heads) * ROWB;
    const int64_t new_row_bytes = int64_t(p.kv_stride) * 2;
    const int64_t block_bytes = cache_row_bytes << p.block_shift;
    const int bmask = (1 << p.block_shift) - 1;
    const int wrow0 = 16 * wave;                            // first tile row this wavefront copies
    // Lane terms of the copy addresses: the lane's row among its instruction's rows and the
    // logical chunk its physical LDS unit holds (the residues of the row mod CH and mod 4 depend
    // only on j and the lane).  They come from the lane id (an asm read, so the compiler neither
    // hoists nor merges them on its own); where they are held across the loop is decided below.
    auto lane_terms = [&](int &lrow, int &pc) __attribute__((always_inline)) {
        int l;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
        lrow = l / CH;
        pc = l % CH;
    };
    auto k_chunk = [&](int lrow, int pc, int j) __attribute__((always_inline)) -> uint32_t {
        return uint32_t(pc ^ ((j * RPI + lrow) % CH)) * 16;
    };
    // V swizzle: the 32-byte unit u of tile row r sits at unit u ^ vswz(r); vswz depends on r only
    // through r mod 8 (D = 128) or r mod 8 / 2 (D = 64), so rows 16 w + j RPI + lrow and
    // j RPI + lrow share it.
    auto v_chunk = [&](int lrow, int pc, int j) __attribute__((always_inline)) -> uint32_t {
        return uint32_t((((pc >> 1) ^ vswz<D>(j * RPI + lrow)) * 2 + (pc & 1)) * 16);
    };
    // Up to head size 128 the lane offsets of the two fast copy paths (whole cached or whole new
    // runs of rows) are computed once and held in registers: 4 NJ values, against ~40 ALU ops per
    // tile to rebuild them.  At head size 256 the registers are needed elsewhere.
    constexpr bool HOLD = D <= 128;
    constexpr int NH = HOLD ? NJ : 1;
    uint32_t koc[NH], voc[NH], kon[NH], von[NH];
    if constexpr (HOLD) {
        int lrow, pc;
        lane_terms(lrow, pc);
        const uint32_t lc = uint32_t(lrow) * uint32_t(cache_row_bytes);
        const uint32_t ln = uint32_t(lrow) * uint32_t(new_row_bytes);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            koc[j] = lc + k_chunk(lrow, pc, j);
            voc[j] = lc + v_chunk(lrow, pc, j);
            kon[j] = ln + k_chunk(lrow, pc, j);
            von[j] = ln + v_chunk(lrow, pc, j);
        }
    }
    auto clamp_block = [&](int64_t bl) __attribute__((always_inline)) -> int64_t {
        return bl < 0 ? 0 : (bl >= p.num_blocks ? p.num_blocks - 1 : bl);
    };
    // Block ids of this wavefront's 16 rows of tile kt: lane 0 gets the first row's block, lane 1
    // the last (cached) row's.  A vector load, so the wait at the end of the tile covers it.
    auto fetch_ids = [&](int kt) __attribute__((always_inline)) -> int {
        const int r0 = kt * kBN + wrow0;
        int id = 0;
        if (r0 < si.c) {
            const int r = (lane & 1) ? min(r0 + 15, si.c - 1) : r0;
            id = p.block_tables[int64_t(seq) * p.max_blocks + (r >> p.block_shift)];
        }
        return id;
    };
    // ---- FP8 cache (element types with kFp8Cache): cached rows cannot go through the load-to-LDS
    // path, which copies bytes unchanged.  Each lane instead loads 16 codes of a row (one 16-byte
    // load per slot, slot s = lane + 64 j: tile row 16 w + s / (D / 16), codes 16 (s % (D / 16)) ..
    // + 15) for K and for V when the tile's copies are issued, and a tile later, when they have
    // long arrived, turns them into 16-bit values (the codes exactly; V without EXACT_V as
    // code * v_scale) and writes them into the same swizzled places the copies would have filled.
    // New-token rows still use the copies.
    // Rows past key_hi (the last key any row of the workgroup sees) stand in for the row key_hi in
    // the copies; when that row is cached (always so in the uniform multi-token mode, where every
    // key is cached) no copy fills them, so their codes are zeros here: masked keys then meet
    // zero V rows, never unwritten LDS.
    constexpr int NS8 = C8 ? D / 64 : 1;    // slots per lane per operand and tile
    constexpr int SPR8 = D / 16;            // slots per row
    uint4 raw8[2][NS8];
    uint32_t raw8_mask = 0;                 // bit j: slot j holds codes to write
    const int64_t row8 = int64_t(p.num_kv_heads) * D;          // bytes per cached token (all heads)
    const int64_t block8 = row8 << p.block_shift;
    auto fp8_issue = [&](int kt, int id0, int id1) __attribute__((always_inline)) {
        const int w0 = kt * kBN + wrow0;
        raw8_mask = 0;
#pragma unroll
        for (int j = 0; j < NS8; ++j) {
            const int sl = lane + 64 * j, r = sl / SPR8, m = sl % SPR8;
            const int key = w0 + r;
            if (key > key_hi) {
                if (key_hi < si.c) {
                    raw8[0][j] = make_uint4(0u, 0u, 0u, 0u);
                    raw8[1][j] = make_uint4(0u, 0u, 0u, 0u);
                    raw8_mask |= 1u << j;
                }
            } else if (key < si.c) {
                const int64_t blk = clamp_block(((key >> p.block_shift) == (w0 >> p.block_shift)) ? id0 : id1);
                const int64_t off = blk * block8 + int64_t(key & bmask) * row8 + int64_t(g) * D + 16 * m;
                raw8[0][j] = *reinterpret_cast<const uint4 *>(kc_bytes + off);
                raw8[1][j] = *reinterpret_cast<const uint4 *>(vc_bytes + off);
                raw8_mask |= 1u << j;
            }
        }
    };
    auto fp8_commit = [&](bf16_t *kdst, bf16_t *vdst) __attribute__((always_inline)) {
        if constexpr (C8) {
#pragma unroll
            for (int j = 0; j < NS8; ++j) {
                if ((raw8_mask >> j) & 1u) {
                    const int sl = lane + 64 * j, r = sl / SPR8, m = sl % SPR8;
                    const int rr = wrow0 + r;
#pragma unroll
                    for (int o = 0; o < 2; ++o) {
                        // K codes exactly (every E4M3 value is a 16-bit value); V likewise, or
                        // (without EXACT_V) as code * v_scale rounded to the element type
                        uint32_t w[8];
                        if constexpr (EXACT_V) {
                            const uint4 w0 = widen_e4m3<T>(make_uint2(raw8[o][j].x, raw8[o][j].y));
                            const uint4 w1 = widen_e4m3<T>(make_uint2(raw8[o][j].z, raw8[o][j].w));
                            w[0] = w0.x; w[1] = w0.y; w[2] = w0.z; w[3] = w0.w;
                            w[4] = w1.x; w[5] = w1.y; w[6] = w1.z; w[7] = w1.w;
                        } else {
                            const float sc = o ? p.v_scale : 1.f;
                            const uint32_t cw[4] = {raw8[o][j].x, raw8[o][j].y, raw8[o][j].z, raw8[o][j].w};
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(cw[q]), false);
                                const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(cw[q]), true);
                                w[2 * q] = pack_x2<T>(lo[0] * sc, lo[1] * sc);
                                w[2 * q + 1] = pack_x2<T>(hi[0] * sc, hi[1] * sc);
                            }
                        }
                        int off0, off1;
                        if (o == 0) {
                            // K: 16-byte chunk c of row rr at c ^ ((rr mod 16) mod CH), the swizzle the
                            // copies and the operand reads use (they see rows 16 w .. 16 w + 15)
                            const int sw = (rr & 15) % CH;
                            off0 = rr * D + (((2 * m) ^ sw) << 3);
                            off1 = rr * D + (((2 * m + 1) ^ sw) << 3);
                        } else {                            // V: 32-byte unit u of row rr at u ^ vswz(rr)
                            off0 = rr * D + ((m ^ vswz<D>(rr)) << 4);
                            off1 = off0 + 8;
                        }
                        bf16_t *dst = o ? vdst : kdst;
                        *reinterpret_cast<uint4 *>(dst + off0) = make_uint4(w[0], w[1], w[2], w[3]);
                        *reinterpret_cast<uint4 *>(dst + off1) = make_uint4(w[4], w[5], w[6], w[7]);
                    }
                }
            }
            raw8_mask = 0;
        }
    };

    // Copy this wavefront's 16 rows of tile kt into (kdst, vdst); id0 / id1 are the blocks of its
    // first and last cached row (wave-uniform).  The rows are all cached, all new and at or below
    // key_hi (one descriptor per block, scalar offsets per instruction), or -- at most twice per
    // sequence -- mixed, which takes a per-lane path.  Rows past key_hi re-read row key_hi; every
    // query row masks them.
    auto copy_tile = [&](int kt, int id0_raw, int id1_raw, bf16_t *kdst, bf16_t *vdst) __attribute__((always_inline)) {
        const int w0 = kt * kBN + wrow0;                  // first key of this wavefront (uniform)
        if constexpr (C8) {
            if (w0 < si.c || key_hi < si.c) fp8_issue(kt, id0_raw, id1_raw);
            if (w0 + 15 < si.c) return;                   // all cached: nothing for the copies
        }
        if (!C8 && w0 + 15 < si.c) {
            const int64_t off0 = clamp_block(id0_raw) * block_bytes + head_off + int64_t(w0 & bmask) * cache_row_bytes;
            const int64_t off1 = clamp_block(id1_raw) * block_bytes + head_off;
            int lrow = 0, pc = 0;
            if constexpr (!HOLD) lane_terms(lrow, pc);
            const uint32_t lro = uint32_t(lrow) * uint32_t(cache_row_bytes);
            const bool one_block = (1 << p.block_shift) >= 16;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const bool second = !one_block && j >= NJ / 2;
                const int64_t off = second ? off1 : off0;
                const uint32_t soff = uint32_t((second ? j - NJ / 2 : j) * RPI) * uint32_t(cache_row_bytes);
                const uint32_t kl = HOLD ? koc[j % NH] : lro + k_chunk(lrow, pc, j);
                const uint32_t vl = HOLD ? voc[j % NH] : lro + v_chunk(lrow, pc, j);
                dma16(kc_bytes + off, kl, soff, kdst + (NJ * wave + j) * 512);
                dma16(vc_bytes + off, vl, soff, vdst + (NJ * wave + j) * 512);
            }
        } else if (w0 >= si.c && w0 + 15 <= key_hi) {
            const int64_t off = int64_t(si.start + (w0 - si.c)) * new_row_bytes + head_off;
            int lrow = 0, pc = 0;
            if constexpr (!HOLD) lane_terms(lrow, pc);
            const uint32_t lro = uint32_t(lrow) * uint32_t(new_row_bytes);
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const uint32_t soff = uint32_t(j * RPI) * uint32_t(new_row_bytes);
                const uint32_t kl = HOLD ? kon[j % NH] : lro + k_chunk(lrow, pc, j);
                const uint32_t vl = HOLD ? von[j % NH] : lro + v_chunk(lrow, pc, j);
                dma16(kn_bytes + off, kl, soff, kdst + (NJ * wave + j) * 512);
                dma16(vn_bytes + off, vl, soff, vdst + (NJ * wave + j) * 512);
            }
        } else {
            int lrow, pc;
            lane_terms(lrow, pc);
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int kk = min(w0 + j * RPI + lrow, key_hi);
                const bool cached = kk < si.c;
                // the table is read only for cached rows: without a context it may be null
                int64_t bl = 0;
                if (cached) bl = clamp_block(p.block_tables[int64_t(seq) * p.max_blocks + (kk >> p.block_shift)]);
                const int64_t off = cached ? bl * block_bytes + int64_t(kk & bmask) * cache_row_bytes + head_off
                                           : int64_t(si.start + (kk - si.c)) * new_row_bytes + head_off;
                bf16_t *kd = kdst + (NJ * wave + j) * 512;
                bf16_t *vd = vdst + (NJ * wave + j) * 512;
                // (a branch rather than a select of the two bases keeps the bases in scalar registers)
                if (C8 && cached) {
                    // an FP8 cache row: written by fp8_commit
                } else if (cached) {
                    dma16_lane(kc_bytes + off + k_chunk(lrow, pc, j), kd);
                    dma16_lane(vc_bytes + off + v_chunk(lrow, pc, j), vd);
                } else {
                    dma16_lane(kn_bytes + off + k_chunk(lrow, pc, j), kd);
                    dma16_lane(vn_bytes + off + v_chunk(lrow, pc, j), vd);
                }
            }
        }
    };

    // ---- deferred copies.  The copies of the two fast paths (a wavefront's 16 rows all cached, or
    // all new and at or below key_hi) are planned before the tile that streams them starts --
    // scalar arithmetic only: a 32-bit block clamp and one 64-bit base per block, the value plane
    // lying a constant distance from the key plane -- and issued one (K, V) pair after each group
    // of score MFMAs of that tile's first half, so the matrix unit stays fed while they go out.
    // Other tiles (mixed rows, an FP8 cache's cached rows) are copied by copy_tile up front.
    const int nbm1 = int(p.num_blocks - 1);             // block ids fit int32 (checked on the host)
    const uint32_t crow32 = uint32_t(cache_row_bytes), nrow32 = uint32_t(new_row_bytes);
    const uint32_t blk32 = uint32_t(block_bytes);
    const char *kc_head = kc_bytes + head_off;
    const char *kn_head = kn_bytes + head_off;
    const int64_t vc_diff = vc_bytes - kc_bytes;
    const int64_t vn_diff = vn_bytes - kn_bytes;
    const bool one_block = (1 << p.block_shift) >= 16;
    struct CopyPlan {
        const char *b0;      // key bytes of this wavefront's first row (its block for cached rows)
        const char *b1;      // cached rows in a second block (block size 8): that block's key row 0
        int mode;            // 0: nothing deferred, 1: cached rows, 2: new rows
    };
    auto plan_copy = [&](int kt, int id0_raw, int id1_raw) __attribute__((always_inline)) -> CopyPlan {
        CopyPlan cp{nullptr, nullptr, 0};
        const int w0 = kt * kBN + wrow0;
        if (!C8 && w0 + 15 < si.c) {
            const int b0 = min(max(id0_raw, 0), nbm1), b1 = min(max(id1_raw, 0), nbm1);
            cp.b0 = kc_head + int64_t(uint32_t(b0)) * blk32 + uint32_t(w0 & bmask) * crow32;
            cp.b1 = kc_head + int64_t(uint32_t(b1)) * blk32;
            cp.mode = 1;
        } else if (w0 >= si.c && w0 + 15 <= key_hi) {
            cp.b0 = kn_head + int64_t(si.start + (w0 - si.c)) * nrow32;
            cp.mode = 2;
        }
        return cp;
    };
    // Copy instruction pair j (tile rows 16 w + j RPI ..) of a planned tile into the LDS stretches
    // at byte addresses kb + 1 KB j and vb + 1 KB j; soff is the pair's row offset in bytes.
    // MODE is the plan's mode (1 or 2).
    auto issue_pair = [&](const CopyPlan &cp, auto mode_c, int j, uint32_t kb, uint32_t vb, uint32_t soff)
                          __attribute__((always_inline)) {
        constexpr int MODE = decltype(mode_c)::value;
        int lrow = 0, pc = 0;
        if constexpr (!HOLD) lane_terms(lrow, pc);
        if constexpr (MODE == 1) {
            const bool second = !one_block && j >= NJ / 2;
            const char *base = second ? cp.b1 : cp.b0;
            const uint32_t lro = uint32_t(lrow) * crow32;
            const uint32_t kl = HOLD ? koc[j % NH] : lro + k_chunk(lrow, pc, j);
            const uint32_t vl = HOLD ? voc[j % NH] : lro + v_chunk(lrow, pc, j);
            dma16_at(base, kl, soff, kb + 1024u * j);
            dma16_at(base + vc_diff, vl, soff, vb + 1024u * j);
        } else {
            const uint32_t lro = uint32_t(lrow) * nrow32;
            const uint32_t kl = HOLD ? kon[j % NH] : lro + k_chunk(lrow, pc, j);
            const uint32_t vl = HOLD ? von[j % NH] : lro + v_chunk(lrow, pc, j);
            dma16_at(cp.b0, kl, soff, kb + 1024u * j);
            dma16_at(cp.b0 + vn_diff, vl, soff, vb + 1024u * j);
        }
    };
    // All copies of a planned tile (one branch on the mode per tile).  The tile's LDS bases and the
    // row step pass through empty asm statements, so the compiler forms each copy's LDS address and
    // row offset with one scalar add instead of holding every one of them in a register across the
    // loop.
    auto issue_all = [&](const CopyPlan &cp, bf16_t *kdst, bf16_t *vdst) __attribute__((always_inline)) {
        uint32_t kb = lds_address(kdst) + 1024u * NJ * wave, vb = lds_address(vdst) + 1024u * NJ * wave;
        asm volatile("" : "+s"(kb), "+s"(vb));
        if (cp.mode == 1) {
            uint32_t step = RPI * crow32;
            asm volatile("" : "+s"(step));
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const uint32_t soff = (!one_block && j >= NJ / 2 ? j - NJ / 2 : j) * step;
                issue_pair(cp, std::integral_constant<int, 1>(), j, kb, vb, soff);
            }
        } else if (cp.mode == 2) {
            uint32_t step = RPI * nrow32;
            asm volatile("" : "+s"(step));
#pragma unroll
            for (int j = 0; j < NJ; ++j) issue_pair(cp, std::integral_constant<int, 2>(), j, kb, vb, j * step);
        }
    };

    // ---- operand read offsets (elements), fixed for the whole loop.  The K swizzle of row 16 kb +
    // l16 is l16 mod CH (the copies use the row's offset inside its wavefront's 16 rows, the same
    // value), so it depends on the lane only and kb adds a constant.
    int k_off[DC];
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) k_off[dc] = l16 * D + (((4 * dc + lg) ^ (l16 % CH)) << 3);
    // V^T operand for (d-block db, key chunk kc, half hh): lane l16 = 4 a + c of group lg reads,
    // through the transposing load, key 32 kc + 16 hh + 4 lg + a at d = 16 db + 4 c.  32 kc + 16 hh
    // does not change vswz of that key, so its unit db sits at db ^ vswz(4 lg + a): one lane offset
    // per d-block, and kc and hh add constants.
    const int va = l16 >> 2;
    int v_off[DB];
#pragma unroll
    for (int u = 0; u < DB; ++u) v_off[u] = (4 * lg + va) * D + ((u ^ vswz<D>(4 * lg + va)) << 4) + 4 * (l16 & 3);

    float m_run[2] = {-INFINITY, -INFINITY};   // row max (base 2), uniform over the row's 4 lanes
    // kept beside it, changed only when it is raised: the raise threshold m_run + kRescaleSlack and
    // the exponent's finite stand-in for m_run (0 while no visible key has been seen)
    float m_thr[2] = {-INFINITY, -INFINITY};
    float m_fin[2] = {0.f, 0.f};
    floatx4_v o[2][DB];
    // Row sums of the rounded weights, accumulated by the MFMA unit: an all-ones block times P^T
    // gives sum_k P[q][k] in every element of lane (q, .).
    floatx4_v lsum[2], lsum_c[2];        // lsum_c (EXACT_V): cached keys (weights times v_scale)
#pragma unroll
    for (int qbk = 0; qbk < 2; ++qbk) {
        lsum[qbk] = floatx4_v{0.f, 0.f, 0.f, 0.f};
        lsum_c[qbk] = floatx4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < DB; ++db) o[qbk][db] = floatx4_v{0.f, 0.f, 0.f, 0.f};
    }
    const uint32_t one2 = elt_bits(to_elt<T>(1.f)) * 0x10001u;
    const V8 ones = __builtin_bit_cast(V8, make_uint4(one2, one2, one2, one2));

    // One 32-key half (keys k0h .. k0h + 31, key chunk kc of the tile in (ks, vs)).
    // LDS operand reads are issued one phase ahead of their MFMAs: the K operands of a half are
    // read while the previous half finishes (or right after the tile barrier for the first half
    // of a tile), the V operands right after the half's S^T MFMAs, before its softmax.
    V8 ka[DC][2];                // K operands of the coming half
    V8 vop[DB];                  // V^T operands of the current half
    auto load_k = [&](const bf16_t *ks, int kc) __attribute__((always_inline)) {
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                ka[dc][kk] = *reinterpret_cast<const V8 *>(ks + k_off[dc] + 16 * (2 * kc + kk) * D);
    };
    auto load_v = [&](const bf16_t *vs, int kc) __attribute__((always_inline)) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const bf16_t *vb = vs + v_off[db] + 32 * kc * D;
            const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)vb);
            const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vb + 16 * D));
            const v4i16 both[2] = {lo, hi};
            vop[db] = __builtin_bit_cast(V8, both);
        }
    };

    // One 32-key half (keys k0h .. k0h + 31, key chunk kc of the tile in (ks, vs)); ka holds its
    // K operands on entry.  next_kc >= 0: the next half is chunk next_kc of the same tile, whose
    // K operands are read into ka here.
    auto half = [&](int k0h, int kc, const bf16_t *ks, const bf16_t *vs, int next_kc) __attribute__((always_inline)) {
        // wavefront rows are positions p0 .. p0 + 31; a key is visible from pos iff
        // pos - W < key <= pos
        const bool empty = k0h > p0 + 31 || (p.window > 0 && k0h + 31 <= p0 - p.window);
        if (empty) {
            if (next_kc >= 0) load_k(ks, next_kc);
            return;
        }
        const bool full = k0h + 31 <= p0 && (p.window <= 0 || k0h > p0 + 31 - p.window);
        // FP8 cache (EXACT_V): the half's keys are all cached (c_half), all new (n_half) or both
        bool c_half = false, n_half = true;
        if constexpr (EXACT_V) {
            c_half = k0h + 31 < si.c;
            n_half = k0h >= si.c;
        }

        // ---- S^T = K Q^T (+ ALiBi term): s[kk][qbk] holds keys k0h + 16 kk + 4 lg + i of row 16 qbk + l16
        // crow: the ALiBi term of the half's first key for the row (base 2), a per-row constant
        float crow[2];
#pragma unroll
        for (int qbk = 0; qbk < 2; ++qbk) crow[qbk] = ALIBI ? slope2 * float(k0h - (p0 + 16 * qbk + l16)) : 0.f;
        floatx4_v s[2][2];
#pragma unroll
        for (int qbk = 0; qbk < 2; ++qbk)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) s[kk][qbk] = kb_n[kk];
        // Raised wave priority while the score MFMAs issue: when both wavefronts of a SIMD want the
        // matrix unit, this one goes first and the other turns to its exponentials, so the two
        // drift into alternating phases instead of colliding.
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int qbk = 0; qbk < 2; ++qbk)
                    s[kk][qbk] = mfma16(ka[dc][kk], qf[qbk][dc], s[kk][qbk]);
        }
        __builtin_amdgcn_s_setprio(0);
        load_v(vs, kc);
        if constexpr (PRE) {
            // s = m (dot + b_key / m) + (c_row - m_fin): the base-2 logit relative to the running
            // max's finite stand-in (FP8 cache: s = m dot + (c_row - m_fin + b_key), m times
            // k_scale, and with EXACT_V log2 v_scale added, for a cached key).  The multiplier is
            // uniform over the half unless an FP8 half holds both cached and new keys.
            if constexpr (EXACT_V) {
                const bool mixed = !c_half && !n_half;
                if (!mixed) {
                    const float mul = c_half ? mul_c : mul_n;
                    float a0[2];
#pragma unroll
                    for (int qbk = 0; qbk < 2; ++qbk)
                        a0[qbk] = c_half ? crow[qbk] - m_fin[qbk] + lvs : crow[qbk] - m_fin[qbk];
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int qbk = 0; qbk < 2; ++qbk)
                                s[kk][qbk][i] = fmaf(s[kk][qbk][i], mul, ALIBI ? a0[qbk] + kbias[kk][i] : a0[qbk]);
                } else {
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const bool cached = k0h + 16 * kk + 4 * lg + i < si.c;
                            const float mk = cached ? mul_c : mul_n;
                            const float lk = cached ? lvs : 0.f;
#pragma unroll
                            for (int qbk = 0; qbk < 2; ++qbk)
                                s[kk][qbk][i] = fmaf(s[kk][qbk][i], mk,
                                                     ALIBI ? crow[qbk] - m_fin[qbk] + kbias[kk][i] + lk
                                                           : crow[qbk] - m_fin[qbk] + lk);
                        }
                }
            } else {
                float mul = mul_n;
                bool mixed = false;
                if constexpr (C8) {
                    if (k0h + 31 < si.c) mul = mul_c;
                    else mixed = k0h < si.c;
                }
                if (!mixed) {
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int qbk = 0; qbk < 2; ++qbk)
                                s[kk][qbk][i] = fmaf(s[kk][qbk][i], mul,
                                                     C8 && ALIBI ? crow[qbk] - m_fin[qbk] + kbias[kk][i] : crow[qbk] - m_fin[qbk]);
                } else {
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float mk = k0h + 16 * kk + 4 * lg + i < si.c ? mul_c : mul_n;
#pragma unroll
                            for (int qbk = 0; qbk < 2; ++qbk)
                                s[kk][qbk][i] = fmaf(s[kk][qbk][i], mk,
                                                     ALIBI ? crow[qbk] - m_fin[qbk] + kbias[kk][i] : crow[qbk] - m_fin[qbk]);
                        }
                }
            }
        }
        if constexpr (SOFTCAP) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // FP8 cache: cached keys' raw products carry the codes, so their cap input takes
                    // k_scale, and (EXACT_V) their exponent log2 v_scale
                    const bool cached = C8 && k0h + 16 * kk + 4 * lg + i < si.c;
                    const float cin = cached ? cap_in * p.k_scale : cap_in;
                    const float kb = EXACT_V ? kbias[kk][i] + (cached ? lvs : 0.f) : kbias[kk][i];
#pragma unroll
                    for (int qbk = 0; qbk < 2; ++qbk)
                        s[kk][qbk][i] = fmaf(cap2, tanh_fast(s[kk][qbk][i] * cin), kb);
                }
        }

        // ---- mask (partial halves): key k0h + 16 kk + 4 lg + i is visible from row pos iff
        // 16 kk + i <= x and x - (16 kk + i) < W, x = pos - k0h - 4 lg.
        if (!full) {
#pragma unroll
            for (int qbk = 0; qbk < 2; ++qbk) {
                const int x = p0 + 16 * qbk + l16 - k0h - 4 * lg;
                if (p.window > 0) {
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int rel = 16 * kk + i;
                            s[kk][qbk][i] = ((rel <= x) & (x - rel < p.window)) ? s[kk][qbk][i] : -INFINITY;
                        }
                } else {
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            s[kk][qbk][i] = (16 * kk + i <= x) ? s[kk][qbk][i] : -INFINITY;
                }
            }
        }

        // ---- running max (lazy: raised only when a row's max grows by more than kRescaleSlack).
        // PRE: tmax is relative to m_fin and m_thr holds the relative threshold (kRescaleSlack, or
        // -inf until the row has seen a visible key); otherwise both are absolute.
        float tmax[2];
#pragma unroll
        for (int qbk = 0; qbk < 2; ++qbk) {
            // a chain of three-way maxima (exact in any order)
            float mx = fmaxf(fmaxf(s[0][qbk][0], s[0][qbk][1]), s[0][qbk][2]);
            mx = fmaxf(fmaxf(mx, s[0][qbk][3]), s[1][qbk][0]);
            mx = fmaxf(fmaxf(mx, s[1][qbk][1]), s[1][qbk][2]);
            mx = fmaxf(mx, s[1][qbk][3]);
            tmax[qbk] = PRE ? mx : mx + crow[qbk];
        }
        const bool raise = tmax[0] > m_thr[0] || tmax[1] > m_thr[1];
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {
#pragma unroll
            for (int qbk = 0; qbk < 2; ++qbk) {
                const float r = max_xor32(max_xor16(tmax[qbk]));
                const float m_new = fmaxf(m_run[qbk], PRE ? m_fin[qbk] + r : r);
                const float alpha = (m_run[qbk] == -INFINITY) ? 0.f : fast_exp2(m_run[qbk] - m_new);
                const float fin = m_new == -INFINITY ? 0.f : m_new;
                if constexpr (PRE) {
                    // this half's scores were formed against the old stand-in: move them to the new one
                    const float delta = fin - m_fin[qbk];
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                        for (int i = 0; i < 4; ++i) s[kk][qbk][i] -= delta;
                    m_thr[qbk] = m_new == -INFINITY ? -INFINITY : kRescaleSlack;
                } else {
                    m_thr[qbk] = m_new + kRescaleSlack;
                }
                m_run[qbk] = m_new;
                m_fin[qbk] = fin;
                lsum[qbk] *= alpha;
                if constexpr (EXACT_V) lsum_c[qbk] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db) o[qbk][db] *= alpha;
            }
        }

        if (next_kc >= 0) load_k(ks, next_kc);

        // ---- P (16-bit) as the B operand of O^T = V^T P^T: slots 0-3 are keys k0h + 4 lg + i,
        // slots 4-7 keys k0h + 16 + 4 lg + i.  A row whose max is still -inf has seen no visible
        // key; its weights are exp2(-inf) = 0 against a finite stand-in max.
        V8 pb[2];
#pragma unroll
        for (int qbk = 0; qbk < 2; ++qbk) {
            const float off = crow[qbk] - m_fin[qbk];
            uint32_t pk[2][2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                float pf[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    pf[i] = fast_exp2(PRE ? s[kk][qbk][i] : s[kk][qbk][i] + off);
                pk[kk][0] = pack_x2<T>(pf[0], pf[1]);
                pk[kk][1] = pack_x2<T>(pf[2], pf[3]);
            }
            pb[qbk] = __builtin_bit_cast(V8, make_uint4(pk[0][0], pk[0][1], pk[1][0], pk[1][1]));
        }

        // ---- O^T += V^T P^T (V^T read transposed from the row-major V tile), row sums += 1^T P^T
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int qbk = 0; qbk < 2; ++qbk)
                o[qbk][db] = mfma16(vop[db], pb[qbk], o[qbk][db]);
        if constexpr (EXACT_V) {
            // cached keys' weights carry v_scale: their sums go to lsum_c.  Operand slot j holds
            // key k0h + 4 lg + j (j < 4) or k0h + 16 + 4 lg + j - 4.  Both sums are formed for every
            // half (all-ones or all-zero operands unless the half holds both kinds): a branch around
            // the row-sum MFMAs makes the compiler spill their accumulators.
            const int xc = si.c - k0h - 4 * lg;        // slot offsets below xc are cached keys
            const uint32_t one = one2 & 0xffffu;
            uint32_t wc[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int off = 16 * (w >> 1) + 2 * (w & 1);
                wc[w] = (off < xc ? one : 0u) | (off + 1 < xc ? one << 16 : 0u);
            }
            const V8 ones_c = __builtin_bit_cast(V8, make_uint4(wc[0], wc[1], wc[2], wc[3]));
            const V8 ones_n = __builtin_bit_cast(V8, make_uint4(one2 ^ wc[0], one2 ^ wc[1], one2 ^ wc[2], one2 ^ wc[3]));
#pragma unroll
            for (int qbk = 0; qbk < 2; ++qbk) {
                lsum_c[qbk] = mfma16(ones_c, pb[qbk], lsum_c[qbk]);
                lsum[qbk] = mfma16(ones_n, pb[qbk], lsum[qbk]);
            }
        } else {
#pragma unroll
            for (int qbk = 0; qbk < 2; ++qbk) lsum[qbk] = mfma16(ones, pb[qbk], lsum[qbk]);
        }
    };
    // Tile kt from stage (ks, vs), second half first; the first half's K operands are read here.
    auto compute_tile = [&](int kt, const bf16_t *ks, const bf16_t *vs) __attribute__((always_inline)) {
        half(kt * kBN + 32, 1, ks, vs, 0);
        half(kt * kBN, 0, ks, vs, -1);
    };

    // ---- pipeline.  Tiles are taken from the last (nearest the diagonal) to the first: with
    // ALiBi the largest logits of a row sit near its own position, so the running max is found
    // early and later tiles rarely raise it.  While tile kt is computed from one LDS stage, tile
    // kt - 1 streams into the other; block ids run two tiles ahead.  The loop is unrolled by two
    // so each stage is a distinct LDS object.  The explicit vmcnt(0) waits cover every global
    // load of the loop (copies, ids); passing the loaded registers through an empty asm after
    // them keeps the compiler from adding waits of its own further down, which would also wait
    // for the copies in flight.  The first tile's ids are scalar loads, so its copies go out
    // together with Q.
    {
        int i0 = 0, i1 = 0;
        const int r0 = kt_hi * kBN + wrow0;
        if (r0 < si.c) {
            const int32_t *tab = p.block_tables + int64_t(seq) * p.max_blocks;
            i0 = tab[r0 >> p.block_shift];
            i1 = tab[min(r0 + 15, si.c - 1) >> p.block_shift];
        }
        copy_tile(kt_hi, i0, i1, Ks0, Vs0);
    }
    int ids = kt_hi > kt_lo ? fetch_ids(kt_hi - 1) : 0;
    __builtin_amdgcn_s_waitcnt(0x0F70);     // vmcnt(0): this wavefront's copies, ids and Q landed
    fp8_commit(Ks0, Vs0);
#pragma unroll
    for (int qbk = 0; qbk < 2; ++qbk)
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) asm volatile("" : "+v"(qf[qbk][dc]));
    asm volatile("" : "+v"(ids));
    __syncthreads();
    for (int kt = kt_hi; kt >= kt_lo; kt -= 2) {
        CopyPlan cp{nullptr, nullptr, 0};
        // the first half's K operands are read before the next tile's copies go out: the copies may
        // stall at issue, and the reads (of the other LDS stage) need not wait behind them
        load_k(Ks0, 1);
        if (kt > kt_lo) {
            const int i0 = __builtin_amdgcn_readlane(ids, 0), i1 = __builtin_amdgcn_readlane(ids, 1);
            cp = plan_copy(kt - 1, i0, i1);
            if (cp.mode == 0) copy_tile(kt - 1, i0, i1, Ks1, Vs1);
            else issue_all(cp, Ks1, Vs1);
            if (kt - 2 >= kt_lo) ids = fetch_ids(kt - 2);
        }
        compute_tile(kt, Ks0, Vs0);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        fp8_commit(Ks1, Vs1);
        asm volatile("" : "+v"(ids));
        __syncthreads();
        if (kt - 1 < kt_lo) break;
        CopyPlan cq{nullptr, nullptr, 0};
        load_k(Ks1, 1);
        if (kt - 1 > kt_lo) {
            const int i0 = __builtin_amdgcn_readlane(ids, 0), i1 = __builtin_amdgcn_readlane(ids, 1);
            cq = plan_copy(kt - 2, i0, i1);
            if (cq.mode == 0) copy_tile(kt - 2, i0, i1, Ks0, Vs0);
            else issue_all(cq, Ks0, Vs0);
            if (kt - 3 >= kt_lo) ids = fetch_ids(kt - 3);
        }
        compute_tile(kt - 1, Ks1, Vs1);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        fp8_commit(Ks0, Vs0);
        asm volatile("" : "+v"(ids));
        __syncthreads();
    }

    // ---- epilogue: O = O^T / l, rounded to the element type; lane holds d = 16 db + 4 lg + i of its row
#pragma unroll
    for (int qbk = 0; qbk < 2; ++qbk) {
        const int trow = t0 + 16 * qbk + l16;
        if (trow < si.n) {
            // a sink logit joins the row sum only (m_run is finite: the diagonal key is visible)
            const float sink = p.sinks ? fast_exp2(p.sinks[h] * kLog2e - m_run[qbk]) : 0.f;
            const float l = EXACT_V ? lsum[qbk][0] + lsum_c[qbk][0] / p.v_scale : lsum[qbk][0];
            const float inv = 1.f / (l + sink);
            bf16_t *orow = reinterpret_cast<bf16_t *>(p.out) + int64_t(si.start + trow) * p.num_heads * D +
                           int64_t(h) * D + 4 * lg;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                uint2 w;
                w.x = pack_x2<T>(o[qbk][db][0] * inv, o[qbk][db][1] * inv);
                w.y = pack_x2<T>(o[qbk][db][2] * inv, o[qbk][db][3] * inv);
                *reinterpret_cast<uint2 *>(orow + 16 * db) = w;
            }
        }
    }
}

// fp32: a workgroup of 4 wavefronts takes up to 128 (query row, head) pairs of one KV head --
// 32 rows of one query head per wavefront, as in the 16-bit kernel -- and walks their keys in
// 32-key tiles staged in LDS, so each K/V row read from memory serves every row of the workgroup.
// Products run on the fp32 matrix unit (v_mfma_f32_16x16x4_f32): S^T = K Q^T with Q held in
// registers, then O^T += V^T P^T with the weights kept in fp32.  Operand k-slots are permuted
// consistently on both sides (a sum does not depend on its order): in the score MFMAs, step j of
// d-block b gives lane group g the element d = 16 b + 4 g + j, so K and Q are read as float4; in
// the P.V MFMAs, step v of key block kk gives lane group g the key 16 kk + 4 g + v, which is where
// that lane's score already sits.  Softmax in base 2 with an exact running max.
constexpr int kF32Keys = 32;        // keys per tile
constexpr int kF32Pad = 4;          // floats of padding per LDS row (conflict-free operand reads)

struct F32Grid {
    int heads;          // query heads per workgroup (1, 2 or 4: a divisor of the group)
    int rows;           // query rows per workgroup (128 / heads)
    int row_blocks;     // ceil(max_subquery_len / rows)
    int head_blocks;    // group / heads
};

template <int D>
__global__ __launch_bounds__(kThreads, D > 128 ? 1 : 2) void prefill_f32_kernel(PrefillParams p, F32Grid grid) {
    constexpr int DB = D / 16;                              // 16-wide d blocks
    constexpr int LD = D + kF32Pad;                         // LDS row stride (floats)
    constexpr int CPR = D / 4;                              // float4 chunks per row
    constexpr int KPP = kThreads / CPR;                     // key rows per copy pass
    constexpr int PASSES = kF32Keys / KPP;
    // Up to head size 128 the next tile is fetched into registers during the compute and the LDS
    // holds two stages (one barrier per tile); at 256 the registers are taken, and one stage is
    // refilled after the compute.
    constexpr bool PREFETCH = D <= 128;
    constexpr int STAGES = PREFETCH ? 2 : 1;
    constexpr int STAGE = kF32Keys * LD;                    // floats per stage
    __shared__ __attribute__((aligned(16))) float ks[STAGES * STAGE];
    __shared__ __attribute__((aligned(16))) float vs[STAGES * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    // block -> (row block, sequence, KV head, head block); late row blocks first (they see the most keys)
    const int64_t per_level = int64_t(p.num_seqs) * p.num_kv_heads * grid.head_blocks;
    const int rb = grid.row_blocks - 1 - int(blockIdx.x / per_level);
    int64_t rem = blockIdx.x % per_level;
    const int seq = int(rem / (int64_t(p.num_kv_heads) * grid.head_blocks));
    rem %= int64_t(p.num_kv_heads) * grid.head_blocks;
    const int kvh = int(rem / grid.head_blocks);
    const int hblk = int(rem % grid.head_blocks);
    const SeqInfo si = seq_info(p, seq);
    const int t0 = rb * grid.rows;
    if (t0 >= si.n) return;                                 // the whole workgroup: no barrier yet
    const int t_last = min(t0 + grid.rows, si.n) - 1;
    const int key_hi = si.q0 + t_last;
    const int key_lo = p.window > 0 ? max(0, si.q0 + t0 - p.window + 1) : 0;
    const int kt_lo = key_lo / kF32Keys, kt_hi = key_hi / kF32Keys;

    const int group = p.num_heads / p.num_kv_heads;
    const int h = kvh * group + hblk * grid.heads + wave % grid.heads;
    const int w0 = t0 + (wave / grid.heads) * 32;          // first row of this wavefront
    const bool active = w0 < si.n;
    const int wpos_lo = si.q0 + w0, wpos_hi = si.q0 + min(w0 + 31, si.n - 1);

    // Q as the B operand: lane (l16, lg) holds row w0 + 16 qbk + l16, d = 16 b + 4 lg .. + 3
    floatx4_v qf[2][DB];
#pragma unroll
    for (int qbk = 0; qbk < 2; ++qbk) {
        const int trow = min(w0 + 16 * qbk + l16, si.n - 1);
        const float *qrow = reinterpret_cast<const float *>(p.query) + int64_t(si.start + trow) * p.q_stride +
                            int64_t(h) * D + 4 * lg;
#pragma unroll
        for (int b = 0; b < DB; ++b) {
            const float4 v = *reinterpret_cast<const float4 *>(qrow + 16 * b);
            qf[qbk][b] = floatx4_v{v.x, v.y, v.z, v.w};
        }
    }
    const bool has_cap = p.softcap > 0.f;
    const float qk_scale = has_cap ? p.scale / p.softcap : p.scale * kLog2e;
    const float cap2 = p.softcap * kLog2e;
    const float slope2 = p.alibi_slopes ? p.alibi_slopes[h] * kLog2e : 0.f;

    // ---- copies: thread tid moves float4 chunk (tid % CPR) of key rows tid / CPR + KPP * pass.
    // Keys past key_hi re-read row key_hi (masked for every row; a visible row, so finite).
    float4 kr[PASSES], vr[PASSES];
    auto fetch = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps) {
            const int j = min(kt * kF32Keys + tid / CPR + KPP * ps, key_hi);
            const float *kp, *vp;
            row_ptrs<float>(p, si, seq, kvh, D, j, kp, vp);
            kr[ps] = *reinterpret_cast<const float4 *>(kp + 4 * (tid % CPR));
            vr[ps] = *reinterpret_cast<const float4 *>(vp + 4 * (tid % CPR));
        }
    };
    auto commit = [&](int st) __attribute__((always_inline)) {
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps) {
            const int r = tid / CPR + KPP * ps;
            *reinterpret_cast<float4 *>(ks + st * STAGE + r * LD + 4 * (tid % CPR)) = kr[ps];
            *reinterpret_cast<float4 *>(vs + st * STAGE + r * LD + 4 * (tid % CPR)) = vr[ps];
        }
    };

    floatx4_v o[2][DB];
    float m_run[2] = {-INFINITY, -INFINITY}, l_part[2] = {0.f, 0.f};
#pragma unroll
    for (int qbk = 0; qbk < 2; ++qbk)
#pragma unroll
        for (int b = 0; b < DB; ++b) o[qbk][b] = floatx4_v{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int kt, int st) __attribute__((always_inline)) {
        const float *kst = ks + st * STAGE;
        const float *vst = vs + st * STAGE;
        const int k0 = kt * kF32Keys;
        // tiles no row of this wavefront sees
        if (!active || k0 > wpos_hi || (p.window > 0 && k0 + kF32Keys - 1 <= wpos_lo - p.window)) return;
        // ---- S^T = K Q^T: s[kk][qbk] holds keys k0 + 16 kk + 4 lg + v of row 16 qbk + l16
        floatx4_v s[2][2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int qbk = 0; qbk < 2; ++qbk) s[kk][qbk] = floatx4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < DB; ++b) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const float4 kv = *reinterpret_cast<const float4 *>(kst + (16 * kk + l16) * LD + 16 * b + 4 * lg);
                const float ka[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int qbk = 0; qbk < 2; ++qbk)
                        s[kk][qbk] = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[j], qf[qbk][b][j], s[kk][qbk], 0, 0, 0);
            }
        }
        // ---- scale (or soft-cap), ALiBi, mask; the running max and the weights
#pragma unroll
        for (int qbk = 0; qbk < 2; ++qbk) {
            const int pos = si.q0 + w0 + 16 * qbk + l16;
            float mx = -INFINITY;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int key = k0 + 16 * kk + 4 * lg + v;
                    float x = s[kk][qbk][v] * qk_scale;
                    if (has_cap) x = cap2 * tanh_fast(x);
                    x += slope2 * float(key - pos);
                    const bool vis = key <= pos && (p.window <= 0 || key > pos - p.window);
                    x = vis ? x : -INFINITY;
                    s[kk][qbk][v] = x;
                    mx = fmaxf(mx, x);
                }
            mx = max_xor32(max_xor16(mx));
            const float m_new = fmaxf(m_run[qbk], mx);
            const float alpha = m_run[qbk] == -INFINITY ? 0.f : fast_exp2(m_run[qbk] - m_new);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            float ls = 0.f;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float w = fast_exp2(s[kk][qbk][v] - m_use);
                    s[kk][qbk][v] = w;
                    ls += w;
                }
            l_part[qbk] = fmaf(l_part[qbk], alpha, ls);
            m_run[qbk] = m_new;
#pragma unroll
            for (int b = 0; b < DB; ++b) o[qbk][b] *= alpha;
        }
        // ---- O^T += V^T P^T: step v of key block kk gives lane group lg the key 16 kk + 4 lg + v
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                // (at head size 256 the V reads are held back to one key ahead: registers)
                if constexpr (D > 128) __builtin_amdgcn_sched_barrier(0);
                const float *vrow = vst + (16 * kk + 4 * lg + v) * LD + l16;
#pragma unroll
                for (int b = 0; b < DB; ++b) {
                    const float a = vrow[16 * b];
#pragma unroll
                    for (int qbk = 0; qbk < 2; ++qbk)
                        o[qbk][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, s[kk][qbk][v], o[qbk][b], 0, 0, 0);
                }
            }
    };

    // ---- pipeline.  Two stages: tile kt is computed from stage st while tile kt - 1 goes into the
    // other one (last read by the previous tile's compute, which every wavefront finished before
    // the previous barrier); one stage: the fetch and the refill follow the compute.
    fetch(kt_hi);
    commit(0);
    __syncthreads();
    int st = 0;
    for (int kt = kt_hi; kt >= kt_lo; --kt) {
        if constexpr (PREFETCH) {
            if (kt > kt_lo) fetch(kt - 1);
            compute(kt, st);
            if (kt > kt_lo) commit(st ^ 1);
            __syncthreads();
            st ^= 1;
        } else {
            compute(kt, 0);
            __syncthreads();
            if (kt > kt_lo) {
                fetch(kt - 1);
                commit(0);
                __syncthreads();
            }
        }
    }

    // ---- epilogue: lane (l16, lg) holds O^T[d = 16 b + 4 lg + v][row 16 qbk + l16]
    if (!active) return;
#pragma unroll
    for (int qbk = 0; qbk < 2; ++qbk) {
        const int trow = w0 + 16 * qbk + l16;
        float l = xor_sum_from<16>(l_part[qbk]);
        if (p.sinks) l += fast_exp2(p.sinks[h] * kLog2e - m_run[qbk]);
        if (trow < si.n) {
            const float inv = 1.f / l;
            float *orow = reinterpret_cast<float *>(p.out) + int64_t(si.start + trow) * p.num_heads * D +
                          int64_t(h) * D + 4 * lg;
#pragma unroll
            for (int b = 0; b < DB; ++b)
                *reinterpret_cast<float4 *>(orow + 16 * b) =
                    make_float4(o[qbk][b][0] * inv, o[qbk][b][1] * inv, o[qbk][b][2] * inv, o[qbk][b][3] * inv);
        }
    }
}

template <typename T>
hipError_t launch_mfma(const PrefillParams &p, int head_size, hipStream_t stream) {
    PrefillGrid grid;
    const int group = p.num_heads / p.num_kv_heads;
    grid.heads = group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1);
    grid.rows = kRowsPerBlock / grid.heads;
    grid.num_qtiles = (p.max_subquery_len + grid.rows - 1) / grid.rows;
    const int hblocks = group / grid.heads;
    grid.compact = p.num_seqs <= 64 && grid.num_qtiles <= 64 ? 1 : 0;
    grid.qtiles_per_group = grid.compact || hblocks >= 8 ? 1 : min(8 / hblocks, grid.num_qtiles);
    if (grid.qtiles_per_group < 1) grid.qtiles_per_group = 1;
    grid.num_qblocks = (grid.num_qtiles + grid.qtiles_per_group - 1) / grid.qtiles_per_group;
    grid.group_size = hblocks * grid.qtiles_per_group;
    int64_t groups = int64_t(grid.num_qblocks) * p.num_seqs * p.num_kv_heads;
    if (grid.compact) {
        // sum over sequences of ceil(n / rows) <= num_tokens / rows + num_seqs
        const int64_t tiles = p.num_tokens / grid.rows + p.num_seqs;
        groups = min(groups, tiles * p.num_kv_heads);
    }
    if (groups == 0) return hipSuccess;
    const int64_t blocks = (groups + 7) / 8 * 8 * grid.group_size;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    grid.num_groups = int(groups);
    const dim3 nb = dim3(unsigned(blocks)), nt = dim3(kThreads);
    const int variant = (p.alibi_slopes != nullptr ? 1 : 0) | (p.softcap > 0.f ? 2 : 0);
    if (head_size != 128 && head_size != 64 && head_size != 256) return hipErrorInvalidValue;
    auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, nb, nt, 0, stream, p, grid); };
    if (head_size == 256) {
        switch (variant) {
            case 0: go(prefill_mfma_kernel<T, 256, false, false>); break;
            case 1: go(prefill_mfma_kernel<T, 256, true, false>); break;
            case 2: go(prefill_mfma_kernel<T, 256, false, true>); break;
            default: go(prefill_mfma_kernel<T, 256, true, true>); break;
        }
    } else if (head_size == 128) {
        switch (variant) {
            case 0: go(prefill_mfma_kernel<T, 128, false, false>); break;
            case 1: go(prefill_mfma_kernel<T, 128, true, false>); break;
            case 2: go(prefill_mfma_kernel<T, 128, false, true>); break;
            default: go(prefill_mfma_kernel<T, 128, true, true>); break;
        }
    } else {
        switch (variant) {
            case 0: go(prefill_mfma_kernel<T, 64, false, false>); break;
            case 1: go(prefill_mfma_kernel<T, 64, true, false>); break;
            case 2: go(prefill_mfma_kernel<T, 64, false, true>); break;
            default: go(prefill_mfma_kernel<T, 64, true, true>); break;
        }
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillParams &p, int dtype, int head_size, hipStream_t stream) {
    if (dtype == 1) return launch_mfma<bf16_t>(p, head_size, stream);
    if (dtype == 2) return launch_mfma<f16_t>(p, head_size, stream);
    if (dtype == 3) return launch_mfma<bf16_c8_t>(p, head_size, stream);
    if (dtype == 4) return launch_mfma<f16_c8_t>(p, head_size, stream);
    if (p.uniform_qlen > 0) return hipErrorInvalidValue;      // the uniform mode has 16-bit kernels only
    F32Grid grid;
    const int group = p.num_heads / p.num_kv_heads;
    grid.heads = group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1);
    grid.rows = kRowsPerBlock / grid.heads;
    grid.row_blocks = (p.max_subquery_len + grid.rows - 1) / grid.rows;
    grid.head_blocks = group / grid.heads;
    const int64_t blocks = int64_t(grid.row_blocks) * p.num_seqs * p.num_kv_heads * grid.head_blocks;
    if (blocks == 0 || p.num_tokens == 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 nb = dim3(unsigned(blocks)), nt = dim3(kThreads);
    if (head_size == 256)
        hipLaunchKernelGGL(prefill_f32_kernel<256>, nb, nt, 0, stream, p, grid);
    else if (head_size == 128)
        hipLaunchKernelGGL(prefill_f32_kernel<128>, nb, nt, 0, stream, p, grid);
    else if (head_size == 64)
        hipLaunchKernelGGL(prefill_f32_kernel<64>, nb, nt, 0, stream, p, grid);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace pa
