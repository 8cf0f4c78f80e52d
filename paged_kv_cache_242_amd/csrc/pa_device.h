// Device-side helpers shared by the gfx950 kernels of libpa (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// bf16 values travel as raw 16-bit patterns; arithmetic is done in fp32.
typedef uint16_t bf16_t;
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef float floatx4_v __attribute__((ext_vector_type(4)));
typedef float floatx16_v __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16_t x) { return __uint_as_float(uint32_t(x) << 16); }

// fp32 -> bf16, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ bf16_t f32_to_bf16(float x) {
    __bf16 b = static_cast<__bf16>(x);
    return __builtin_bit_cast(bf16_t, b);
}

// Two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float float2_v __attribute__((ext_vector_type(2)));
    const float2_v v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_v));
}

// c + a.lo * b.lo + a.hi * b.hi with bf16 pairs (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, a), __builtin_bit_cast(bf16x2_v, b), c,
                                           false);
}

// fp16 values travel as raw 16-bit patterns too, in a type of their own so that templates can
// tell them from bf16; arithmetic is done in fp32.
enum class f16_t : uint16_t {};
typedef _Float16 halfx2_v __attribute__((ext_vector_type(2)));
typedef _Float16 halfx8_v __attribute__((ext_vector_type(8)));

template <typename T>
inline constexpr bool kIsF16 = false;
template <>
inline constexpr bool kIsF16<f16_t> = true;

__device__ __forceinline__ float f16_to_f32(f16_t x) { return float(__builtin_bit_cast(_Float16, x)); }

// fp32 -> fp16, round to nearest even (v_cvt_f16_f32 under the default rounding mode).
__device__ __forceinline__ f16_t f32_to_f16(float x) { return __builtin_bit_cast(f16_t, static_cast<_Float16>(x)); }

// Two fp32 -> packed fp16 pair (lo in bits 0..15), round to nearest even.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    typedef float float2_v __attribute__((ext_vector_type(2)));
    const float2_v v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, halfx2_v));
}

// c + a.lo * b.lo + a.hi * b.hi with fp16 pairs (v_dot2_f32_f16).
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(halfx2_v, a), __builtin_bit_cast(halfx2_v, b), c, false);
}

// The 16-bit element types by name: conversions and pair dot products.
template <typename T>
__device__ __forceinline__ T to_elt(float x);
template <>
__device__ __forceinline__ bf16_t to_elt<bf16_t>(float x) { return f32_to_bf16(x); }
template <>
__device__ __forceinline__ f16_t to_elt<f16_t>(float x) { return f32_to_f16(x); }
__device__ __forceinline__ float elt_to_f32(bf16_t x) { return bf16_to_f32(x); }
__device__ __forceinline__ float elt_to_f32(f16_t x) { return f16_to_f32(x); }
template <typename T>
__device__ __forceinline__ uint32_t pack_x2(float lo, float hi) {
    if constexpr (kIsF16<T>) return pack_f16x2(lo, hi);
    else return pack_bf16x2(lo, hi);
}
template <typename T>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    if constexpr (kIsF16<T>) return dot2_f16(a, b, c);
    else return dot2_bf16(a, b, c);
}

// Query / output element types (bf16, fp16) of layers whose paged cache holds FP8 E4M3 codes: the
// kernels take them as their element type and read the cache as one byte per element.
enum class bf16_c8_t : uint16_t {};
enum class f16_c8_t : uint16_t {};
template <>
inline constexpr bool kIsF16<f16_c8_t> = true;
template <typename T>
inline constexpr bool kFp8Cache = false;
template <>
inline constexpr bool kFp8Cache<bf16_c8_t> = true;
template <>
inline constexpr bool kFp8Cache<f16_c8_t> = true;
template <>
__device__ __forceinline__ bf16_c8_t to_elt<bf16_c8_t>(float x) { return bf16_c8_t(f32_to_bf16(x)); }
template <>
__device__ __forceinline__ f16_c8_t to_elt<f16_c8_t>(float x) { return f16_c8_t(uint16_t(f32_to_f16(x))); }
__device__ __forceinline__ float elt_to_f32(bf16_c8_t x) { return bf16_to_f32(uint16_t(x)); }
__device__ __forceinline__ float elt_to_f32(f16_c8_t x) { return f16_to_f32(f16_t(uint16_t(x))); }

// Eight E4M3 codes (bytes 0..7 of c) -> four pairs of the 16-bit type T (element 2k in the low
// half of word k), exactly: every E4M3 value is representable in bf16 and in fp16.
template <typename T, bool HI>
__device__ __forceinline__ uint32_t widen_e4m3_pair(uint32_t src) {
    if constexpr (kIsF16<T>)
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(src, 1.f, HI));
    else
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src, 1.f, HI));
}
template <typename T>
__device__ __forceinline__ uint4 widen_e4m3(uint2 c) {
    return make_uint4(widen_e4m3_pair<T, false>(c.x), widen_e4m3_pair<T, true>(c.x), widen_e4m3_pair<T, false>(c.y),
                      widen_e4m3_pair<T, true>(c.y));
}

// Byte permute: result byte k = byte sel[k] of the 8-byte value {hi:lo}.
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}
// From two bf16 pairs a = (a0, a1) and b = (b0, b1): (a0, b0) and (a1, b1).
__device__ __forceinline__ uint32_t interleave_lo(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t interleave_hi(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x07060302u); }

// DPP lane moves inside a row of 16 lanes.
enum : int {
    kDppQuadXor1 = 0xB1,      // quad_perm [1,0,3,2]: lane ^ 1
    kDppQuadXor3 = 0x1B,      // quad_perm [3,2,1,0]: lane ^ 3
    kDppHalfMirror = 0x141,   // lane ^ 7 inside each 8 lanes
    kDppMirror = 0x140,       // lane ^ 15 inside each 16 lanes
    kDppRowRor8 = 0x128,      // (lane + 8) mod 16: lane ^ 8 inside each 16 lanes
};

template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Value of lane (lane ^ mask) for masks of the form 2^k - 1 (k = 1..6) or 2^k.
template <int MASK>
__device__ __forceinline__ float lane_xor(float x) {
    if constexpr (MASK == 1) return dpp_move<kDppQuadXor1>(x);
    else if constexpr (MASK == 3) return dpp_move<kDppQuadXor3>(x);
    else if constexpr (MASK == 7) return dpp_move<kDppHalfMirror>(x);
    else if constexpr (MASK == 15) return dpp_move<kDppMirror>(x);
    else if constexpr (MASK == 8) return dpp_move<kDppRowRor8>(x);
    else return __shfl_xor(x, MASK, 64);
}

// Sum / max over the lanes lane ^ M, lane ^ 2M, ... (M a power of two): combines the row groups
// of a wavefront whose rows are M lanes wide.
template <int M>
__device__ __forceinline__ float xor_sum_from(float x) {
    if constexpr (M < 64) {
        x += lane_xor<M>(x);
        return xor_sum_from<M * 2>(x);
    } else {
        return x;
    }
}
template <int M>
__device__ __forceinline__ float xor_max_from(float x) {
    if constexpr (M < 64) {
        x = fmaxf(x, lane_xor<M>(x));
        return xor_max_from<M * 2>(x);
    } else {
        return x;
    }
}

__device__ __forceinline__ float readlane_f(float x, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// tanh x = 1 - 2 / (e^(2x) + 1): v_exp and v_rcp, absolute error a few 1e-7; saturates to +-1
// (e^(2x) overflows to infinity or underflows to 0).
__device__ __forceinline__ float tanh_fast(float x) {
    const float e = fast_exp2(x * (2.f * kLog2e));
    return 1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f);
}

// Compiler barrier for LDS traffic that stays inside one wavefront.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// max(x, x of lane ^ 16) and max(x, x of lane ^ 32) with the gfx950 row-swap moves (VALU, no
// LDS traffic): swapping x with itself leaves each lane one of its own value and its partner's.
__device__ __forceinline__ float max_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// 8 elements of a 16x16x32 MFMA operand, by element type (an FP8-cache type computes in its
// 16-bit type).
template <typename T>
struct Operand8 { typedef bf16x8_v type; };
template <>
struct Operand8<f16_t> { typedef halfx8_v type; };
template <>
struct Operand8<f16_c8_t> { typedef halfx8_v type; };

__device__ __forceinline__ floatx4_v mfma16(bf16x8_v a, bf16x8_v b, floatx4_v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4_v mfma16(halfx8_v a, halfx8_v b, floatx4_v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// One 16-byte-per-lane global -> LDS copy: lane l reads base + soff + lane_off (bytes) and fills
// 16-byte unit l of the 1 KB stretch at lds_dst.  base and soff must be wave-uniform; base goes
// into a raw buffer descriptor (scalar registers), soff into the scalar offset and the lane
// offset into the vector offset.
__device__ __forceinline__ void dma16(const char *base, uint32_t lane_off, uint32_t soff, bf16_t *lds_dst) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), 0, 0x7fffffff, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds_dst, 16, lane_off, soff, 0, 0);
}

// The same copy into the LDS byte address lds_addr.
__device__ __forceinline__ void dma16_at(const char *base, uint32_t lane_off, uint32_t soff, uint32_t lds_addr) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), 0, 0x7fffffff, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(uintptr_t)lds_addr, 16, lane_off, soff, 0, 0);
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_address(const void *p) {
    return uint32_t(uintptr_t((const lds_void *)p));
}

// The same copy from a per-lane address.
__device__ __forceinline__ void dma16_lane(const char *src, bf16_t *lds_dst) {
    __builtin_amdgcn_global_load_lds((global_void *)src, (lds_void *)lds_dst, 16, 0, 0);
}

}  // namespace pa
