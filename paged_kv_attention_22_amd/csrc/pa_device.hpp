// Device helpers for gfx950 (CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace pa {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// bf16 halves of a 32-bit word -> fp32 (exact).
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

// fp16 halves of a 32-bit word -> fp32 (exact), and fp32 -> fp16 bits with the
// conversion instruction's round-to-nearest-even.
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float h_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)w); }
__device__ __forceinline__ float h_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }
__device__ __forceinline__ uint32_t f16_rne(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) { return f16_rne(lo) | (f16_rne(hi) << 16); }

// 2-wide fp16 dot product accumulated into fp32 (v_dot2_f32_f16).
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, a), __builtin_bit_cast(half2v, b), c, false);
}

// 2-wide bf16 dot product accumulated into fp32 (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

// 16-bit element types: uint16_t carries bf16 bit patterns, _Float16 carries
// fp16.  These pick the conversions and the dot product per type.
template <typename T>
inline constexpr bool kIs16 = std::is_same_v<T, uint16_t> || std::is_same_v<T, _Float16>;
template <typename T>
__device__ __forceinline__ float lo16(uint32_t w) {
    if constexpr (std::is_same_v<T, uint16_t>) return bf_lo(w); else return h_lo(w);
}
template <typename T>
__device__ __forceinline__ float hi16(uint32_t w) {
    if constexpr (std::is_same_v<T, uint16_t>) return bf_hi(w); else return h_hi(w);
}
template <typename T>
__device__ __forceinline__ uint32_t to16(float f) {  // rounded bits (conversion instruction, nearest even)
    if constexpr (std::is_same_v<T, uint16_t>) return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
    else return f16_rne(f);
}
template <typename T>
__device__ __forceinline__ uint32_t pack16(float lo, float hi) {
    if constexpr (std::is_same_v<T, uint16_t>) return pack_bf16x2(lo, hi); else return pack_f16x2(lo, hi);
}
template <typename T>
__device__ __forceinline__ float dot16(uint32_t a, uint32_t b, float c) {
    if constexpr (std::is_same_v<T, uint16_t>) return dot2_bf16(a, b, c); else return dot2_f16(a, b, c);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}

// Sum over aligned groups of R consecutive lanes; every lane of the group gets
// the total.  Steps: swap neighbours (quad_perm 1,0,3,2), swap pairs
// (quad_perm 2,3,0,1), then mirror within 8 lanes and within 16 lanes, which
// pair each lane with one in the other half of the group.
template <int R>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(R == 4 || R == 8 || R == 16 || R == 32 || R == 64, "group size");
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    if constexpr (R >= 8) x += dpp<0x141>(x);
    if constexpr (R >= 16) x += dpp<0x140>(x);
    if constexpr (R >= 32) x += __shfl_xor(x, 16);
    if constexpr (R >= 64) x += __shfl_xor(x, 32);
    return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte global load / store.
// 16-byte loads and stores go through a native 4 x u32 vector so that the
// compiler keeps the values in registers (a struct copy can end up as a
// memcpy through private memory).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16(const void* p) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// 16-byte load marked non-temporal: data read once (K/V streamed from HBM)
// should not displace cached data that is reused.
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st16(void* p, uint4 v) {
    *reinterpret_cast<u32x4*>(p) = u32x4{v.x, v.y, v.z, v.w};
}

}  // namespace pa
