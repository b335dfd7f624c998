// q8_device.hpp -- device-side helpers shared by the libq8 kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned u32;
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// bf16 bits -> fp32 (exact: the bf16 pattern is the top half of the fp32 one)
__device__ __forceinline__ float bf16_lo(u32 w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(u32 w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((u32)b << 16); }

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ u32 pack_bf16x2(float lo, float hi) {
    return (u32)f32_to_bf16(lo) | ((u32)f32_to_bf16(hi) << 16);
}

// fp16 bits -> fp32 (exact) and fp32 -> fp16 bits, round to nearest even
// (v_cvt_f16_f32 under the default rounding mode, fp16 denormals kept).
__device__ __forceinline__ float f16_lo(u32 w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float f16_hi(u32 w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }
__device__ __forceinline__ uint16_t f32_to_f16(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
__device__ __forceinline__ u32 pack_f16x2(float lo, float hi) {
    return (u32)f32_to_f16(lo) | ((u32)f32_to_f16(hi) << 16);
}

// The 16-bit activation / output formats of the layer: bf16 (F16 = false)
// or IEEE fp16 (F16 = true).
template <bool F16>
__device__ __forceinline__ float h16_lo(u32 w) { if constexpr (F16) return f16_lo(w); else return bf16_lo(w); }
template <bool F16>
__device__ __forceinline__ float h16_hi(u32 w) { if constexpr (F16) return f16_hi(w); else return bf16_hi(w); }
template <bool F16>
__device__ __forceinline__ float h16_to_f32(uint16_t b) {
    if constexpr (F16) return (float)__builtin_bit_cast(_Float16, b); else return bf16_to_f32(b);
}
template <bool F16>
__device__ __forceinline__ u32 pack16x2(float lo, float hi) {
    if constexpr (F16) return pack_f16x2(lo, hi); else return pack_bf16x2(lo, hi);
}

// Symmetric INT8 code of x for scale s: clamp(rne(x / s), -127, 127), with
// x / s the correctly rounded fp32 quotient (IEEE division; the library is
// built without fast-math so '/' is exact-rounded).  s == 0 gives 0.
__device__ __forceinline__ int code_of(float x, float s) {
    if (s == 0.0f) return 0;
    float r = __builtin_rintf(x / s);
    r = __builtin_fminf(__builtin_fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

__device__ __forceinline__ u32 pack_i8x4(int a, int b, int c, int d) {
    return (u32)(a & 0xFF) | ((u32)(b & 0xFF) << 8) | ((u32)(c & 0xFF) << 16) |
           ((u32)(d & 0xFF) << 24);
}

// 4 int8 codes (one dword) -> 4 exact bf16 values (two dwords).
__device__ __forceinline__ v2u i8x4_to_bf16x4(u32 d) {
    const float f0 = (float)(int8_t)(d & 0xFF);
    const float f1 = (float)(int8_t)((d >> 8) & 0xFF);
    const float f2 = (float)(int8_t)((d >> 16) & 0xFF);
    const float f3 = (float)(int8_t)(d >> 24);
    // the conversions are exact, so truncating to the top 16 bits is exact;
    // one v_perm_b32 per pair takes bytes 2-3 of each (the shift + and-or
    // the plain expression compiles to is two instructions)
    return v2u{__builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u),
               __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u)};
}

// 4 int8 codes (one dword) -> 4 exact fp16 values (two dwords): |q| <= 128
// fits the 11-bit fp16 significand, so the round-toward-zero pack of the
// exact fp32 values (one v_cvt_pkrtz_f16_f32 per pair) is exact.
__device__ __forceinline__ v2u i8x4_to_f16x4(u32 d) {
    const float f0 = (float)(int8_t)(d & 0xFF);
    const float f1 = (float)(int8_t)((d >> 8) & 0xFF);
    const float f2 = (float)(int8_t)((d >> 16) & 0xFF);
    const float f3 = (float)(int8_t)(d >> 24);
    return v2u{__builtin_bit_cast(u32, __builtin_amdgcn_cvt_pkrtz(f0, f1)),
               __builtin_bit_cast(u32, __builtin_amdgcn_cvt_pkrtz(f2, f3))};
}
template <bool F16>
__device__ __forceinline__ v2u i8x4_to_h16x4(u32 d) {
    if constexpr (F16) return i8x4_to_f16x4(d); else return i8x4_to_bf16x4(d);
}

typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// Wave-wide (64 lanes) maximum of a non-negative float.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Remap a linear workgroup id so that the ids one XCD receives (the hardware
// deals workgroups round-robin over the 8 XCDs) form one contiguous range of
// tile ids: neighbouring tiles then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
    const int q = total >> 3, r = total & 7;
    const int xcd = bid & 7, local = bid >> 3;
    return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

}  // namespace q8
