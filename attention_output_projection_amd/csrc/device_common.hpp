// device_common.hpp -- small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oproj {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr float kFp8Max = 448.0f;       // largest finite e4m3fn magnitude
constexpr float kAmaxFloor = 1e-10f;    // all-zero block floor

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite values).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Round a positive normal fp32 up to a power of two (kept when already one).
__device__ __forceinline__ float pow2_ceil(float s) {
    uint32_t u = __float_as_uint(s);
    if (u & 0x007FFFFFu) u = (u & 0xFF800000u) + 0x00800000u;
    return __uint_as_float(u);
}

// v / s, correctly rounded, from r = 1/s (correctly rounded) with one
// Markstein correction step: q0 = v*r, e = v - q0*s (exact), q = q0 + e*r.
// For every quotient of magnitude >= 2^-20 this equals the IEEE quotient;
// smaller quotients all encode to an FP8 zero of the same sign either way.
__device__ __forceinline__ float div_by_scale(float v, float s, float r) {
    float q0 = v * r;
    float e = __builtin_fmaf(-q0, s, v);
    return __builtin_fmaf(e, r, q0);
}

// Two fp32 -> two e4m3fn codes (hardware conversion, round to nearest even)
// written into the low (HI = false) or high 16 bits of `old`; inputs are
// clamped to +-448 first.
template <bool HI>
__device__ __forceinline__ uint32_t cvt2_fp8(float a, float b, uint32_t old) {
    a = __builtin_amdgcn_fmed3f(a, -kFp8Max, kFp8Max);
    b = __builtin_amdgcn_fmed3f(b, -kFp8Max, kFp8Max);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

// E8M0 byte of a power-of-two fp32 scale (its biased exponent).
__device__ __forceinline__ int e8m0_of(float s) { return (int)((__float_as_uint(s) >> 23) & 0xFFu); }

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Max over each row of 16 lanes (DPP: quad swaps, half-row mirror, row mirror).
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp_f<0xB1>(x));   // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp_f<0x4E>(x));   // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp_f<0x141>(x));  // row_half_mirror
    x = fmaxf(x, dpp_f<0x140>(x));  // row_mirror
    return x;
}

}  // namespace oproj
