// Device helpers shared by the libmla kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short short4_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float float4_t;

// float32 -> bfloat16 bits, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Element `i` of an array stored as bf16 (is_bf16) or float32.
__device__ __forceinline__ float load_elem(const void* p, int64_t i, bool is_bf16) {
  return is_bf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i])
                 : static_cast<const float*>(p)[i];
}

__device__ __forceinline__ void store_elem(void* p, int64_t i, float v, bool is_bf16) {
  if (is_bf16)
    static_cast<uint16_t*>(p)[i] = f32_to_bf16_bits(v);
  else
    static_cast<float*>(p)[i] = v;
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

// Two float32 -> bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 r;
  r[0] = static_cast<__bf16>(a);
  r[1] = static_cast<__bf16>(b);
  return __builtin_bit_cast(uint32_t, r);
}

// theta_k = rope_base^(-2k / d_h^R) for the 32 rotation pairs of the 64-wide
// RoPE part, computed on the host in float64 and passed by value
struct RopeTheta {
  double t[32];
};

// sin and cos of a float64 angle x: x reduced to [-pi, pi] in float64 (two-term
// Cody-Waite with fused multiply-adds, error ~1e-15 for |x| < 2^20), then sin/cos
// of the reduced angle in float32 (about 1 float32 ulp from the float64 result
// rounded to float32)
__device__ __forceinline__ void sincos_reduced(double x, float& sn, float& cs) {
  constexpr double kTwoPiHi = 6.283185307179586, kTwoPiLo = 2.4492935982947064e-16;
  const double n = rint(x * (1.0 / kTwoPiHi));
  double r = fma(-n, kTwoPiHi, x);
  r = fma(-n, kTwoPiLo, r);
  sincosf(static_cast<float>(r), &sn, &cs);
}

}  // namespace mla
