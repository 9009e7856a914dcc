// Device helpers shared by the libmoe355 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe355 {

constexpr int kWave = 64;
constexpr float kE4M3Max = 448.0f;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// fp32 -> OCP e4m3fn code: nearest, ties to even mantissa, saturating at
// +-448, sign kept (so -0 and negative underflow give 0x80).  Integer ops
// only, so the rounding is exactly the one stated; inputs are finite.
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  // |y| < 2^-6: multiples of 2^-9, nearest-even (8 encodes 2^-6 itself)
  const uint32_t sub = (uint32_t)__builtin_rintf(__uint_as_float(a < 0x3C800000u ? a : 0x3C800000u) * 512.0f);
  // normal range: keep 3 mantissa bits, nearest-even on the 20 dropped bits
  const uint32_t mant = a & 0x7fffffu;
  uint32_t code = (((a >> 23) - 120u) << 3) | (mant >> 20);
  const uint32_t rem = mant & 0xfffffu;
  code += (rem > 0x80000u || (rem == 0x80000u && (code & 1u))) ? 1u : 0u;  // carry into exponent is right
  uint32_t r = a < 0x3C800000u ? sub : code;
  r = a >= 0x43E00000u ? 0x7Eu : r;  // |y| >= 448 saturates
  return sign | r;
}

// Four fp32 values -> their e4m3 codes (byte i = value i) by the hardware conversion
// (v_cvt_pk_fp8_f32: OCP e4m3, nearest-even).  On every finite fp32 with |y| <= 460 it gives
// exactly f32_to_e4m3's code (an exhaustive check over all such bit patterns,
// tuning/e4m3_cvt_check.hip), so inputs are first clamped to +-460, which leaves their codes
// unchanged (everything from 448 up saturates to 448).  Inputs are finite.
__device__ __forceinline__ uint32_t f32x4_to_e4m3(float a, float b, float c, float d) {
  auto cl = [](float y) { return __builtin_amdgcn_fmed3f(y, -460.0f, 460.0f); };
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), r, true);
  return (uint32_t)r;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> bf16 bits, nearest-even (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// fp16 bits of x, round to nearest even (the hardware conversion)
__device__ __forceinline__ uint32_t f32_to_f16(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

// 16-bit output element: bf16 or fp16 bits of x, nearest even
__device__ __forceinline__ uint32_t f32_to_out16(float x, bool fp16) { return fp16 ? f32_to_f16(x) : f32_to_bf16(x); }

__device__ __forceinline__ float wave_max_f32(float v, int width) {
  for (int o = width / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// D = A(16x128 e4m3) * B(128x16 e4m3) + C.  Lane l holds row/column l%16 and
// 32 of the K slots (slots [32*(l/16), 32*(l/16)+32)); A and B must place the
// same K index in the same slot.  Output element (4*(l/16)+i, l%16) in c[i].
__device__ __forceinline__ v4f mfma16x16x128_fp8(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

}  // namespace moe355
