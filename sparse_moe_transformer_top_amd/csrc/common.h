// Device-side helpers shared by the layer's HIP kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// Native 16-byte vector (clang ext vector). Register arrays of HIP's uint4
// (a union struct) are not split into registers by SROA; arrays of u32x4 are.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define MOE_DEV __device__ __forceinline__

// bf16 halves of a packed 32-bit word -> float32 (exact)
MOE_DEV float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
MOE_DEV float bf16hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// float32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
MOE_DEV uint16_t f32_to_bf16_bits(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}
MOE_DEV uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// silu(g) * u in float32: g * u / (1 + exp(-g)). expf is the device math
// library's; for g -> -inf the quotient goes to -0, for g -> +inf to g * u.
MOE_DEV float swiglu(float g, float u) { return g * u / (1.0f + __expf(-g)); }

// Four int8 values packed in a word -> two words of packed bf16 (exact:
// |q| <= 127 fits the 8-bit bf16 significand). The signed byte is biased to
// unsigned (xor 0x80), converted with v_cvt_f32_ubyteN, and 128 subtracted.
MOE_DEV void i8x4_to_bf16x4(uint32_t q, uint32_t& lo, uint32_t& hi) {
  uint32_t u = q ^ 0x80808080u;
  float f0 = (float)(u & 0xffu) - 128.0f;
  float f1 = (float)((u >> 8) & 0xffu) - 128.0f;
  float f2 = (float)((u >> 16) & 0xffu) - 128.0f;
  float f3 = (float)(u >> 24) - 128.0f;
  // exact values: taking the high halves is exact
  lo = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xffff0000u);
  hi = (__float_as_uint(f2) >> 16) | (__float_as_uint(f3) & 0xffff0000u);
}

// Eight int8 values (two words) -> eight bf16 (one 16-byte vector), exact.
MOE_DEV u32x4 i8x8_to_bf16x8(uint32_t q0, uint32_t q1) {
  uint32_t a, b, c, d;
  i8x4_to_bf16x4(q0, a, b);
  i8x4_to_bf16x4(q1, c, d);
  return u32x4{a, b, c, d};
}

MOE_DEV bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
MOE_DEV bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Work-group id -> logical tile id so that consecutive logical tiles run on
// the same XCD (the hardware deals work-groups round-robin over 8 XCDs, each
// with its own L2). Valid for any grid size n.
MOE_DEV uint32_t xcd_swizzle(uint32_t bid, uint32_t n) {
  const uint32_t X = 8;
  uint32_t xcd = bid % X, slot = bid / X;
  uint32_t base = n / X, rem = n % X;
  // XCDs [0, rem) hold base+1 logical tiles, the rest hold base
  uint32_t start = xcd < rem ? xcd * (base + 1) : rem * (base + 1) + (xcd - rem) * base;
  return start + slot;
}

template <typename T>
MOE_DEV T wave_sum_xor(T v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}
