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

// silu(g) * u in float32: g * u * (1 / (1 + exp(-g))), with the device
// library's fast exp and the hardware reciprocal (v_rcp_f32, 1 ulp) instead
// of an IEEE division (a dozen instructions, which made the gate/up
// epilogue a measurable part of each tile); both errors are far below the
// bf16 rounding of h and the float32 path's 1e-4 tolerance. For g -> -inf
// the product goes to -0 (rcp(inf) = 0, g finite), for g -> +inf to g * u.
MOE_DEV float swiglu(float g, float u) {
  return g * u * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// Four int8 values packed in a word -> two words of packed bf16 (exact: an
// int8 has at most 8 significant bits, which the bf16 significand holds, so
// the high half of the float32 is the bf16 value). Each byte converts with
// one sign-extending v_cvt_f32_i32 (SDWA byte select); v_perm_b32 packs the
// high halves of two floats into one word.
MOE_DEV uint32_t pack_hi_halves(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}
MOE_DEV void i8x4_to_bf16x4(uint32_t q, uint32_t& lo, uint32_t& hi) {
  const float f0 = (float)(int8_t)q, f1 = (float)(int8_t)(q >> 8);
  const float f2 = (float)(int8_t)(q >> 16), f3 = (float)((int32_t)q >> 24);
  lo = pack_hi_halves(f0, f1);
  hi = pack_hi_halves(f2, f3);
}

// Eight int8 values (two words) -> eight bf16 (one 16-byte vector), exact.
MOE_DEV u32x4 i8x8_to_bf16x8(uint32_t q0, uint32_t q1) {
  uint32_t a, b, c, d;
  i8x4_to_bf16x4(q0, a, b);
  i8x4_to_bf16x4(q1, c, d);
  return u32x4{a, b, c, d};
}

// Eight 4-bit codes u (one word; byte j holds element 2j in its low nibble
// and element 2j+1 in its high nibble) -> eight bf16 values 128 + u, exact:
// bf16 0x4300 is 128 with an empty 7-bit mantissa, which the code fills. The
// values come out in the element order 0, 2, 4, 6, 1, 3, 5, 7 (the MFMA's k
// order within a lane is free as long as the activations take the same
// order: bf16x8_even_odd). The low nibbles (even elements) and the high
// nibbles (odd elements) are first split into one code per byte; a byte
// permute then interleaves two codes with the exponent byte 0x43 taken from
// a constant word: 7 VALU operations per word of codes. The caller removes
// the bias.
MOE_DEV u32x4 u4x8_to_bf16x8_biased(uint32_t w) {
  const uint32_t ev = w & 0x0F0F0F0Fu;          // byte j: element 2j
  const uint32_t od = (w >> 4) & 0x0F0F0F0Fu;   // byte j: element 2j + 1
  constexpr uint32_t kExp = 0x43434343u;
  u32x4 r;
  // selector bytes 0..3 pick bytes of the second operand, 4 the constant's
  r.x = __builtin_amdgcn_perm(kExp, ev, 0x04010400u);   // elements 0, 2
  r.y = __builtin_amdgcn_perm(kExp, ev, 0x04030402u);   // 4, 6
  r.z = __builtin_amdgcn_perm(kExp, od, 0x04010400u);   // 1, 3
  r.w = __builtin_amdgcn_perm(kExp, od, 0x04030402u);   // 5, 7
  return r;
}
// Eight bf16 activations in element order 0 … 7 -> 0, 2, 4, 6, 1, 3, 5, 7,
// the order of u4x8_to_bf16x8_biased's values.
MOE_DEV u32x4 bf16x8_even_odd(u32x4 a) {
  u32x4 r;
  r.x = __builtin_amdgcn_perm(a.y, a.x, 0x05040100u);   // low halves: 0, 2
  r.y = __builtin_amdgcn_perm(a.w, a.z, 0x05040100u);   // 4, 6
  r.z = __builtin_amdgcn_perm(a.y, a.x, 0x07060302u);   // high halves: 1, 3
  r.w = __builtin_amdgcn_perm(a.w, a.z, 0x07060302u);   // 5, 7
  return r;
}

// Full-line weight streaming for v_mfma_f32_16x16x32_bf16, whose B operand
// puts weight row i (of 16) in lanes i, i+16, i+32, i+48, each with 16 bytes
// (8 k): a load per MFMA therefore covers only 64 bytes of each row, half of
// every 128-byte line. Measured at the decode layout (12 KB rows), such
// half-line loads stream 5.9 TB/s cached and 4.9 TB/s nontemporal, while
// loads whose lanes cover whole lines reach 6.9 TB/s nontemporal. So a
// "double step" (128 bytes = 64 k of each of 16 rows) is read by two loads,
// load h covering rows 8h .. 8h+7 whole: lane (g, i) (g = lane / 16,
// i = lane % 16) reads row 8h + i % 8 at 16-byte chunk g when (i < 8) ==
// (h == 0), else at chunk 4 + g. The MFMA operand for the first 64 bytes
// (chunk g of row i) is the lane's own load h = (i >= 8); for the second 64
// bytes (chunk 4 + g) it is the other load of lane i ^ 8, a rotation by 8
// lanes within each 16-lane row (DPP row_ror:8).
MOE_DEV int dstep_chunk(int h, int i, int g) { return ((h == 0) == (i < 8)) ? g : 4 + g; }
MOE_DEV u32x4 row_ror8(u32x4 v) {
  u32x4 r;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    r[q] = (uint32_t)__builtin_amdgcn_mov_dpp((int)v[q], 0x128, 0xF, 0xF, false);
  return r;
}
// the two MFMA operands of a double step from its loads v0 (h = 0), v1 (h = 1)
MOE_DEV void dstep_operands(u32x4 v0, u32x4 v1, int i, u32x4& first, u32x4& second) {
  const bool lo = i < 8;
  first = lo ? v0 : v1;
  second = row_ror8(lo ? v1 : v0);
}
MOE_DEV u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
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
