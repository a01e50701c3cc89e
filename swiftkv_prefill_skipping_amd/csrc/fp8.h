// Per-token FP8 KV cache: OCP E4M3 codes (sign, 4 exponent bits with bias
// 7, 3 mantissa bits; exponent 0 is subnormal, m * 2^-9; largest finite
// value 448) with one fp32 scale per token and KV slot, for K and V
// separately ("Complementarity with KV quantization", Appendix B.1 /
// Table B.1 of the SwiftKV paper: a per-token FP8 cache composed with
// AcrossKV).
//
// Quantisation of one token's K (or V) row over all kv heads:
//   scale = max|x| / 448,  code = E4M3(x * (1 / scale)) rounded to nearest
//   even, clamped to +-448 (a zero row: scale 0, codes 0).
// Each step is one fp32 operation (correctly rounded division and
// reciprocal, a lone product), so the integer code decisions are fixed by
// fp32 arithmetic.  Dequantisation: value = E4M3 value of the code * scale.
#pragma once
#include "common.h"

// One KV slot of the FP8 cache: codes in the [num_blocks, hkv, 16, dh]
// layout of CacheSlot; scales [num_blocks * 16] indexed by physical slot.
struct Fp8Slot {
  uint8_t* k;
  uint8_t* v;
  float* ks;
  float* vs;
  int hkv;
  int dh;
};

// E4M3 code -> fp32 value (exact), in vector ALU operations.  The NaN code
// is never produced by the quantiser and decodes as 480.
SKV_DEV float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15, m = c & 7;
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  return __uint_as_float(__float_as_uint(mag) | ((c & 0x80u) << 24));
}

// fp32 value with |y| <= 448 -> nearest E4M3 code, ties to even.
SKV_DEV uint32_t f32_to_e4m3(float y) {
  const uint32_t bits = __float_as_uint(y);
  const uint32_t s = (bits >> 24) & 0x80u;
  const float a = __uint_as_float(bits & 0x7fffffffu);
  if (a < 0x1p-6f) return s | (uint32_t)__builtin_rintf(a * 512.0f);  // subnormal steps; 8 = smallest normal
  int e = (int)((bits >> 23) & 255) - 127;                                // a is a normal fp32 here
  const uint32_t mant = bits & 0x7fffffu;
  uint32_t m = mant >> 20;
  const uint32_t rem = mant & 0xfffffu;
  m += (rem > 0x80000u || (rem == 0x80000u && (m & 1))) ? 1u : 0u;
  if (m == 8) {
    m = 0;
    ++e;
  }
  return s | ((uint32_t)(e + 7) << 3) | m;
}

// Four codes packed in a dword (byte b = code b) -> four floats through
// gfx950's hardware conversion (v_cvt_pk_f32_fp8: OCP E4M3, exact).
SKV_DEV void decode4_e4m3_hw(uint32_t w, float* out) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  out[0] = lo[0];
  out[1] = lo[1];
  out[2] = hi[0];
  out[3] = hi[1];
}

// 16 codes (one 16-byte load, element order preserved) -> 16 floats, with
// e4m3_to_f32 (the prompt attention's register-staged tiles keep fewer
// values live this way) or with the hardware conversion.
SKV_DEV void decode16_e4m3(u32x4_t w, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int b = 0; b < 4; ++b) out[4 * i + b] = e4m3_to_f32((w[i] >> (8 * b)) & 255u);
}
SKV_DEV void decode16_e4m3_hw(u32x4_t w, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) decode4_e4m3_hw(w[i], out + 4 * i);
}
