// Shared device helpers for the gfx950 SwiftKV kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // raw IEEE bfloat16 bits

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define SKV_DEV __device__ __forceinline__

SKV_DEV float bf16_to_f32(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16 with round to nearest even (NaN stays NaN): gfx950's
// v_cvt_pk_bf16_f32, two values per instruction.
SKV_DEV uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
SKV_DEV bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// Split-bf16 form of a float: hi = bf16(v) and lo = bf16(v - hi).  v - hi
// is exact in fp32, so hi + lo carries 16 significant bits of v; a bf16
// MFMA over both parts then sees the operand to about 2^-17 instead of
// 2^-9.
SKV_DEV float bf16_hi(float v) { return bf16_to_f32(f32_to_bf16(v)); }
SKV_DEV float bf16_lo_part(float v) { return v - bf16_hi(v); }

template <typename T>
SKV_DEV float to_f32(T v);
template <>
SKV_DEV float to_f32<float>(float v) { return v; }
template <>
SKV_DEV float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

template <typename T>
SKV_DEV T from_f32(float v);
template <>
SKV_DEV float from_f32<float>(float v) { return v; }
template <>
SKV_DEV bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

SKV_DEV bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// 16 loaded bytes -> 16 / sizeof(T) floats, element order preserved.
template <typename T>
SKV_DEV void unpack16(u32x4_t w, float* out);
template <>
SKV_DEV void unpack16<float>(u32x4_t w, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(w[i]);
}
template <>
SKV_DEV void unpack16<bf16_t>(u32x4_t w, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

SKV_DEV float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
SKV_DEV float warp_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// silu(x) = x / (1 + e^-x), with the hardware reciprocal (1 ulp)
SKV_DEV float silu_f(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// Per-token metadata of one prefill call, filled by the meta kernel.
struct TokenMeta {
  const int32_t* pos;   // [T] position of the token within its prompt
  const int32_t* slot;  // [T] physical cache slot = block * block_size + offset, -1 if unmapped
};

// Paged cache geometry of one KV slot (one layer or AcrossKV group).
// K and V share the layout [num_blocks, hkv, BS, dh]: a (token, head) row of
// dh values is contiguous, so GEMM epilogues write whole row segments.
template <typename T>
struct CacheSlot {
  T* k;
  T* v;
  int hkv;
  int dh;
};

constexpr int kBlockSize = 16;

// Panel layout of the bf16 GEMM operands (activations of the prompt-token
// path and the weights of unskipped layers): rows are grouped in panels of
// 256, and each panel is stored as consecutive blocks of 32 columns, each
// block [256 rows][32] contiguous (16 KB).  One k-stage of the GEMM is then
// one contiguous 16 KB block per operand.  K must be a multiple of 32; the
// row count is padded to a multiple of 256.
//
// The weights of the last-token path use the same layout with 64-row
// panels (kSkinnyPanelRows): a wave that owns 64 output columns then streams
// one contiguous run of its panel.
constexpr int kPanelRows = 256, kPanelCols = 32, kSkinnyPanelRows = 64;
SKV_DEV int64_t panel_off(int r, int k, int K) {
  return ((int64_t)(r >> 8) * (K >> 5) + (k >> 5)) * (kPanelRows * kPanelCols) + (r & 255) * kPanelCols + (k & 31);
}

// element index of (physical slot, head, dim) in one cache tensor
SKV_DEV int64_t kv_index(int slot_phys, int h, int d, int hkv, int dh) {
  int blk = slot_phys >> 4, off = slot_phys & 15;
  return (((int64_t)blk * hkv + h) * kBlockSize + off) * dh + d;
}
