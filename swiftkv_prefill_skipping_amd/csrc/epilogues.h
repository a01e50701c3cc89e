// GEMM epilogues.  Every GEMM in the library hands its results to an
// epilogue as column pairs (col, col + P) of one output row, so that the
// rotate-half RoPE pair (i, i + head_dim/2) and the interleaved SwiGLU pair
// (gate, up) meet in one thread.  P is the pair distance the producing GEMM
// was built for.
#pragma once
#include "common.h"

// Plain fp32 store (logits).
struct EpiStoreF32 {
  float* out;
  int ld;
  int P;
  SKV_DEV void operator()(int row, int col, float v0, float v1) const {
    out[(int64_t)row * ld + col] = v0;
    out[(int64_t)row * ld + col + P] = v1;
  }
};

// Plain store in the activation type (tests and intermediate buffers).
template <typename T>
struct EpiStore {
  T* out;
  int ld;
  int P;
  SKV_DEV void operator()(int row, int col, float v0, float v1) const {
    out[(int64_t)row * ld + col] = from_f32<T>(v0);
    out[(int64_t)row * ld + col + P] = from_f32<T>(v1);
  }
};

// Residual add into the fp32 residual stream: x += o W^T  (O and down projections).
struct EpiResidual {
  float* x;
  int ld;
  int P;
  SKV_DEV void operator()(int row, int col, float v0, float v1) const {
    float* p = x + (int64_t)row * ld + col;
    p[0] += v0;
    p[P] += v1;
  }
};

// SwiGLU on gate/up rows interleaved in blocks of P: GEMM column
// b*2P + c (c < P) is gate feature b*P + c, column b*2P + P + c is up
// feature b*P + c.  h = silu(gate) * up.
template <typename T>
struct EpiSwiGLU {
  T* h;
  int ld;
  int P;
  SKV_DEV void operator()(int row, int col, float g, float u) const {
    int blk = col / (2 * P);
    int c = col - blk * 2 * P;
    h[(int64_t)row * ld + blk * P + c] = from_f32<T>(silu_f(g) * u);
  }
};

SKV_DEV void rope_pair(float x0, float x1, float c, float s, float& y0, float& y1) {
  y0 = x0 * c - x1 * s;
  y1 = x1 * c + x0 * s;
}

// Q/K/V projection of an unskipped layer (or Q alone for the last-token
// path, where n_cols == dq).  Columns [0, dq) are query heads, [dq, dq+dkv)
// key heads, [dq+dkv, dq+2dkv) value heads.  RoPE rotates q and k at the
// token's position; q goes to a [rows, hq, dh] buffer, k and v into the
// paged cache slot of this layer.  P = dh / 2.
template <typename T>
struct EpiQKV {
  T* q;
  CacheSlot<T> cache;
  const int32_t* pos;
  const int32_t* slot;
  const float* rope_cos;  // [max_pos, P]
  const float* rope_sin;
  int dq, dkv, dh, P;
  SKV_DEV void operator()(int row, int col, float v0, float v1) const {
    if (col < dq) {
      int i = col % dh;
      int p = pos[row];
      float c = rope_cos[(int64_t)p * P + i], s = rope_sin[(int64_t)p * P + i];
      float y0, y1;
      rope_pair(v0, v1, c, s, y0, y1);
      T* qp = q + (int64_t)row * dq + col;
      qp[0] = from_f32<T>(y0);
      qp[P] = from_f32<T>(y1);
      return;
    }
    int sl = slot[row];
    if (sl < 0) return;
    if (col < dq + dkv) {
      int kc = col - dq, h = kc / dh, i = kc % dh;
      int p = pos[row];
      float c = rope_cos[(int64_t)p * P + i], s = rope_sin[(int64_t)p * P + i];
      float y0, y1;
      rope_pair(v0, v1, c, s, y0, y1);
      cache.k[kv_index(sl, h, i, cache.hkv, dh)] = from_f32<T>(y0);
      cache.k[kv_index(sl, h, i + P, cache.hkv, dh)] = from_f32<T>(y1);
    } else {
      int vc = col - dq - dkv, h = vc / dh, i = vc % dh;
      cache.v[kv_index(sl, h, i, cache.hkv, dh)] = from_f32<T>(v0);
      cache.v[kv_index(sl, h, i + P, cache.hkv, dh)] = from_f32<T>(v1);
    }
  }
};

// Skipped-layer KV (Eq. 2 / AcrossKV): column block g of width 2*dkv holds
// group g's folded K rows then V rows; K is rotated at the token position
// and written to slot (first_skip_slot + g), V likewise unrotated.
template <typename T>
struct EpiKVSkip {
  T* k0;  // K of the first skipped slot
  T* v0;
  int64_t slot_stride;  // elements between consecutive slots
  const int32_t* pos;
  const int32_t* slot;
  const float* rope_cos;
  const float* rope_sin;
  int dkv, dh, P, hkv;
  SKV_DEV void operator()(int row, int col, float a, float b) const {
    int sl = slot[row];
    if (sl < 0) return;
    int g = col / (2 * dkv);
    int c = col - g * 2 * dkv;
    if (c < dkv) {
      int h = c / dh, i = c % dh;
      int p = pos[row];
      float cs = rope_cos[(int64_t)p * P + i], sn = rope_sin[(int64_t)p * P + i];
      float y0, y1;
      rope_pair(a, b, cs, sn, y0, y1);
      T* kp = k0 + g * slot_stride;
      kp[kv_index(sl, h, i, hkv, dh)] = from_f32<T>(y0);
      kp[kv_index(sl, h, i + P, hkv, dh)] = from_f32<T>(y1);
    } else {
      int vc = c - dkv, h = vc / dh, i = vc % dh;
      T* vp = v0 + g * slot_stride;
      vp[kv_index(sl, h, i, hkv, dh)] = from_f32<T>(a);
      vp[kv_index(sl, h, i + P, hkv, dh)] = from_f32<T>(b);
    }
  }
};
