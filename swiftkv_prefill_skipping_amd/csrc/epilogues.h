// GEMM epilogues.  Every GEMM in the library hands its results to an
// epilogue as column pairs (col, col + P) of one output row, so that the
// rotate-half RoPE pair (i, i + head_dim/2) and the interleaved SwiGLU pair
// (gate, up) meet in one thread.  P is the pair distance the producing GEMM
// was built for.
//
// Two entry points: operator()(row, col, v0, v1) takes one pair, and
// vec8(row, col, a, b) takes eight: a[e] is column col + e and b[e] column
// col + P + e (col % 8 == 0).  The bf16 MFMA GEMM uses vec8 so that every
// lane stores whole 16-byte runs.  An epilogue that reads the output it
// updates (the residual add) also offers pre8(row, col), which loads those
// values early, and vec8(row, col, a, b, pre), which consumes them.
//
// On gfx9 one vector-memory counter covers loads and stores, so a load
// issued after a store can only be waited for together with that store.
// The MFMA GEMM therefore reads everything its epilogue needs (per-row
// positions, cache slots and RMSNorm factors; RoPE tables; RMSNorm gains)
// before the stores it would otherwise queue behind: the epilogues offer
// those reads separately (row_info, rope_tab, gains8) and vec8 forms that
// take their results.
#pragma once
#include "common.h"

SKV_DEV void load8(const float* p, float* v) {
  const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(p);
  const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = x0[e];
    v[e + 4] = x1[e];
  }
}
SKV_DEV void store8(float* p, const float* v) {
  *reinterpret_cast<f32x4_t*>(p) = f32x4_t{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4_t*>(p + 4) = f32x4_t{v[4], v[5], v[6], v[7]};
}
SKV_DEV void store8(bf16_t* p, const float* v) {
  *reinterpret_cast<u32x4_t*>(p) =
      u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
}
// The low parts bf16(v - bf16(v)) of eight values (split-bf16 form).
SKV_DEV void store8_lo(bf16_t* p, const float* v) {
  float l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) l[e] = bf16_lo_part(v[e]);
  store8(p, l);
}

// Plain fp32 store (logits).
struct EpiStoreF32 {
  float* out;
  int ld;
  int P;
  SKV_DEV void operator()(int row, int col, float v0, float v1) const {
    out[(int64_t)row * ld + col] = v0;
    out[(int64_t)row * ld + col + P] = v1;
  }
  SKV_DEV void vec8(int row, int col, const float* a, const float* b) const {
    store8(out + (int64_t)row * ld + col, a);
    store8(out + (int64_t)row * ld + col + P, b);
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
  SKV_DEV void vec8(int row, int col, const float* a, const float* b) const {
    store8(out + (int64_t)row * ld + col, a);
    store8(out + (int64_t)row * ld + col + P, b);
  }
};

// Residual add into the fp32 residual stream: x += o W^T  (O and down projections).
// Optionally (act != NULL, vec8 only) it also hands the next projection its
// input: act = bf16(x * gain) of the new x in the panel layout (gain: the
// next RMSNorm's weights, NULL = 1), and ss = the sum of squares of each
// eight-pair unit's 16 new x values at [row * ld/16 + (col / 2P) * P/8 +
// (col % 2P) / 8], from which the row's RMSNorm factor is summed in fixed
// order.  The next projection multiplies its products by that factor, so it
// computes RMSNorm(x; gain) W^T with the weights exactly as given.
struct EpiResidual {
  float* x;
  int ld;
  int P;
  bf16_t* act = nullptr;
  float* ss = nullptr;
  const float* gain = nullptr;
  SKV_DEV void operator()(int row, int col, float v0, float v1) const {
    float* p = x + (int64_t)row * ld + col;
    p[0] += v0;
    p[P] += v1;
  }
  // the residual values of an eight-pair unit, loaded ahead of the sums
  struct Pre {
    float r0[8], r1[8];
  };
  SKV_DEV Pre pre8(int row, int col) const {
    Pre r;
    const float* p = x + (int64_t)row * ld + col;
    load8(p, r.r0);
    load8(p + P, r.r1);
    return r;
  }
  // the next RMSNorm's gains of the pair's columns (1 without a gain)
  SKV_DEV void gains8(int col, float* g0, float* g1) const {
    if (gain) {
      load8(gain + col, g0);
      load8(gain + col + P, g1);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) g0[e] = g1[e] = 1.0f;
    }
  }
  SKV_DEV void vec8(int row, int col, const float* a, const float* b, const Pre& r) const {
    float g0[8], g1[8];
    gains8(col, g0, g1);
    vec8g(row, col, a, b, r, g0, g1);
  }
  SKV_DEV void vec8g(int row, int col, const float* a, const float* b, const Pre& r, const float* g0,
                     const float* g1) const {
    float* p = x + (int64_t)row * ld + col;
    float y0[8], y1[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      y0[e] = r.r0[e] + a[e];
      y1[e] = r.r1[e] + b[e];
    }
    store8(p, y0);
    store8(p + P, y1);
    if (act) {
      float q = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) q += y0[e] * y0[e] + y1[e] * y1[e];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y0[e] *= g0[e];
        y1[e] *= g1[e];
      }
      store8(act + panel_off(row, col, ld), y0);
      store8(act + panel_off(row, col + P, ld), y1);
      // (the bf16 GEMM's pairs are 64 apart: shifts instead of a division)
      const int u = P == 64 ? ((col >> 7) << 3) + ((col & 127) >> 3) : (col / (2 * P)) * (P / 8) + (col % (2 * P)) / 8;
      ss[(int64_t)row * (ld / 16) + u] = q;
    }
  }
  SKV_DEV void vec8(int row, int col, const float* a, const float* b) const { vec8(row, col, a, b, pre8(row, col)); }
};

// Residual add for the skinny (row-major, at most 32 rows) products:
// x += o W^T on the column pair (col, col + 64), act = bf16(x * gain) of the
// new x in the same row-major layout (the next projection's input before
// its RMSNorm factor; gain = the next RMSNorm's weights, NULL = 1), and the
// pair's sum of squares of x handed back to the finalize pass, which
// reduces it over the wave's 128 columns.
struct EpiResidualRow {
  float* x;
  int ld;
  bf16_t* act;
  const float* gain = nullptr;
  SKV_DEV float operator()(int row, int col, float v0, float v1) const {
    float* p = x + (int64_t)row * ld + col;
    const float y0 = p[0] + v0, y1 = p[64] + v1;
    p[0] = y0;
    p[64] = y1;
    const float g0 = gain ? gain[col] : 1.0f, g1 = gain ? gain[col + 64] : 1.0f;
    bf16_t* a = act + (int64_t)row * ld + col;
    a[0] = from_f32<bf16_t>(y0 * g0);
    a[64] = from_f32<bf16_t>(y1 * g1);
    return y0 * y0 + y1 * y1;
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
  SKV_DEV void vec8(int row, int col, const float* g, const float* u) const {
    int blk = col / (2 * P);
    int c = col - blk * 2 * P;
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = silu_f(g[e]) * u[e];
    store8(h + (int64_t)row * ld + blk * P + c, y);
  }
};

// SwiGLU for the prompt-token GEMM: h is written in the panel layout
// (panel_off with F columns), where it is the A operand of the down
// projection.  Gate/up columns interleaved in blocks of P = 64 as in
// EpiSwiGLU (a compile-time distance: the column split is two bit
// operations).  rs (optional): per-row factor applied to gate and up first
// (the RMSNorm factor of an input that reached the GEMM un-normalised).
// With x = g*r: silu(x) * (u*r) = (g*u) * r^2 / (1 + 2^(g * (-r*log2 e))),
// one multiply fewer per output than evaluating silu(x) and u*r apart.
struct EpiSwiGLUPanel {
  static constexpr int P = 64;
  bf16_t* h;
  int F;
  const float* rs = nullptr;
  SKV_DEV float scale(int row) const { return rs ? rs[row] : 1.0f; }
  SKV_DEV void vec8(int row, int col, const float* g, const float* u) const { vec8s(row, col, g, u, scale(row)); }
  SKV_DEV void vec8s(int row, int col, const float* g, const float* u, float sr) const {
    const int oc = (col >> 7) * P + (col & (2 * P - 1));  // col = blk*2P + c, c < P -> blk*P + c
    const float ce = sr * -1.4426950408889634f;
    const float s2 = sr * sr;
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      y[e] = (g[e] * u[e]) * (s2 * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g[e] * ce)));
    store8(h + panel_off(row, oc, F), y);
  }
  // The GEMM hands this epilogue its gate/up pairs straight from the
  // accumulator registers, without staging them in LDS: lane group rg =
  // lane / 16 holds gate columns col + 4 rg .. +4 of two adjacent 16-column
  // blocks (g0 / g1, col and col + 16) of one row, and their up partners 64
  // columns on.  One permlane16 swap per packed dword trades values between
  // the groups of a pair (0 <-> 1, 2 <-> 3; both lanes hold the same row), so
  // group rg ends with eight consecutive outputs of block rg & 1, from
  // column 8 (rg >> 1) of it: one 16-byte store per lane instead of two of
  // 8 bytes, and each store instruction covers whole 64-byte panel rows.
  static constexpr bool kFromRegisters = true;
  SKV_DEV void vec4x2s(int row, int col, const float* g0, const float* u0, const float* g1, const float* u1, float sr,
                       int rg) const {
    const float ce = sr * -1.4426950408889634f;
    const float s2 = sr * sr;
    float y0[4], y1[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y0[e] = (g0[e] * u0[e]) * (s2 * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g0[e] * ce)));
      y1[e] = (g1[e] * u1[e]) * (s2 * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g1[e] * ce)));
    }
    const auto a = __builtin_amdgcn_permlane16_swap(pack_bf16x2(y0[0], y0[1]), pack_bf16x2(y1[0], y1[1]), false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(pack_bf16x2(y0[2], y0[3]), pack_bf16x2(y1[2], y1[3]), false, false);
    const int c = col + (rg & 1) * 16 + (rg >> 1) * 8;
    const int oc = (c >> 7) * P + (c & (2 * P - 1));
    *reinterpret_cast<u32x4_t*>(h + panel_off(row, oc, F)) = u32x4_t{a[0], b[0], a[1], b[1]};
  }
};

SKV_DEV void rope_pair(float x0, float x1, float c, float s, float& y0, float& y1) {
  y0 = x0 * c - x1 * s;
  y1 = x1 * c + x0 * s;
}

// Per-row values of the RoPE / KV-cache epilogues: the row's RMSNorm
// factor, position and cache slot.
struct RowInfo {
  float sr;
  int pos;
  int slot;
};

// Q/K/V projection of an unskipped layer (or Q alone for the last-token
// path, where n_cols == dq).  Columns [0, dq) are query heads, [dq, dq+dkv)
// key heads, [dq+dkv, dq+2dkv) value heads.  RoPE rotates q and k at the
// token's position; q goes to a [rows, hq, dh] buffer, k and v into the
// paged cache slot of this layer.  P = dh / 2.
//
// Optional split-bf16 low parts (bf16 only): q_lo receives bf16(q - bf16(q))
// in q's layout, k_lo / v_lo the same of k and v in the cache layout (a
// side buffer with the cache slot's geometry), for an attention that
// computes with both parts.
template <typename T>
struct EpiQKV {
  T* q;
  CacheSlot<T> cache;
  const int32_t* pos;
  const int32_t* slot;
  const float* rope_cos;  // [max_pos, P]
  const float* rope_sin;
  int dq, dkv, dh, P;
  const float* rs = nullptr;  // optional per-row factor (RMSNorm of an un-normalised input)
  T* q_lo = nullptr;
  T* k_lo = nullptr;
  T* v_lo = nullptr;
  static constexpr bool kSplit = sizeof(T) == 2;
  SKV_DEV void put(T* base, T* lo, int64_t i, float v) const {
    base[i] = from_f32<T>(v);
    if constexpr (kSplit)
      if (lo) lo[i] = from_f32<T>(bf16_lo_part(v));
  }
  SKV_DEV void operator()(int row, int col, float v0, float v1) const {
    if (rs) {
      v0 *= rs[row];
      v1 *= rs[row];
    }
    if (col < dq) {
      int i = col % dh;
      int p = pos[row];
      float c = rope_cos[(int64_t)p * P + i], s = rope_sin[(int64_t)p * P + i];
      float y0, y1;
      rope_pair(v0, v1, c, s, y0, y1);
      const int64_t qi = (int64_t)row * dq + col;
      put(q, q_lo, qi, y0);
      put(q, q_lo, qi + P, y1);
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
      put(cache.k, k_lo, kv_index(sl, h, i, cache.hkv, dh), y0);
      put(cache.k, k_lo, kv_index(sl, h, i + P, cache.hkv, dh), y1);
    } else {
      int vc = col - dq - dkv, h = vc / dh, i = vc % dh;
      put(cache.v, v_lo, kv_index(sl, h, i, cache.hkv, dh), v0);
      put(cache.v, v_lo, kv_index(sl, h, i + P, cache.hkv, dh), v1);
    }
  }
  SKV_DEV float scale(int row) const { return rs ? rs[row] : 1.0f; }
  SKV_DEV RowInfo row_info(int row) const { return RowInfo{scale(row), pos[row], slot[row]}; }
  // q and k columns are rotated; a pair's angle index is col % dh for both
  SKV_DEV bool roped(int col) const { return col < dq + dkv; }
  SKV_DEV void rope_tab(int p, int col, float* c, float* s) const {
    load8(rope_cos + (int64_t)p * P + col % dh, c);
    load8(rope_sin + (int64_t)p * P + col % dh, s);
  }
  SKV_DEV void vec8(int row, int col, const float* a_in, const float* b_in) const {
    const RowInfo ri = row_info(row);
    float c[8], s[8];
    if (roped(col)) rope_tab(ri.pos, col, c, s);
    vec8t(row, col, a_in, b_in, ri, c, s);
  }
  // c, s: the rotation of the pair's eight angles (q and k columns only)
  SKV_DEV void vec8t(int row, int col, const float* a_in, const float* b_in, const RowInfo& ri, const float* c,
                     const float* s) const {
    float a[8], b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = a_in[e] * ri.sr;
      b[e] = b_in[e] * ri.sr;
    }
    float y0[8], y1[8];
    if (col < dq) {
#pragma unroll
      for (int e = 0; e < 8; ++e) rope_pair(a[e], b[e], c[e], s[e], y0[e], y1[e]);
      const int64_t qi = (int64_t)row * dq + col;
      store8(q + qi, y0);
      store8(q + qi + P, y1);
      if constexpr (kSplit)
        if (q_lo) {
          store8_lo(q_lo + qi, y0);
          store8_lo(q_lo + qi + P, y1);
        }
      return;
    }
    const int sl = ri.slot;
    if (sl < 0) return;
    if (col < dq + dkv) {
      int kc = col - dq, h = kc / dh, i = kc % dh;
#pragma unroll
      for (int e = 0; e < 8; ++e) rope_pair(a[e], b[e], c[e], s[e], y0[e], y1[e]);
      const int64_t i0 = kv_index(sl, h, i, cache.hkv, dh), i1 = kv_index(sl, h, i + P, cache.hkv, dh);
      store8(cache.k + i0, y0);
      store8(cache.k + i1, y1);
      if constexpr (kSplit)
        if (k_lo) {
          store8_lo(k_lo + i0, y0);
          store8_lo(k_lo + i1, y1);
        }
    } else {
      int vc = col - dq - dkv, h = vc / dh, i = vc % dh;
      const int64_t i0 = kv_index(sl, h, i, cache.hkv, dh), i1 = kv_index(sl, h, i + P, cache.hkv, dh);
      store8(cache.v + i0, a);
      store8(cache.v + i1, b);
      if constexpr (kSplit)
        if (v_lo) {
          store8_lo(v_lo + i0, a);
          store8_lo(v_lo + i1, b);
        }
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
  const float* rs = nullptr;  // optional per-row factor (the row-rms of x_{l+1})
  SKV_DEV void operator()(int row, int col, float a, float b) const {
    int sl = slot[row];
    if (sl < 0) return;
    if (rs) {
      a *= rs[row];
      b *= rs[row];
    }
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
  SKV_DEV float scale(int row) const { return rs ? rs[row] : 1.0f; }
  SKV_DEV RowInfo row_info(int row) const { return RowInfo{scale(row), pos[row], slot[row]}; }
  // K columns are rotated; a pair's angle index is col % dh
  SKV_DEV bool roped(int col) const { return col % (2 * dkv) < dkv; }
  SKV_DEV void rope_tab(int p, int col, float* c, float* s) const {
    load8(rope_cos + (int64_t)p * P + col % dh, c);
    load8(rope_sin + (int64_t)p * P + col % dh, s);
  }
  SKV_DEV void vec8(int row, int col, const float* a_in, const float* b_in) const {
    const RowInfo ri = row_info(row);
    float c[8], s[8];
    if (roped(col)) rope_tab(ri.pos, col, c, s);
    vec8t(row, col, a_in, b_in, ri, c, s);
  }
  SKV_DEV void vec8t(int row, int col, const float* a_in, const float* b_in, const RowInfo& ri, const float* cs,
                     const float* sn) const {
    const int sl = ri.slot;
    if (sl < 0) return;
    float a[8], b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = a_in[e] * ri.sr;
      b[e] = b_in[e] * ri.sr;
    }
    int g = col / (2 * dkv);
    int c = col - g * 2 * dkv;
    if (c < dkv) {
      int h = c / dh, i = c % dh;
      float y0[8], y1[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) rope_pair(a[e], b[e], cs[e], sn[e], y0[e], y1[e]);
      T* kp = k0 + g * slot_stride;
      store8(kp + kv_index(sl, h, i, hkv, dh), y0);
      store8(kp + kv_index(sl, h, i + P, hkv, dh), y1);
    } else {
      int vc = c - dkv, h = vc / dh, i = vc % dh;
      T* vp = v0 + g * slot_stride;
      store8(vp + kv_index(sl, h, i, hkv, dh), a);
      store8(vp + kv_index(sl, h, i + P, hkv, dh), b);
    }
  }
};
