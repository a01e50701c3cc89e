// Attention kernels.
//
// 1. attn_prefill8_kernel (bf16, MFMA): causal GQA flash attention of the
//    prompt tokens of layers 1..l, reading K/V from the paged cache.  A
//    sequence's new tokens may follow positions already cached (a prompt
//    chunk, a decode token): they attend to those as well as to each other.
//    A workgroup = 8 wave64s = 4 query heads of one kv-head group x two
//    32-query blocks of one prompt (64 queries).  Per 64-key tile:
//      S^T (keys x queries) = K Q^T   with A = K from LDS, B = Q^T from
//                                     registers (v_mfma_f32_32x32x16_bf16);
//      each lane then owns one query column, so the online-softmax max and
//      sum need only the lane's own 32 scores plus one exchange with lane^32;
//      O^T (dims x queries) += V^T P^T with B = P^T taken straight from the
//      score registers (rounded to bf16) and A = V^T read from the
//      token-major V tile with ds_read_b64_tr_b16 (gfx950's transposing LDS
//      read: within 16 lanes, lane j receives element j%4 of the rows
//      addressed by lanes 4e+j/4, e = 0..3).
//    The score accumulator holds, in lane half h and element e of 16-key
//    step kk, key kk*16 + 8*(e/4) + 4*h + e%4; the V^T reads gather the same
//    keys, so both operands agree.  K and V tiles share one LDS layout
//    ([64 keys][128 dims], 16-byte chunk c of key row r at c ^ kv_swz(r)).
//    O^T is transposed through LDS at the end and written 8 bytes per lane
//    into the panel layout of the O projection's A operand.
//    K/V tiles move global -> LDS directly (global_load_lds_dwordx4) into
//    two-stage rings (64 KB); the block ids of the next tiles are fetched
//    one iteration ahead.  Keys past the prompt (or causally masked) get
//    probability exactly 0, so the cache contents loaded for them only need
//    to be finite, which the cache guarantees (zero-filled at creation,
//    written only with results).  One workgroup per CU (256 VGPRs per wave).
//
//    With a per-token FP8 cache the tiles move through registers instead and
//    are dequantised (code * the key's scale, rounded to bf16) on the way
//    into the same LDS layout.
//
// 2. attn_rows_kernel / attn_dec_kernel + attn_combine_kernel (vector
//    ALU): attention of an explicit list of query rows (the last prompt
//    token of each prompt at layers l+1..L, decode rows; every token for
//    fp32 models), split over key chunks (64 keys for bf16 rows of head_dim
//    128, 256 otherwise) with a fixed-order combine.  attn_dec1_kernel does
//    the same for bf16 rows of contexts up to 1024 keys in one launch, the
//    chunks of a row and kv head combined inside one workgroup.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef s16x4_t short4_lds_t;

constexpr int FA_DH = 128;
constexpr int FA_KT = 64;  // keys per tile

// Physical 16-byte chunk of logical chunk c in key row r of a K/V tile:
// c ^ kv_swz(r), kv_swz swapping the two 2-bit halves of r & 15.  A phase
// of the score reads (sixteen consecutive keys at one chunk) covers all
// sixteen chunk positions, and so does a phase of the transposing P.V reads
// (four consecutive keys times four consecutive chunks), so neither read
// conflicts on the banks.
SKV_DEV int kv_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }


// x combined with lane (l ^ 32)'s value through gfx950's v_permlane32_swap:
// the swap leaves lane l holding (value of lane l & 31, value of lane l | 32),
// so both halves see the pair in the same order
SKV_DEV float xor32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
SKV_DEV float xor32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

SKV_DEV float xor16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
template <int CTRL>
SKV_DEV float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// x + (value of lane l ^ off) without going through LDS: DPP within a row of
// 16 lanes (quad permutes for 1 and 2, row rotate by 8 for 8) and the
// gfx950 permlane swaps across rows.  uniform4: lanes already agree within
// aligned groups of 4 (a butterfly that started at 1), so the half-row
// mirror stands in for xor 4.
SKV_DEV float xor_add(float x, int off, bool uniform4) {
  switch (off) {
    case 1: return x + dpp_f<0xB1>(x);
    case 2: return x + dpp_f<0x4E>(x);
    case 4: return uniform4 ? x + dpp_f<0x141>(x) : x + __shfl_xor(x, 4, 64);
    case 8: return x + dpp_f<0x128>(x);
    case 16: return xor16_sum(x);
    case 32: return xor32_sum(x);
    default: return x + __shfl_xor(x, off, 64);
  }
}

// Whole-wave max / sum through the same DPP and permlane steps (offsets
// 1, 2, 4, 8, 16, 32); every lane ends with the result.
SKV_DEV float wave_max_x(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x128>(v));
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  return xor32_max(v);
}
SKV_DEV float wave_sum_x(float v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v = xor_add(v, off, true);
  return v;
}

// Transposing LDS read (ds_read_b64_tr_b16) through a restrict-qualified
// pointer.  The alias scope the qualifier gives the access lets the
// compiler's wait insertion see that the read does not touch the ring
// buffers the direct-to-LDS loads in flight are filling; through a plain
// pointer it waits for every such load (vmcnt(0)) before the first read.
// The kernel's own barrier waits publish each tile before it is read.
SKV_DEV s16x4_t lds_read_tr(const bf16_t* __restrict__ p) {
  typedef __attribute__((address_space(3))) short4_lds_t* lds_s4p;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4p)(p));
}

SKV_DEV void wait_loads_then_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Prefill attention: one workgroup = the 4 q heads of one kv group x 64
// queries (two 32-query blocks, 8 waves, two per SIMD), so every K/V tile is
// loaded once for 8 waves.  K and V move through two-stage rings; within a
// wave the score MFMAs of tile t+1 are issued before the softmax of tile t,
// so the vector ALU work of one tile overlaps the matrix-core work of the
// next.
//
// SPLIT: q, K and V come in split-bf16 form (hi + lo parts, see bf16_hi):
// scores = q_hi.k_hi + q_hi.k_lo + q_lo.k_hi and O += P_hi.V_hi + P_hi.V_lo
// + P_lo.V_hi (the lo.lo products are below 2^-16 of the result), three
// MFMAs for each one of the plain kernel; the output is written in split
// form too.
template <bool SPLIT>
SKV_DEV void f8_qk(const bf16_t* sk, const bf16_t* sk_lo, const bf16x8_t* qf, const bf16x8_t* qf_lo, int lane,
                   f32x16_t* sacc) {
  const int hh = lane >> 5;
  sacc[0] = sacc[1] = f32x16_t{0};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const int ch = ks * 2 + hh;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int key = st * 32 + (lane & 31);
      bf16x8_t kf = as_bf16x8(*reinterpret_cast<const u32x4_t*>(sk + key * FA_DH + ((ch ^ kv_swz(key)) << 3)));
      sacc[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc[st], 0, 0, 0);
      if constexpr (SPLIT) {
        const int off = key * FA_DH + ((ch ^ kv_swz(key)) << 3);
        bf16x8_t kl = as_bf16x8(*reinterpret_cast<const u32x4_t*>(sk_lo + off));
        sacc[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kl, qf[ks], sacc[st], 0, 0, 0);
        sacc[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf_lo[ks], sacc[st], 0, 0, 0);
      }
    }
  }
}

// F8: K/V tiles come from the per-token FP8 cache c8 and move through
// registers: each thread fetches 16 codes of one key and its scale, and
// writes code * scale as bf16 into the same LDS layout the direct loads
// produce; everything after the tile loads is shared.
template <bool F8, bool SPLIT, int NW = 8>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_prefill8_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ q_lo, CacheSlot<bf16_t> cache, CacheSlot<bf16_t> lo,
    Fp8Slot c8, const int32_t* __restrict__ cu, const int32_t* __restrict__ ctx, const int32_t* __restrict__ bt,
    int max_blocks, int hq, int rep, float scale_log2, bf16_t* __restrict__ o) {
  static_assert(!(F8 && SPLIT), "the FP8 cache has no split form");
  // buffers 0, 1: K ring; 2, 3: V ring ([64 keys][128 dims] each); SPLIT:
  // 4, 5 and 6, 7 the same for the low parts.  The first 64 KB stage the
  // output at the end (SPLIT: the low parts in the next 64 KB)
  __shared__ __attribute__((aligned(1024))) bf16_t smem[SPLIT ? 8 : 4][FA_KT * FA_DH];

  // grid: x = (prompt, head group), y = query tile counted from the last, so
  // workgroups are dispatched longest first across the whole batch
  const int ngrp = hq / 4;
  const int b = blockIdx.x / ngrp;
  const int zg = blockIdx.x - b * ngrp;
  const int tok0 = cu[b];
  const int N = cu[b + 1] - tok0;  // new queries, at positions C .. C + N - 1
  const int C = ctx ? ctx[b] : 0;  // positions cached before them
  const int NK = C + N;            // keys
  static_assert(NW == 8 || (NW == 4 && !F8 && !SPLIT), "the 4-wave form serves the plain bf16 cache");
  constexpr int QT = NW * 8;  // queries per workgroup
  const int nqb = (N + QT - 1) / QT;
  const int qb = gridDim.y - 1 - blockIdx.y;
  if (qb >= nqb) return;
  const int q0w = qb * QT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5;
  const int h = zg * 4 + (wave & 3);
  const int q0 = q0w + (wave >> 2) * 32;  // this wave's 32 queries
  const int g = (zg * 4) / rep;
  const int hkv = cache.hkv;
  const int dq = hq * FA_DH;

  const int kend = min(NK, C + q0w + QT);
  const int ntiles = (kend + FA_KT - 1) / FA_KT;
  const int nblk_need = (kend + kBlockSize - 1) / kBlockSize;
  const int32_t* btb = bt + (int64_t)b * max_blocks;

  bf16x8_t qf[8], qf_lo[SPLIT ? 8 : 1];
  {
    const int qi = min(q0 + (lane & 31), N - 1);
    const int64_t qo = (int64_t)(tok0 + qi) * dq + h * FA_DH + hh * 8;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(q + qo + ks * 16));
    if constexpr (SPLIT) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qf_lo[ks] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(q_lo + qo + ks * 16));
    }
  }

  // Tile loads: wave w moves 16-key block r = w/2, key rows (w%2)*8 .. +8
  // of it, for K and for V (two 1 KB instructions each).  Lane l's 16 bytes
  // land at tile row (instruction base + l/16), physical chunk l%16, so it
  // fetches logical chunk (l%16) ^ (row & 15).  Entries past the keys this
  // workgroup needs read block 0, a valid block of the prompt.
  // (4 waves: wave w moves all 16 rows of block w, four instructions each.)
  constexpr int NLI = NW == 8 ? 2 : 4;  // load instructions per wave per K or V tile
  const int r_blk = NW == 8 ? wave >> 1 : wave;
  const int row0 = NW == 8 ? (wave & 1) * 8 : 0;
  // key row row0 + i*4 + lane/16 has kv_swz = ((lane/16) & 3) << 2 | (row0/4 + i) & 3
  const int src_base = (row0 + (lane >> 4)) * FA_DH;
  const int src_chunk = (lane & 15) ^ (((lane >> 4) & 3) << 2);
  auto src_off = [&](int i) { return src_base + i * 4 * FA_DH + ((src_chunk ^ ((row0 / 4 + i) & 3)) << 3); };
  auto block_of = [&](int t) {
    const int bi = t * (FA_KT / kBlockSize) + r_blk;
    return btb[bi < nblk_need ? bi : 0];
  };
  // FP8 tiles: thread tid moves key fk = tid / 8 of the tile (block row
  // r_blk, as above), dims fq * 16 .. + 16: two 16-byte bf16 chunks after
  // dequantisation, placed at the swizzled chunk positions
  const int fk = tid >> 3, fq = tid & 7;
  auto fetch8 = [&](const uint8_t* codes, const float* scales, int blk, u32x4_t& w, float& sc) {
    const int64_t row = ((int64_t)blk * hkv + g) * kBlockSize + (fk & 15);
    w = *reinterpret_cast<const u32x4_t*>(codes + row * FA_DH + fq * 16);
    sc = scales[(int64_t)blk * kBlockSize + (fk & 15)];
  };
  auto store8 = [&](const u32x4_t& w, float sc, int buf) {
    float x[16];
    decode16_e4m3(w, x);
    u32x4_t lo, hi;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo[e] = pack_bf16x2(x[2 * e] * sc, x[2 * e + 1] * sc);
      hi[e] = pack_bf16x2(x[8 + 2 * e] * sc, x[8 + 2 * e + 1] * sc);
    }
    bf16_t* row = &smem[buf][fk * FA_DH];
    *reinterpret_cast<u32x4_t*>(row + (((2 * fq) ^ kv_swz(fk)) << 3)) = lo;
    *reinterpret_cast<u32x4_t*>(row + (((2 * fq + 1) ^ kv_swz(fk)) << 3)) = hi;
  };
  auto issue = [&](const bf16_t* base_ptr, int blk, int buf) {
    const bf16_t* src = base_ptr + ((int64_t)blk * hkv + g) * (kBlockSize * FA_DH);
    typedef __attribute__((address_space(3))) void* lds_ptr;
#pragma unroll
    for (int i = 0; i < NLI; ++i) {
      const bf16_t* sp = src + src_off(i);
      __builtin_amdgcn_global_load_lds(sp, (lds_ptr)(&smem[buf][(r_blk * 16 + row0 + i * 4) * FA_DH]), 16, 0,
                                       0);
    }
  };

  f32x16_t oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16_t{0};
  float m_run = -INFINITY, l_run = 0.f;
  constexpr float kLazy = 8.0f;

  // Softmax of tile t in two parts.  Scores stay raw; the scale c =
  // log2(e)/sqrt(dh) enters the exponent, p = 2^(c*s - m).  The running
  // offset m only moves when a column's tile maximum exceeds it by more than
  // kLazy (then every column of the wave rescales); otherwise p <= 2^kLazy,
  // which fp32 sums and bf16 probabilities hold exactly as well.
  // softmax(s) does not depend on the offset, so this is the same function;
  // it saves the rescale of the output accumulators on most tiles.
  // soft_prep masks (diagonal / prompt-end tiles only), takes the column
  // maxima and moves the offset if needed; exp_pv turns the scores into bf16
  // probabilities and accumulates O^T += V^T P^T from V buffer vb.  Only
  // soft_prep branches, so exp_pv and the next tile's score MFMAs form one
  // straight block the scheduler can interleave.
  auto soft_prep = [&](int t, f32x16_t* sacc) {
    const int k0 = t * FA_KT;
    const int qi = C + q0 + (lane & 31);  // the column's position
    if ((k0 + FA_KT - 1 > C + q0) || (k0 + FA_KT > NK)) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = k0 + st * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
          if (key > qi || key >= NK) sacc[st][v] = -INFINITY;
        }
    }
    float mt = sacc[0][0];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int v = 0; v < 16; ++v) mt = fmaxf(mt, sacc[st][v]);
    mt = xor32_max(mt) * scale_log2;
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kLazy) != 0) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[dt][v] *= alpha;
    }
  };
  auto exp_pv = [&](const f32x16_t* sacc, int vb) {
    const float mneg = -m_run;
    float ls = 0.f;
    bf16x8_t pf[4], pf_lo[SPLIT ? 4 : 1];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int st = kk >> 1, vb8 = 8 * (kk & 1);
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(fmaf(sacc[st][vb8 + e], scale_log2, mneg));
        if constexpr (SPLIT) ls += p[e];
      }
      pf[kk] = as_bf16x8(u32x4_t{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                                 pack_bf16x2(p[6], p[7])});
      if constexpr (SPLIT) {
        float pl[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pl[e] = bf16_lo_part(p[e]);
        pf_lo[kk] = as_bf16x8(u32x4_t{pack_bf16x2(pl[0], pl[1]), pack_bf16x2(pl[2], pl[3]), pack_bf16x2(pl[4], pl[5]),
                                      pack_bf16x2(pl[6], pl[7])});
      }
    }
    if constexpr (!SPLIT) {
      // The row sum of the bf16 probabilities the P.V products use, two per
      // v_dot2_f32_bf16 against (1, 1): half the vector instructions of a
      // sum over the fp32 values, and the normaliser then matches the
      // weights exactly.  Two chains keep the dependent adds apart.
      const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};
      float l2[2] = {0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8_t v = pf[kk];
        l2[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one2, l2[0], false);
        l2[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one2, l2[1], false);
        l2[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one2, l2[0], false);
        l2[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one2, l2[1], false);
      }
      ls = l2[0] + l2[1];
    }
    ls = xor32_sum(ls);
    l_run += ls;
    const bf16_t* sv = smem[2 + vb];
    const bf16_t* sv_lo = smem[SPLIT ? 6 + vb : 2 + vb];
    const int tj = lane & 15, ta = tj >> 2, tb = tj & 3;
    // key steps outer, dims inner: consecutive MFMAs feed four independent
    // accumulators
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int d = dt * 32 + 16 * ((lane >> 4) & 1) + 4 * tb;
        const int k1 = kk * 16 + 4 * hh + ta, k2 = k1 + 8;
        s16x4_t lo = lds_read_tr(sv + k1 * FA_DH + (((d >> 3) ^ kv_swz(k1)) << 3) + (d & 7));
        s16x4_t hi = lds_read_tr(sv + k2 * FA_DH + (((d >> 3) ^ kv_swz(k2)) << 3) + (d & 7));
        u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo), hi2 = __builtin_bit_cast(u32x2_t, hi);
        bf16x8_t vf = as_bf16x8(u32x4_t{lo2.x, lo2.y, hi2.x, hi2.y});
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kk], oacc[dt], 0, 0, 0);
        if constexpr (SPLIT) {
          const int o1 = k1 * FA_DH + (((d >> 3) ^ kv_swz(k1)) << 3) + (d & 7);
          const int o2 = k2 * FA_DH + (((d >> 3) ^ kv_swz(k2)) << 3) + (d & 7);
          s16x4_t llo = lds_read_tr(sv_lo + o1);
          s16x4_t lhi = lds_read_tr(sv_lo + o2);
          u32x2_t a2 = __builtin_bit_cast(u32x2_t, llo), b2 = __builtin_bit_cast(u32x2_t, lhi);
          bf16x8_t vl = as_bf16x8(u32x4_t{a2.x, a2.y, b2.x, b2.y});
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vl, pf[kk], oacc[dt], 0, 0, 0);
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf_lo[kk], oacc[dt], 0, 0, 0);
        }
      }
    }
  };

  // Pipeline.  Iteration t < ntiles - 1: loads of K(t+2) (into the buffer
  // K(t) used) and V(t+1) (into V(t-1)'s) go out; the scores of tile t+1
  // are computed from K(t+1) (landed at the end of iteration t-1) while the
  // softmax and P.V of tile t run; then every wave waits for its loads and
  // the workgroup synchronises.  Loads for tiles past the end read block 0
  // of the prompt (in bounds, unused), so they need no branch.  The last
  // tile only runs its softmax and P.V.  Stage parity is unrolled so the two
  // score accumulators stay in registers.
  // blk1 / blk2: block ids of tiles t+1 / t+2, fetched one iteration ahead
  // so no load waits on a block-table read
  if constexpr (SPLIT) {
    // Split form: one tile at a time (the extra q / P parts leave no
    // registers for the next tile's scores).  Iteration t waits for tile t,
    // then loads tile t + 1 into the buffers tile t - 1 used while it
    // computes tile t.
    auto issue_tile = [&](int t) {
      const int blk = block_of(t);
      issue(cache.k, blk, t & 1);
      issue(cache.v, blk, 2 + (t & 1));
      issue(lo.k, blk, 4 + (t & 1));
      issue(lo.v, blk, 6 + (t & 1));
    };
    issue_tile(0);
    for (int t = 0; t < ntiles; ++t) {
      wait_loads_then_barrier();
      if (t + 1 < ntiles) issue_tile(t + 1);
      f32x16_t sa[2];
      f8_qk<true>(smem[t & 1], smem[4 + (t & 1)], qf, qf_lo, lane, sa);
      soft_prep(t, sa);
      exp_pv(sa, t & 1);
    }
  } else {
    int blk1 = block_of(1), blk2 = block_of(2);
    u32x4_t wk, wv;  // FP8: codes of K(t+2) / V(t+1) in flight through registers
    float sk, sv;
    if constexpr (F8) {
      const int blk0 = block_of(0);
      fetch8(c8.k, c8.ks, blk0, wk, sk);
      fetch8(c8.v, c8.vs, blk0, wv, sv);
      store8(wk, sk, 0);
      store8(wv, sv, 2);
      fetch8(c8.k, c8.ks, blk1, wk, sk);
      store8(wk, sk, 1);
    } else {
      issue(cache.k, block_of(0), 0);
      issue(cache.v, block_of(0), 2);
      issue(cache.k, blk1, 1);
    }
    wait_loads_then_barrier();
    f32x16_t sa[2], sb[2];
    f8_qk<false>(smem[0], smem[0], qf, qf_lo, lane, sa);
    wait_loads_then_barrier();  // every wave has read K(0) before its buffer takes K(2)
    auto full = [&](int t, f32x16_t* cur, f32x16_t* nxt) {
      const int blk3 = block_of(t + 3);
      if constexpr (F8) {
        fetch8(c8.k, c8.ks, blk2, wk, sk);
        fetch8(c8.v, c8.vs, blk1, wv, sv);
      } else {
        issue(cache.k, blk2, t & 1);
        issue(cache.v, blk1, 2 + ((t + 1) & 1));
      }
      soft_prep(t, cur);
      f8_qk<false>(smem[(t + 1) & 1], smem[0], qf, qf_lo, lane, nxt);
      exp_pv(cur, t & 1);
      if constexpr (F8) {
        // K(t) and V(t-1), whose buffers these take, were last read in the
        // previous iteration
        store8(wk, sk, t & 1);
        store8(wv, sv, 2 + ((t + 1) & 1));
      }
      wait_loads_then_barrier();
      blk1 = blk2;
      blk2 = blk3;
    };
    auto last = [&](int t, f32x16_t* cur) {
      soft_prep(t, cur);
      exp_pv(cur, t & 1);
    };
    const int n1 = ntiles - 1;  // iterations that also compute the next tile's scores
    int t = 0;
    for (; t + 1 < n1; t += 2) {
      full(t, sa, sb);
      full(t + 1, sb, sa);
    }
    if (t < n1) {
      full(t, sa, sb);
      last(t + 1, sb);
    } else {
      last(t, sa);
    }
  }
  wait_loads_then_barrier();  // all P.V reads done before the buffers stage the output

  // normalise and write: O^T -> LDS [32 q][128 d] per wave (8-byte quads
  // swizzled by q) -> panel rows (a row's 128 dims are four 64-byte runs)
  bf16_t* so = &smem[0][0] + wave * (32 * FA_DH);
  bf16_t* so_lo = &smem[0][0] + (SPLIT ? 4 * FA_KT * FA_DH : 0) + wave * (32 * FA_DH);
  {
    const float inv = 1.0f / l_run;
    const int ql = lane & 31;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        const int u = dt * 8 + vq * 2 + hh;
        u32x2_t w;
        w.x = pack_bf16x2(oacc[dt][vq * 4 + 0] * inv, oacc[dt][vq * 4 + 1] * inv);
        w.y = pack_bf16x2(oacc[dt][vq * 4 + 2] * inv, oacc[dt][vq * 4 + 3] * inv);
        *reinterpret_cast<u32x2_t*>(so + ql * FA_DH + ((u ^ ql) << 2)) = w;
        if constexpr (SPLIT) {
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = oacc[dt][vq * 4 + e] * inv;
          u32x2_t wl;
          wl.x = pack_bf16x2(bf16_lo_part(y[0]), bf16_lo_part(y[1]));
          wl.y = pack_bf16x2(bf16_lo_part(y[2]), bf16_lo_part(y[3]));
          *reinterpret_cast<u32x2_t*>(so_lo + ql * FA_DH + ((u ^ ql) << 2)) = wl;
        }
      }
  }
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  // SPLIT: o has 2 dq columns, hi at column c and lo at column dq + c
  const int ocols = SPLIT ? 2 * dq : dq;
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const int idx = it * 64 + lane;
    const int ql2 = idx >> 5, u = idx & 31;
    const int qi = q0 + ql2;
    if (qi < N) {
      u32x2_t w = *reinterpret_cast<const u32x2_t*>(so + ql2 * FA_DH + ((u ^ ql2) << 2));
      *reinterpret_cast<u32x2_t*>(o + panel_off(tok0 + qi, h * FA_DH + u * 4, ocols)) = w;
      if constexpr (SPLIT) {
        u32x2_t wl = *reinterpret_cast<const u32x2_t*>(so_lo + ql2 * FA_DH + ((u ^ ql2) << 2));
        *reinterpret_cast<u32x2_t*>(o + panel_off(tok0 + qi, dq + h * FA_DH + u * 4, ocols)) = wl;
      }
    }
  }
}

constexpr int RW_CH = 256;     // keys per chunk (one workgroup, 4 waves x 64 keys)
constexpr int RW_MAXREP = 16;  // q heads per kv head
constexpr int RW_MAXDH = 128;
constexpr int RW_HG = 4;       // q heads handled per pass over the chunk

// One query row (a token with its position and prompt) against one kv head's
// keys [c*256, c*256+256) of that prompt, for the rep q heads that share the
// kv head.  Writes (max, sum, unnormalised o) per head for the combine pass.
// Lanes read key and value rows as 16-byte slices: LPK lanes cover one row
// (DH elements), so one wave load instruction covers 64/LPK whole rows.
// F8: K/V come from the per-token FP8 cache c8 (codes times the token's
// scale, in fp32); otherwise from `cache` in the activation type.
template <typename T, int DH, bool F8>
__global__ __launch_bounds__(256) void attn_rows_kernel(const T* __restrict__ q, CacheSlot<T> cache, Fp8Slot c8,
                                                        const int32_t* __restrict__ row_seq,
                                                        const int32_t* __restrict__ row_pos,
                                                        const int32_t* __restrict__ bt, int max_blocks, int hq,
                                                        int nchunks, float scale, float* __restrict__ ws) {
  constexpr int VEC = F8 ? 16 : 16 / (int)sizeof(T);  // elements per lane load
  constexpr int LPK = DH / VEC;             // lanes per key row
  constexpr int KPI = 64 / LPK;             // key rows per wave load
  constexpr int ITERS = 64 / KPI;           // loads per wave per chunk
  static_assert(LPK >= 1 && LPK <= 64 && 64 % LPK == 0, "head_dim / vector width");
  __shared__ float qs[RW_MAXREP][DH];
  __shared__ float ps[RW_HG][RW_CH];
  __shared__ int sl_s[RW_CH];
  __shared__ float red[RW_HG][4];
  __shared__ float opart[4][RW_HG][DH];

  const int r = blockIdx.x, g = blockIdx.y, c = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hkv = cache.hkv;
  const int rep = hq / hkv;
  const int ctx = row_pos[r] + 1;
  const int seq = row_seq[r];
  const int kbeg = c * RW_CH;
  const int stride = DH + 2;
  float* wsr = ws + ((int64_t)r * hq + g * rep) * nchunks * stride;

  if (kbeg >= ctx) {  // empty chunk
    for (int hl = tid; hl < rep; hl += 256) {
      float* o = wsr + ((int64_t)hl * nchunks + c) * stride;
      o[0] = -INFINITY;
      o[1] = 0.f;
    }
    return;
  }
  for (int i = tid; i < rep * DH; i += 256) {
    int hl = i / DH, d = i % DH;
    qs[hl][d] = to_f32<T>(q[((int64_t)r * hq + g * rep + hl) * DH + d]);
  }
  {
    const int key = kbeg + tid;
    int sl = -1;
    if (key < ctx) sl = bt[(int64_t)seq * max_blocks + key / kBlockSize] * kBlockSize + key % kBlockSize;
    sl_s[tid] = sl;
  }
  __syncthreads();

  const int nk = min(RW_CH, ctx - kbeg);
  const int sub = lane / LPK;          // key row within one wave load
  const int d0 = (lane % LPK) * VEC;   // first element of this lane's slice
  const int kw = w * 64;               // this wave's first key within the chunk

  for (int h0 = 0; h0 < rep; h0 += RW_HG) {
    // ---- scores s[h][key] for heads h0..h0+3
#pragma unroll 4
    for (int it = 0; it < ITERS; ++it) {
      const int kk = kw + it * KPI + sub;
      float part[RW_HG];
#pragma unroll
      for (int hh = 0; hh < RW_HG; ++hh) part[hh] = 0.f;
      if (kk < nk) {
        float kv[VEC];
        if constexpr (F8) {
          const int sl = sl_s[kk];
          decode16_e4m3(*reinterpret_cast<const u32x4_t*>(c8.k + kv_index(sl, g, d0, hkv, DH)), kv);
          const float sc = c8.ks[sl];
#pragma unroll
          for (int e = 0; e < VEC; ++e) kv[e] *= sc;
        } else {
          unpack16<T>(*reinterpret_cast<const u32x4_t*>(cache.k + kv_index(sl_s[kk], g, d0, hkv, DH)), kv);
        }
#pragma unroll
        for (int hh = 0; hh < RW_HG; ++hh) {
          if (h0 + hh < rep) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) part[hh] = fmaf(qs[h0 + hh][d0 + e], kv[e], part[hh]);
          }
        }
      }
#pragma unroll
      for (int hh = 0; hh < RW_HG; ++hh) {
#pragma unroll
        for (int off = 1; off < LPK; off <<= 1) part[hh] = xor_add(part[hh], off, true);
      }
      if (lane % LPK == 0) {
#pragma unroll
        for (int hh = 0; hh < RW_HG; ++hh) ps[hh][kk] = kk < nk ? part[hh] * scale : -INFINITY;
      }
    }
    __syncthreads();

    // ---- softmax statistics over the chunk; thread t owns key t
    float mh[RW_HG];
#pragma unroll
    for (int hh = 0; hh < RW_HG; ++hh) {
      float m = wave_max_x(ps[hh][tid]);
      if (lane == 0) red[hh][w] = m;
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < RW_HG; ++hh) mh[hh] = fmaxf(fmaxf(red[hh][0], red[hh][1]), fmaxf(red[hh][2], red[hh][3]));
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < RW_HG; ++hh) {
      const float x = ps[hh][tid];
      const float p = x == -INFINITY ? 0.f : __expf(x - mh[hh]);
      ps[hh][tid] = p;
      const float sm = wave_sum_x(p);
      if (lane == 0) red[hh][w] = sm;
    }
    __syncthreads();

    // ---- o[h][d] = sum_k p[h][k] v[k][d], lanes on 16-byte slices of value rows
    float acc[RW_HG][VEC];
#pragma unroll
    for (int hh = 0; hh < RW_HG; ++hh)
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[hh][e] = 0.f;
#pragma unroll 4
    for (int it = 0; it < ITERS; ++it) {
      const int kk = kw + it * KPI + sub;
      if (kk < nk) {
        float vv[VEC];
        if constexpr (F8) {
          const int sl = sl_s[kk];
          decode16_e4m3(*reinterpret_cast<const u32x4_t*>(c8.v + kv_index(sl, g, d0, hkv, DH)), vv);
          const float sc = c8.vs[sl];
#pragma unroll
          for (int e = 0; e < VEC; ++e) vv[e] *= sc;
        } else {
          unpack16<T>(*reinterpret_cast<const u32x4_t*>(cache.v + kv_index(sl_s[kk], g, d0, hkv, DH)), vv);
        }
#pragma unroll
        for (int hh = 0; hh < RW_HG; ++hh) {
          const float p = ps[hh][kk];
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[hh][e] = fmaf(p, vv[e], acc[hh][e]);
        }
      }
    }
    // reduce over the KPI key rows of one wave load, then over the 4 waves
#pragma unroll
    for (int hh = 0; hh < RW_HG; ++hh)
#pragma unroll
      for (int e = 0; e < VEC; ++e)
#pragma unroll
        for (int off = LPK; off < 64; off <<= 1) acc[hh][e] = xor_add(acc[hh][e], off, false);
    if (sub == 0) {
#pragma unroll
      for (int hh = 0; hh < RW_HG; ++hh)
#pragma unroll
        for (int e = 0; e < VEC; ++e) opart[w][hh][d0 + e] = acc[hh][e];
    }
    __syncthreads();
    for (int i = tid; i < RW_HG * DH; i += 256) {
      const int hh = i / DH, d = i % DH;
      if (h0 + hh < rep) {
        float* o = wsr + ((int64_t)(h0 + hh) * nchunks + c) * stride;
        o[2 + d] = opart[0][hh][d] + opart[1][hh][d] + opart[2][hh][d] + opart[3][hh][d];
        if (d == 0) {
          o[0] = mh[hh];
          o[1] = red[hh][0] + red[hh][1] + red[hh][2] + red[hh][3];
        }
      }
    }
    __syncthreads();
  }
}

// bf16 rows with head_dim 128 (the decode and last-token rows): one wave
// per 64-key chunk of one row and kv head, four independent waves per
// workgroup, no workgroup barrier.  Every K and V load of the chunk is
// issued before any result is consumed (keys past the context read slot 0
// and are masked), so a wave waits for memory about twice, not per key.
//  * block ids: the chunk spans four 16-key blocks, uniform across the wave.
//  * scores: lane (k, j) = (lane / 4, lane % 4) takes key pass*16 + k and
//    dims 32 j .. + 32 (four 16-byte loads), bf16 pair dot products
//    (v_dot2c_f32_bf16) against the row's q, then a quad reduction; the
//    chunk's softmax statistics reduce across the 16 key lanes and the
//    probabilities go to wave-local LDS.
//  * P.V: lane (b, c) = (lane / 16, lane % 16) takes the 16 keys of block b,
//    dims 8 c .. + 8 (one 16-byte load per key), for all four heads; a
//    reduce-scatter over the four blocks with the permlane swaps leaves
//    head b's sums in the lanes of block b.
// Writes (max, sum, unnormalised o) per head and chunk like attn_rows_kernel.
// F8: K/V come from the per-token FP8 cache c8; a lane's codes (32 of a key
// row for the scores, 8 per key for P.V, half the bytes of the bf16 loads)
// are decoded and multiplied by their token's scale into the same bf16
// operands, so everything after the loads is shared.
constexpr int DC_KEYS = 64;
template <bool F8>
__global__ __launch_bounds__(256) void attn_dec_kernel(const bf16_t* __restrict__ q, CacheSlot<bf16_t> cache,
                                                       Fp8Slot c8, const int32_t* __restrict__ row_seq,
                                                       const int32_t* __restrict__ row_pos,
                                                       const int32_t* __restrict__ bt, int max_blocks, int hq,
                                                       int nchunks, float scale, float* __restrict__ ws) {
  constexpr int DH = 128;
  // [wave][key] -> probabilities of the wave's four heads.  Key k of 16-key
  // block b sits at b * 17 + k: the P.V reads have the four 16-lane groups
  // of a wave read one entry of each block at once, and with blocks 256 B
  // apart those four 16-byte reads fell on the same banks (3.2 conflict
  // cycles per LDS instruction on the counter)
  __shared__ f32x4_t ps_s[4][4 * 17];
  const int r = blockIdx.x, g = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = blockIdx.z * 4 + wave;
  if (c >= nchunks) return;
  const int hkv = cache.hkv;
  const int rep = hq / hkv;
  const int ctx = row_pos[r] + 1;
  const int seq = row_seq[r];
  const int stride = DH + 2;
  float* wsr = ws + ((int64_t)r * hq + g * rep) * nchunks * stride + (int64_t)c * stride;
  const int kbeg = c * DC_KEYS;
  if (kbeg >= ctx) {  // empty chunk
    if (lane < rep) {
      wsr[(int64_t)lane * nchunks * stride] = -INFINITY;
      wsr[(int64_t)lane * nchunks * stride + 1] = 0.f;
    }
    return;
  }
  const int nk = min(DC_KEYS, ctx - kbeg);
  int blk[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) blk[b] = kbeg + 16 * b < ctx ? bt[(int64_t)seq * max_blocks + kbeg / kBlockSize + b] : 0;
  const int kq = lane >> 2, j = lane & 3;   // score layout
  const int vb = lane >> 4, vc = lane & 15;  // P.V layout
  const int vblk = vb == 0 ? blk[0] : vb == 1 ? blk[1] : vb == 2 ? blk[2] : blk[3];
  for (int h0 = 0; h0 < rep; h0 += RW_HG) {
    const int nh = min(RW_HG, rep - h0);
    // K of the lane's four keys (issued first), then q of heads h0 .. h0 + 3.
    // The bf16 pairs for v_dot2c_f32_bf16 are taken from bf16x8 vectors by
    // shufflevector: hipcc 7.2 lowers a bit_cast of a u32x4 element to bf16x2
    // feeding the dot2 builtin to element 0 of the vector every time.
    // bf16: K of the lane's four keys, issued first; F8: their codes and
    // scales, decoded pass by pass in the score loop
    bf16x8_t kv[F8 ? 1 : 4][4];
    u32x4_t kc[F8 ? 4 : 1][2];
    float ksc[F8 ? 4 : 1];
    if constexpr (F8) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int sl = blk[p] * kBlockSize + kq;
        const uint8_t* kr = c8.k + kv_index(sl, g, j * 32, hkv, DH);
        kc[p][0] = *reinterpret_cast<const u32x4_t*>(kr);
        kc[p][1] = *reinterpret_cast<const u32x4_t*>(kr + 16);
        ksc[p] = c8.ks[sl];
      }
    } else {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const bf16_t* kr = cache.k + kv_index(blk[p] * kBlockSize + kq, g, j * 32, hkv, DH);
#pragma unroll
        for (int i = 0; i < 4; ++i) kv[p][i] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(kr + i * 8));
      }
    }
    bf16x8_t qv[RW_HG][4];
#pragma unroll
    for (int hh = 0; hh < RW_HG; ++hh)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        qv[hh][i] = as_bf16x8(hh < nh ? *reinterpret_cast<const u32x4_t*>(q + ((int64_t)r * hq + g * rep + h0 + hh) * DH + j * 32 + i * 8)
                                      : u32x4_t{0u, 0u, 0u, 0u});
    float sc[4][RW_HG];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      bf16x8_t kp[4];
      if constexpr (F8) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          float x[16];
#pragma unroll
          for (int e = 0; e < 4; ++e) decode4_e4m3_hw(kc[p][h2][e], x + 4 * e);
#pragma unroll
          for (int i2 = 0; i2 < 2; ++i2) {
            const float* y = x + 8 * i2;
            const float s8 = ksc[p];
            kp[2 * h2 + i2] = as_bf16x8(u32x4_t{pack_bf16x2(y[0] * s8, y[1] * s8), pack_bf16x2(y[2] * s8, y[3] * s8),
                                                pack_bf16x2(y[4] * s8, y[5] * s8), pack_bf16x2(y[6] * s8, y[7] * s8)});
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) kp[i] = kv[p][i];
      }
      float acc[RW_HG] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int hh = 0; hh < RW_HG; ++hh) {
          const bf16x8_t kx = kp[i], qx = qv[hh][i];
          float a = acc[hh];
          a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kx, kx, 0, 1), __builtin_shufflevector(qx, qx, 0, 1), a, false);
          a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kx, kx, 2, 3), __builtin_shufflevector(qx, qx, 2, 3), a, false);
          a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kx, kx, 4, 5), __builtin_shufflevector(qx, qx, 4, 5), a, false);
          a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kx, kx, 6, 7), __builtin_shufflevector(qx, qx, 6, 7), a, false);
          acc[hh] = a;
        }
#pragma unroll
      for (int hh = 0; hh < RW_HG; ++hh) {
        float a = xor_add(acc[hh], 1, true);
        a = xor_add(a, 2, true);
        sc[p][hh] = p * 16 + kq < nk ? a * scale : -INFINITY;  // a select: garbage past the context never propagates
      }
    }
    // V of the lane's 16 keys, in flight while the softmax runs (F8: codes
    // and scales, decoded after the softmax)
    bf16x8_t vv[16];
    u32x2_t vcode[F8 ? 16 : 1];
    float vsc[F8 ? 16 : 1];
    if constexpr (F8) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int sl = vblk * kBlockSize + i;
        vcode[i] = *reinterpret_cast<const u32x2_t*>(c8.v + kv_index(sl, g, vc * 8, hkv, DH));
        vsc[i] = c8.vs[sl];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        vv[i] = as_bf16x8(
            *reinterpret_cast<const u32x4_t*>(cache.v + kv_index(vblk * kBlockSize + i, g, vc * 8, hkv, DH)));
    }
    // softmax statistics over the chunk, per head (lanes of a quad agree)
    float mh[RW_HG], lh[RW_HG];
    f32x4_t pe[4];
#pragma unroll
    for (int hh = 0; hh < RW_HG; ++hh) {
      float m = fmaxf(fmaxf(sc[0][hh], sc[1][hh]), fmaxf(sc[2][hh], sc[3][hh]));
      m = fmaxf(m, dpp_f<0x141>(m));
      m = fmaxf(m, dpp_f<0x128>(m));
      {
        auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
        m = fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
      }
      m = xor32_max(m);
      float l = 0.f;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float e = sc[p][hh] == -INFINITY ? 0.f : __expf(sc[p][hh] - m);
        l += e;
        pe[p][hh] = e;
      }
      l = xor_add(l, 4, true);
      l = xor_add(l, 8, true);
      l = xor_add(l, 16, true);
      l = xor_add(l, 32, true);
      mh[hh] = m;
      lh[hh] = l;
    }
    if (j == 0) {
#pragma unroll
      for (int p = 0; p < 4; ++p) ps_s[wave][p * 17 + kq] = pe[p];
    }
    if constexpr (F8) {  // each key's 8 codes times its scale, as bf16 pairs
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float s8 = vsc[i];
        float x[8];
        decode4_e4m3_hw(vcode[i].x, x);
        decode4_e4m3_hw(vcode[i].y, x + 4);
        vv[i] = as_bf16x8(u32x4_t{pack_bf16x2(x[0] * s8, x[1] * s8), pack_bf16x2(x[2] * s8, x[3] * s8),
                                  pack_bf16x2(x[4] * s8, x[5] * s8), pack_bf16x2(x[6] * s8, x[7] * s8)});
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's probabilities are in LDS
    // o[hh][8 vc .. + 8] over the 16 keys of block vb
    float o[RW_HG][8];
#pragma unroll
    for (int hh = 0; hh < RW_HG; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[hh][e] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const f32x4_t pk = ps_s[wave][vb * 17 + i];  // zero past the context
      const bool live = vb * 16 + i < nk;
      const u32x4_t raw = __builtin_bit_cast(u32x4_t, vv[i]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w2 = live ? raw[e] : 0u;  // no 0 * NaN from slots past the context
        const float v0 = __uint_as_float(w2 << 16), v1 = __uint_as_float(w2 & 0xffff0000u);
#pragma unroll
        for (int hh = 0; hh < RW_HG; ++hh) {
          o[hh][2 * e] = fmaf(pk[hh], v0, o[hh][2 * e]);
          o[hh][2 * e + 1] = fmaf(pk[hh], v1, o[hh][2 * e + 1]);
        }
      }
    }
    // reduce-scatter over the four blocks: heads (0, 1) | (2, 3) across
    // lane ^ 32, then head 0 | 1 (2 | 3) across lane ^ 16
    float t2[2][8], u[8];
#pragma unroll
    for (int hp = 0; hp < 2; ++hp)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(o[hp][e]), __float_as_uint(o[hp + 2][e]), false, false);
        t2[hp][e] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(t2[0][e]), __float_as_uint(t2[1][e]), false, false);
      u[e] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    if (vb < nh) {
      float* w = wsr + (int64_t)(h0 + vb) * nchunks * stride + 2 + vc * 8;
#pragma unroll
      for (int e = 0; e < 8; e += 2) *reinterpret_cast<f32x2_t*>(w + e) = f32x2_t{u[e], u[e + 1]};
    }
    if (lane < nh) {
      float* w = wsr + (int64_t)(h0 + lane) * nchunks * stride;
      const float mv = lane == 0 ? mh[0] : lane == 1 ? mh[1] : lane == 2 ? mh[2] : mh[3];
      const float lv = lane == 0 ? lh[0] : lane == 1 ? lh[1] : lane == 2 ? lh[2] : lh[3];
      w[0] = mv;
      w[1] = lv;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // LDS reads of this head group done before the next overwrites ps_s
  }
}

// Single-pass form of attn_dec_kernel for contexts of at most
// DC1_MAX_KEYS keys: one workgroup per (row, kv head), one wave per 64-key
// chunk, so the chunks' (max, sum, o) meet in LDS and the workgroup writes
// the normalised output itself: no workspace, no combine launch.  A wave's
// chunk work is attn_dec_kernel's (the same loads and arithmetic), except
// that the head group's q sits in LDS, read by every wave, rather than in
// each wave's registers: a 16-wave workgroup leaves a wave 128 registers.
// The chunks are combined in chunk order.  F8: the codes and scales of the
// per-token FP8 cache, decoded into the same bf16 operands as in
// attn_dec_kernel<true>.
constexpr int DC1_WAVES = 16;
constexpr int DC1_MAX_KEYS = DC1_WAVES * DC_KEYS;
constexpr int DC1_MAX_REP = 16;  // a multiple of RW_HG
template <bool F8>
__global__ __launch_bounds__(DC1_WAVES * 64) void attn_dec1_kernel(const bf16_t* __restrict__ q,
                                                                   CacheSlot<bf16_t> cache, Fp8Slot c8,
                                                                   const int32_t* __restrict__ row_seq,
                                                                   const int32_t* __restrict__ row_pos,
                                                                   const int32_t* __restrict__ bt, int max_blocks,
                                                                   int hq, float scale, bf16_t* __restrict__ out) {
  constexpr int DH = 128;
  __shared__ __attribute__((aligned(16))) bf16_t q_s[DC1_MAX_REP * DH];
  __shared__ f32x4_t ps_s[DC1_WAVES][4 * 17];  // as in attn_dec_kernel
  __shared__ float po_s[DC1_WAVES][RW_HG][DH];
  __shared__ float pm_s[DC1_WAVES][RW_HG], pl_s[DC1_WAVES][RW_HG];
  const int r = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int hkv = cache.hkv;
  const int rep = hq / hkv;
  const int ctx = row_pos[r] + 1;
  const int seq = row_seq[r];
  // at most DC1_WAVES chunks: the launcher checks the rows' longest context
  const int nch = min((ctx + DC_KEYS - 1) / DC_KEYS, DC1_WAVES);
  const bool active = wave < nch;
  const int kbeg = wave * DC_KEYS;
  const int nk = active ? min(DC_KEYS, ctx - kbeg) : 0;
  const bf16_t* qg = q + ((int64_t)r * hq + g * rep) * DH;
  // q of the group's heads into LDS; heads up to the next multiple of four
  // are zero, so every wave reads four heads without a branch
  const int rep4 = (rep + RW_HG - 1) / RW_HG * RW_HG;
  for (int i = tid; i < rep4 * (DH / 8); i += DC1_WAVES * 64)
    *reinterpret_cast<u32x4_t*>(q_s + i * 8) =
        i < rep * (DH / 8) ? *reinterpret_cast<const u32x4_t*>(qg + i * 8) : u32x4_t{0u, 0u, 0u, 0u};
  int blk[4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
    blk[b] = active && kbeg + 16 * b < ctx ? bt[(int64_t)seq * max_blocks + kbeg / kBlockSize + b] : 0;
  const int kq = lane >> 2, j = lane & 3;   // score layout
  const int vb = lane >> 4, vc = lane & 15;  // P.V layout
  const int vblk = vb == 0 ? blk[0] : vb == 1 ? blk[1] : vb == 2 ? blk[2] : blk[3];
  __syncthreads();  // q in LDS
  for (int h0 = 0; h0 < rep; h0 += RW_HG) {
    const int nh = min(RW_HG, rep - h0);
    if (active) {
      // every K load of the chunk goes out first (64 registers); the scores
      // then take two 16-key passes and one q slice of four heads (16
      // registers, from LDS) at a time, which keeps the wave within its 128
      // registers
      float acc[4][RW_HG];
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int hh = 0; hh < RW_HG; ++hh) acc[p][hh] = 0.f;
      bf16x8_t kvall[F8 ? 1 : 2][2][4];
      u32x4_t kc[F8 ? 4 : 1][2];  // F8: 32 codes of the lane's key per pass
      float ksc[F8 ? 4 : 1];
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const int sl = blk[2 * half + pp] * kBlockSize + kq;
          if constexpr (F8) {
            const uint8_t* kr = c8.k + kv_index(sl, g, j * 32, hkv, DH);
            kc[2 * half + pp][0] = *reinterpret_cast<const u32x4_t*>(kr);
            kc[2 * half + pp][1] = *reinterpret_cast<const u32x4_t*>(kr + 16);
            ksc[2 * half + pp] = c8.ks[sl];
          } else {
            const bf16_t* kr = cache.k + kv_index(sl, g, j * 32, hkv, DH);
#pragma unroll
            for (int i = 0; i < 4; ++i) kvall[half][pp][i] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(kr + i * 8));
          }
        }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        bf16x8_t kv[2][4];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          if constexpr (F8) {  // code * the key's scale, as bf16
            const float s8 = ksc[2 * half + pp];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              float x[16];
#pragma unroll
              for (int e = 0; e < 4; ++e) decode4_e4m3_hw(kc[2 * half + pp][h2][e], x + 4 * e);
#pragma unroll
              for (int i2 = 0; i2 < 2; ++i2) {
                const float* y = x + 8 * i2;
                kv[pp][2 * h2 + i2] =
                    as_bf16x8(u32x4_t{pack_bf16x2(y[0] * s8, y[1] * s8), pack_bf16x2(y[2] * s8, y[3] * s8),
                                      pack_bf16x2(y[4] * s8, y[5] * s8), pack_bf16x2(y[6] * s8, y[7] * s8)});
              }
            }
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) kv[pp][i] = kvall[half][pp][i];
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bf16x8_t qv[RW_HG];
#pragma unroll
          for (int hh = 0; hh < RW_HG; ++hh)
            qv[hh] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(q_s + (h0 + hh) * DH + j * 32 + i * 8));
#pragma unroll
          for (int pp = 0; pp < 2; ++pp)
#pragma unroll
            for (int hh = 0; hh < RW_HG; ++hh) {
              const bf16x8_t kx = kv[pp][i], qx = qv[hh];
              float a = acc[2 * half + pp][hh];
              a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kx, kx, 0, 1), __builtin_shufflevector(qx, qx, 0, 1), a, false);
              a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kx, kx, 2, 3), __builtin_shufflevector(qx, qx, 2, 3), a, false);
              a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kx, kx, 4, 5), __builtin_shufflevector(qx, qx, 4, 5), a, false);
              a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kx, kx, 6, 7), __builtin_shufflevector(qx, qx, 6, 7), a, false);
              acc[2 * half + pp][hh] = a;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      float sc[4][RW_HG];
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int hh = 0; hh < RW_HG; ++hh) {
          float a = xor_add(acc[p][hh], 1, true);
          a = xor_add(a, 2, true);
          sc[p][hh] = p * 16 + kq < nk ? a * scale : -INFINITY;
        }
      // the first half of the lane's V rows goes out now (the second after
      // the first's products: 32 registers of V at a time)
      // F8: a key's 8 codes (one dword pair) and its scale, decoded when used
      bf16x8_t vv[F8 ? 1 : 8];
      u32x2_t vcode[F8 ? 8 : 1];
      float vsc[F8 ? 8 : 1];
      auto load_v = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int sl = vblk * kBlockSize + k0 + i;
          if constexpr (F8) {
            vcode[i] = *reinterpret_cast<const u32x2_t*>(c8.v + kv_index(sl, g, vc * 8, hkv, DH));
            vsc[i] = c8.vs[sl];
          } else {
            vv[i] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(cache.v + kv_index(sl, g, vc * 8, hkv, DH)));
          }
        }
      };
      load_v(0);
      float mh[RW_HG], lh[RW_HG];
      f32x4_t pe[4];
#pragma unroll
      for (int hh = 0; hh < RW_HG; ++hh) {
        float m = fmaxf(fmaxf(sc[0][hh], sc[1][hh]), fmaxf(sc[2][hh], sc[3][hh]));
        m = fmaxf(m, dpp_f<0x141>(m));
        m = fmaxf(m, dpp_f<0x128>(m));
        {
          auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
          m = fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
        }
        m = xor32_max(m);
        float l = 0.f;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float e = sc[p][hh] == -INFINITY ? 0.f : __expf(sc[p][hh] - m);
          l += e;
          pe[p][hh] = e;
        }
        l = xor_add(l, 4, true);
        l = xor_add(l, 8, true);
        l = xor_add(l, 16, true);
        l = xor_add(l, 32, true);
        mh[hh] = m;
        lh[hh] = l;
      }
      if (j == 0) {
#pragma unroll
        for (int p = 0; p < 4; ++p) ps_s[wave][p * 17 + kq] = pe[p];
      }
      if (lane < RW_HG) {  // the chunk's statistics, from lanes 0..3
        pm_s[wave][lane] = lane == 0 ? mh[0] : lane == 1 ? mh[1] : lane == 2 ? mh[2] : mh[3];
        pl_s[wave][lane] = lane == 0 ? lh[0] : lane == 1 ? lh[1] : lane == 2 ? lh[2] : lh[3];
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's probabilities are in LDS
      float o[RW_HG][8];
#pragma unroll
      for (int hh = 0; hh < RW_HG; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] = 0.f;
#pragma unroll
      for (int vh = 0; vh < 2; ++vh) {
        if (vh == 1) load_v(8);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int key = vh * 8 + i;
          const f32x4_t pk = ps_s[wave][vb * 17 + key];
          const bool live = vb * 16 + key < nk;
          u32x4_t raw;
          if constexpr (F8) {
            float x[8];
            decode4_e4m3_hw(vcode[i].x, x);
            decode4_e4m3_hw(vcode[i].y, x + 4);
            const float s8 = vsc[i];
            raw = u32x4_t{pack_bf16x2(x[0] * s8, x[1] * s8), pack_bf16x2(x[2] * s8, x[3] * s8),
                          pack_bf16x2(x[4] * s8, x[5] * s8), pack_bf16x2(x[6] * s8, x[7] * s8)};
          } else {
            raw = __builtin_bit_cast(u32x4_t, vv[i]);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t w2 = live ? raw[e] : 0u;
            const float v0 = __uint_as_float(w2 << 16), v1 = __uint_as_float(w2 & 0xffff0000u);
#pragma unroll
            for (int hh = 0; hh < RW_HG; ++hh) {
              o[hh][2 * e] = fmaf(pk[hh], v0, o[hh][2 * e]);
              o[hh][2 * e + 1] = fmaf(pk[hh], v1, o[hh][2 * e + 1]);
            }
          }
        }
      }
      float t2[2][8], u[8];
#pragma unroll
      for (int hp = 0; hp < 2; ++hp)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(o[hp][e]), __float_as_uint(o[hp + 2][e]), false, false);
          t2[hp][e] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(t2[0][e]), __float_as_uint(t2[1][e]), false, false);
        u[e] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
      // head vb's partial sums, dims 8 vc .. + 8
#pragma unroll
      for (int e = 0; e < 8; e += 4)
        *reinterpret_cast<f32x4_t*>(&po_s[wave][vb][vc * 8 + e]) = f32x4_t{u[e], u[e + 1], u[e + 2], u[e + 3]};
    }
    __syncthreads();  // every chunk's partials in LDS
    if (tid < nh * DH) {
      const int hh = tid / DH, d = tid % DH;
      float M = -INFINITY;
      for (int c = 0; c < nch; ++c) M = fmaxf(M, pm_s[c][hh]);
      float L = 0.f, A = 0.f;
      for (int c = 0; c < nch; ++c) {
        const float e = __expf(pm_s[c][hh] - M);
        L += pl_s[c][hh] * e;
        A += po_s[c][hh][d] * e;
      }
      out[((int64_t)r * hq + g * rep + h0 + hh) * DH + d] = f32_to_bf16(A / L);
    }
    __syncthreads();  // partials read before the next head group overwrites them
  }
}

// One (row, head): 4 chunk groups x head_dim threads.  Group q takes chunks
// q, q+4, ... in order; the maximum, then the weighted sums, are combined
// across the groups in group order (fixed, deterministic).  Four groups cut
// the serial chain of loads per thread four-fold, which matters for one
// row over a long context (hundreds of chunks).
template <typename T>
__global__ __launch_bounds__(4 * RW_MAXDH) void attn_combine_kernel(const float* __restrict__ ws, int hq, int dh,
                                                                    int nchunks, T* __restrict__ o) {
  __shared__ float red_m[4], red_l[4], red_a[4][RW_MAXDH];
  const int r = blockIdx.x, h = blockIdx.y;
  const int d = threadIdx.x % RW_MAXDH, grp = threadIdx.x / RW_MAXDH;
  const int stride = dh + 2;
  const float* w = ws + ((int64_t)r * hq + h) * nchunks * stride;
  float m = -INFINITY;
#pragma unroll 8
  for (int c = grp; c < nchunks; c += 4) m = fmaxf(m, w[c * stride]);
  if (d == 0) red_m[grp] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
  float l = 0.f, acc = 0.f;
#pragma unroll 8
  for (int c = grp; c < nchunks; c += 4) {
    const float mc = w[c * stride];
    if (mc == -INFINITY) continue;
    const float e = __expf(mc - M);
    l += w[c * stride + 1] * e;
    if (d < dh) acc += w[c * stride + 2 + d] * e;
  }
  red_a[grp][d] = acc;
  if (d == 0) red_l[grp] = l;
  __syncthreads();
  if (grp == 0 && d < dh) {
    const float L = ((red_l[0] + red_l[1]) + red_l[2]) + red_l[3];
    const float A = ((red_a[0][d] + red_a[1][d]) + red_a[2][d]) + red_a[3][d];
    o[((int64_t)r * hq + h) * dh + d] = from_f32<T>(A / L);
  }
}

}  // namespace

// Batches whose sequences bring at most this many new tokens take the
// 4-wave form (32 queries per workgroup, two workgroups per CU): a
// workgroup's fixed cost (block-table reads, then Q and the first K/V tiles
// from HBM, and the output pass) is a large share of a short prompt's few
// tiles, and a second workgroup on the CU runs while one waits in it.  On
// long prompts the 8-wave form's shared K/V tiles win.
#ifndef SKV_ATTN_SHORT_MAX_NEW
#define SKV_ATTN_SHORT_MAX_NEW 2048
#endif
constexpr int kAttnShortMaxNew = SKV_ATTN_SHORT_MAX_NEW;

hipError_t launch_attn_prefill_bf16(const bf16_t* q, CacheSlot<bf16_t> cache, const int32_t* cu_seqlens,
                                    const int32_t* ctx_lens, const int32_t* block_tables, int max_blocks, int batch,
                                    int max_new, int hq, bf16_t* o, hipStream_t stream) {
  if (batch <= 0 || max_new <= 0) return hipSuccess;
  const int rep = hq / cache.hkv;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)FA_DH);
  if (max_new <= kAttnShortMaxNew) {
    dim3 grid(batch * (hq / 4), (max_new + 31) / 32);
    hipLaunchKernelGGL((attn_prefill8_kernel<false, false, 4>), grid, dim3(256), 0, stream, q, nullptr, cache,
                       CacheSlot<bf16_t>{nullptr, nullptr, cache.hkv, cache.dh}, Fp8Slot{}, cu_seqlens, ctx_lens,
                       block_tables, max_blocks, hq, rep, scale_log2, o);
  } else {
    dim3 grid(batch * (hq / 4), (max_new + 63) / 64);
    hipLaunchKernelGGL((attn_prefill8_kernel<false, false>), grid, dim3(512), 0, stream, q, nullptr, cache,
                       CacheSlot<bf16_t>{nullptr, nullptr, cache.hkv, cache.dh}, Fp8Slot{}, cu_seqlens, ctx_lens,
                       block_tables, max_blocks, hq, rep, scale_log2, o);
  }
  return hipGetLastError();
}

hipError_t launch_attn_prefill_split(const bf16_t* q, const bf16_t* q_lo, CacheSlot<bf16_t> cache,
                                     CacheSlot<bf16_t> lo, const int32_t* cu_seqlens, const int32_t* ctx_lens,
                                     const int32_t* block_tables, int max_blocks, int batch, int max_new, int hq,
                                     bf16_t* o, hipStream_t stream) {
  if (batch <= 0 || max_new <= 0) return hipSuccess;
  if (!q_lo || !lo.k || !lo.v || lo.hkv != cache.hkv || lo.dh != cache.dh) return hipErrorInvalidValue;
  const int rep = hq / cache.hkv;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)FA_DH);
  dim3 grid(batch * (hq / 4), (max_new + 63) / 64);
  hipLaunchKernelGGL((attn_prefill8_kernel<false, true>), grid, dim3(512), 0, stream, q, q_lo, cache, lo, Fp8Slot{},
                     cu_seqlens, ctx_lens, block_tables, max_blocks, hq, rep, scale_log2, o);
  return hipGetLastError();
}

hipError_t launch_attn_prefill_fp8(const bf16_t* q, Fp8Slot cache, const int32_t* cu_seqlens, const int32_t* ctx_lens,
                                   const int32_t* block_tables, int max_blocks, int batch, int max_new, int hq,
                                   bf16_t* o, hipStream_t stream) {
  if (batch <= 0 || max_new <= 0) return hipSuccess;
  if (cache.dh != FA_DH) return hipErrorInvalidValue;
  const int rep = hq / cache.hkv;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)FA_DH);
  dim3 grid(batch * (hq / 4), (max_new + 63) / 64);
  hipLaunchKernelGGL((attn_prefill8_kernel<true, false>), grid, dim3(512), 0, stream, q, nullptr,
                     CacheSlot<bf16_t>{nullptr, nullptr, cache.hkv, cache.dh},
                     CacheSlot<bf16_t>{nullptr, nullptr, cache.hkv, cache.dh}, cache, cu_seqlens, ctx_lens,
                     block_tables, max_blocks, hq, rep, scale_log2, o);
  return hipGetLastError();
}

int64_t attn_rows_ws_elems(int rows, int max_ctx, int hq, int dh, bool bf16_rows) {
  // bf16 rows of head_dim 128 use attn_dec_kernel's 64-key chunks
  const int ch = bf16_rows && dh == 128 ? DC_KEYS : RW_CH;
  int nchunks = (max_ctx + ch - 1) / ch;
  return (int64_t)rows * hq * nchunks * (dh + 2);
}

namespace {

template <typename T, bool F8>
hipError_t attn_rows_impl(const T* q, CacheSlot<T> cache, Fp8Slot c8, const int32_t* row_seq, const int32_t* row_pos,
                          const int32_t* block_tables, int max_blocks, int rows, int max_ctx, int hq, float* ws, T* o,
                          hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const float scale = 1.0f / sqrtf((float)cache.dh);
  if constexpr (sizeof(T) == 2) {
    if (cache.dh == 128 && max_ctx <= DC1_MAX_KEYS && hq / cache.hkv <= DC1_MAX_REP) {
      hipLaunchKernelGGL((attn_dec1_kernel<F8>), dim3(rows, cache.hkv), dim3(DC1_WAVES * 64), 0, stream, q, cache,
                         c8, row_seq, row_pos, block_tables, max_blocks, hq, scale, o);
      return hipGetLastError();
    }
    if (cache.dh == 128) {
      const int nch = (max_ctx + DC_KEYS - 1) / DC_KEYS;
      hipLaunchKernelGGL((attn_dec_kernel<F8>), dim3(rows, cache.hkv, (nch + 3) / 4), dim3(256), 0, stream, q,
                         cache, c8, row_seq, row_pos, block_tables, max_blocks, hq, nch, scale, ws);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(attn_combine_kernel<T>, dim3(rows, hq), dim3(4 * RW_MAXDH), 0, stream, ws, hq, cache.dh, nch, o);
      return hipGetLastError();
    }
  }
  const int nchunks = (max_ctx + RW_CH - 1) / RW_CH;
  const dim3 grid(rows, cache.hkv, nchunks);
  switch (cache.dh) {
    case 128:
      hipLaunchKernelGGL((attn_rows_kernel<T, 128, F8>), grid, dim3(256), 0, stream, q, cache, c8, row_seq, row_pos,
                         block_tables, max_blocks, hq, nchunks, scale, ws);
      break;
    case 64:
      hipLaunchKernelGGL((attn_rows_kernel<T, 64, F8>), grid, dim3(256), 0, stream, q, cache, c8, row_seq, row_pos,
                         block_tables, max_blocks, hq, nchunks, scale, ws);
      break;
    case 32:
      hipLaunchKernelGGL((attn_rows_kernel<T, 32, F8>), grid, dim3(256), 0, stream, q, cache, c8, row_seq, row_pos,
                         block_tables, max_blocks, hq, nchunks, scale, ws);
      break;
    default:
      return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel<T>, dim3(rows, hq), dim3(4 * RW_MAXDH), 0, stream, ws, hq, cache.dh, nchunks, o);
  return hipGetLastError();
}

}  // namespace

template <typename T>
hipError_t launch_attn_rows(const T* q, CacheSlot<T> cache, const int32_t* row_seq, const int32_t* row_pos,
                            const int32_t* block_tables, int max_blocks, int rows, int max_ctx, int hq, float* ws,
                            T* o, hipStream_t stream) {
  return attn_rows_impl<T, false>(q, cache, Fp8Slot{}, row_seq, row_pos, block_tables, max_blocks, rows, max_ctx, hq,
                                  ws, o, stream);
}

hipError_t launch_attn_rows_fp8(const bf16_t* q, Fp8Slot cache, const int32_t* row_seq, const int32_t* row_pos,
                                const int32_t* block_tables, int max_blocks, int rows, int max_ctx, int hq, float* ws,
                                bf16_t* o, hipStream_t stream) {
  if (cache.dh != 128) return hipErrorInvalidValue;
  return attn_rows_impl<bf16_t, true>(q, CacheSlot<bf16_t>{nullptr, nullptr, cache.hkv, cache.dh}, cache, row_seq,
                                      row_pos, block_tables, max_blocks, rows, max_ctx, hq, ws, o, stream);
}

template hipError_t launch_attn_rows<float>(const float*, CacheSlot<float>, const int32_t*, const int32_t*,
                                            const int32_t*, int, int, int, int, float*, float*, hipStream_t);
template hipError_t launch_attn_rows<bf16_t>(const bf16_t*, CacheSlot<bf16_t>, const int32_t*, const int32_t*,
                                             const int32_t*, int, int, int, int, float*, bf16_t*, hipStream_t);
