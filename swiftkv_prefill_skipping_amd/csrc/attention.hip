// Attention kernels.
//
// 1. attn_prefill_kernel (bf16, MFMA): causal GQA flash attention of the
//    prompt tokens of layers 1..l, reading K/V from the paged cache.
//    A workgroup = 4 wave64s = 4 query heads of one kv-head group, for
//    32*QT consecutive query positions of one prompt.  Per 64-key tile:
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
//    ([64 keys][128 dims], 16-byte chunk c of key row r at c ^ (r & 15)).
//    O^T is transposed through LDS at the end and written 8 bytes per lane
//    into the panel layout of the O projection's A operand.
//    K/V tiles move global -> LDS directly (global_load_lds_dwordx4) into a
//    two-stage ring, the next tile's loads in flight while the current one
//    is computed; the prompt's block ids are staged in LDS so no load waits
//    on a block-table read.  Keys past the prompt (or causally masked) get
//    probability exactly 0, so the cache contents loaded for them only need
//    to be finite, which the cache guarantees (zero-filled at creation,
//    written only with results).  Two workgroups fit per CU (<= 256 VGPRs,
//    66 KB LDS).
//
// 2. attn_rows_kernel + attn_combine_kernel (fp32 or bf16, vector ALU):
//    attention of an explicit list of query rows (the last prompt token of
//    each prompt at layers l+1..L; every token for fp32 models), split over
//    256-key chunks with a fixed-order combine.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef s16x4_t short4_lds_t;

constexpr int FA_DH = 128;
constexpr int FA_KT = 64;  // keys per tile

constexpr int FA_BTW = 32;  // block-table entries staged in LDS at a time (8 key tiles)

SKV_DEV void wait_loads_then_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <int QT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_prefill_kernel(
    const bf16_t* __restrict__ q, CacheSlot<bf16_t> cache, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ bt, int max_blocks, int hq, int rep, float scale_log2, bf16_t* __restrict__ o) {
  // double-buffered K and V tiles, [64 keys][128 dims] each, filled by
  // direct global -> LDS loads
  __shared__ __attribute__((aligned(1024))) bf16_t sK[2][FA_KT * FA_DH];
  __shared__ __attribute__((aligned(1024))) bf16_t sV[2][FA_KT * FA_DH];
  __shared__ int32_t sBT[FA_BTW];

  const int b = blockIdx.y;
  const int tok0 = cu[b];
  const int N = cu[b + 1] - tok0;
  const int QB = 32 * QT;
  const int nqb = (N + QB - 1) / QB;
  const int qb = gridDim.x - 1 - blockIdx.x;  // longest rows first
  if (qb >= nqb) return;
  const int q0 = qb * QB;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5;
  const int h = blockIdx.z * 4 + wave;
  const int g = (blockIdx.z * 4) / rep;
  const int hkv = cache.hkv;
  const int dq = hq * FA_DH;

  const int kend = min(N, q0 + QB);
  const int ntiles = (kend + FA_KT - 1) / FA_KT;
  const int nblk_need = (kend + kBlockSize - 1) / kBlockSize;
  const int32_t* btb = bt + (int64_t)b * max_blocks;

  // Block ids of tiles t0 .. t0+7.  Entries past the keys this workgroup
  // needs (causally masked or beyond the prompt) repeat block 0, a valid
  // block of the prompt, so every load stays inside the cache.
  auto stage_block_ids = [&](int t0) {
    if (tid < FA_BTW) {
      const int i = tid;
      const int bi = t0 * (FA_KT / kBlockSize) + i;
      sBT[i] = btb[bi < nblk_need ? bi : 0];
    }
  };
  stage_block_ids(0);

  // Q^T fragments: lane holds query (lane & 31), dims ks*16 + hh*8 .. +8
  bf16x8_t qf[QT][8];
#pragma unroll
  for (int s = 0; s < QT; ++s) {
    int qi = min(q0 + s * 32 + (lane & 31), N - 1);
    const bf16_t* qp = q + (int64_t)(tok0 + qi) * dq + h * FA_DH + hh * 8;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[s][ks] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(qp + ks * 16));
  }

  f32x16_t oacc[QT][4];
  float m_run[QT], l_run[QT];
#pragma unroll
  for (int s = 0; s < QT; ++s) {
    m_run[s] = -INFINITY;
    l_run[s] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[s][dt] = f32x16_t{0};
  }
  __syncthreads();

  // Tile loads: per 16-key block r of the tile, wave w moves key rows
  // w*4 .. w*4+3 of K and of V (1 KB each, one instruction).  Lane l's 16
  // bytes land at LDS row w*4 + l/16, physical chunk l%16, so it fetches the
  // logical chunk (l%16) ^ (row & 15): the XOR swizzle of the tile layout.
  const int lrow = wave * 4 + (lane >> 4);
  const int lane_off = lrow * FA_DH + (((lane & 15) ^ lrow) << 3);
  auto issue_tile = [&](int t, int buf) {
    const int wb = (t * (FA_KT / kBlockSize)) % FA_BTW;
#pragma unroll
    for (int r = 0; r < FA_KT / kBlockSize; ++r) {
      const int64_t base = ((int64_t)sBT[wb + r] * hkv + g) * (kBlockSize * FA_DH) + lane_off;
      typedef __attribute__((address_space(3))) void* lds_ptr;
      __builtin_amdgcn_global_load_lds(cache.k + base, (lds_ptr)(&sK[buf][(r * 16 + wave * 4) * FA_DH]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(cache.v + base, (lds_ptr)(&sV[buf][(r * 16 + wave * 4) * FA_DH]), 16, 0, 0);
    }
  };

  issue_tile(0, 0);
  wait_loads_then_barrier();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < ntiles) {
      if ((kt + 1) % (FA_BTW / (FA_KT / kBlockSize)) == 0) {  // next window of block ids
        stage_block_ids(kt + 1);
        __syncthreads();
      }
      issue_tile(kt + 1, cur ^ 1);
    }
    const int k0 = kt * FA_KT;
    const bf16_t* sk = sK[cur];
    const bf16_t* sv = sV[cur];

    // S^T = K Q^T, two 32-key subtiles
    f32x16_t sacc[QT][2];
#pragma unroll
    for (int s = 0; s < QT; ++s) sacc[s][0] = sacc[s][1] = f32x16_t{0};
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int key = st * 32 + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int ch = ks * 2 + hh;
        bf16x8_t kf = as_bf16x8(*reinterpret_cast<const u32x4_t*>(sk + key * FA_DH + ((ch ^ (key & 15)) << 3)));
#pragma unroll
        for (int s = 0; s < QT; ++s)
          sacc[s][st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s][ks], sacc[s][st], 0, 0, 0);
      }
    }

    // Online softmax per query column.  Scores stay raw; the scale c =
    // log2(e)/sqrt(dh) enters the exponent, p = 2^(c*s - m).  The running
    // offset m only moves when a column's tile maximum exceeds it by more
    // than kLazy (then every column of the wave rescales); otherwise p <=
    // 2^kLazy, which fp32 sums and bf16 probabilities hold exactly as well.
    // softmax(s) does not depend on the offset, so this is the same
    // function; it saves the rescale of the output accumulators on most
    // tiles.  Masking (causal diagonal, prompt end) only on the tiles that
    // need it.
    constexpr float kLazy = 8.0f;
    bf16x8_t pf[QT][4];
#pragma unroll
    for (int s = 0; s < QT; ++s) {
      const int qi = q0 + s * 32 + (lane & 31);
      const bool need_mask = (k0 + FA_KT - 1 > q0 + s * 32) || (k0 + FA_KT > N);
      if (need_mask) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = k0 + st * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
            if (key > qi || key >= N) sacc[s][st][v] = -INFINITY;
          }
      }
      float mt = sacc[s][0][0];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int v = 0; v < 16; ++v) mt = fmaxf(mt, sacc[s][st][v]);
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * scale_log2;
      if (__builtin_amdgcn_ballot_w64(mt > m_run[s] + kLazy) != 0) {
        const float m_new = fmaxf(m_run[s], mt);
        const float alpha = __builtin_amdgcn_exp2f(m_run[s] - m_new);
        m_run[s] = m_new;
        l_run[s] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int v = 0; v < 16; ++v) oacc[s][dt][v] *= alpha;
      }
      const float mneg = -m_run[s];
      float ls = 0.f;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[s][st][v], scale_log2, mneg));
          sacc[s][st][v] = p;
          ls += p;
        }
      ls += __shfl_xor(ls, 32, 64);
      l_run[s] += ls;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int st = kk >> 1, vb = 8 * (kk & 1);
        u32x4_t w;
        w.x = pack_bf16x2(sacc[s][st][vb + 0], sacc[s][st][vb + 1]);
        w.y = pack_bf16x2(sacc[s][st][vb + 2], sacc[s][st][vb + 3]);
        w.z = pack_bf16x2(sacc[s][st][vb + 4], sacc[s][st][vb + 5]);
        w.w = pack_bf16x2(sacc[s][st][vb + 6], sacc[s][st][vb + 7]);
        pf[s][kk] = as_bf16x8(w);
      }
    }

    // O^T += V^T P^T.  Transposing reads: lane l = 16 grp + 4 a + b points
    // at key kk*16 + 4*(l/32) + a (and +8), dims dbase + 4b .. +3, and
    // receives keys kk*16 + 4*(l/32) + 0..3 (and +8) of dim dbase + l%16.
    const int tj = lane & 15, ta = tj >> 2, tb = tj & 3;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int d = dt * 32 + 16 * ((lane >> 4) & 1) + 4 * tb;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int k1 = kk * 16 + 4 * hh + ta, k2 = k1 + 8;
        typedef __attribute__((address_space(3))) short4_lds_t* lds_s4p;
        s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s4p)(sv + k1 * FA_DH + (((d >> 3) ^ (k1 & 15)) << 3) + (d & 7)));
        s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s4p)(sv + k2 * FA_DH + (((d >> 3) ^ (k2 & 15)) << 3) + (d & 7)));
        u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo), hi2 = __builtin_bit_cast(u32x2_t, hi);
        bf16x8_t vf = as_bf16x8(u32x4_t{lo2.x, lo2.y, hi2.x, hi2.y});
#pragma unroll
        for (int s = 0; s < QT; ++s)
          oacc[s][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[s][kk], oacc[s][dt], 0, 0, 0);
      }
    }

    wait_loads_then_barrier();
  }

  // normalise and write: O^T -> LDS [32 q][128 d] per wave (8-byte quads
  // swizzled by q) -> panel rows (a row's 128 dims are four 64-byte runs)
  bf16_t* so = &sK[0][0] + wave * (32 * FA_DH);
#pragma unroll
  for (int s = 0; s < QT; ++s) {
    const float inv = 1.0f / l_run[s];
    const int ql = lane & 31;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        const int u = dt * 8 + vq * 2 + hh;  // quad of dims dt*32 + 8*vq + 4*hh .. +3
        u32x2_t w;
        w.x = pack_bf16x2(oacc[s][dt][vq * 4 + 0] * inv, oacc[s][dt][vq * 4 + 1] * inv);
        w.y = pack_bf16x2(oacc[s][dt][vq * 4 + 2] * inv, oacc[s][dt][vq * 4 + 3] * inv);
        *reinterpret_cast<u32x2_t*>(so + ql * FA_DH + ((u ^ ql) << 2)) = w;
      }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int idx = it * 64 + lane;
      const int ql2 = idx >> 5, u = idx & 31;
      const int qi = q0 + s * 32 + ql2;
      if (qi < N) {
        u32x2_t w = *reinterpret_cast<const u32x2_t*>(so + ql2 * FA_DH + ((u ^ ql2) << 2));
        *reinterpret_cast<u32x2_t*>(o + panel_off(tok0 + qi, h * FA_DH + u * 4, dq)) = w;
      }
    }
    __syncthreads();
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
template <typename T, int DH>
__global__ __launch_bounds__(256) void attn_rows_kernel(const T* __restrict__ q, CacheSlot<T> cache,
                                                        const int32_t* __restrict__ row_seq,
                                                        const int32_t* __restrict__ row_pos,
                                                        const int32_t* __restrict__ bt, int max_blocks, int hq,
                                                        int nchunks, float scale, float* __restrict__ ws) {
  constexpr int VEC = 16 / (int)sizeof(T);  // elements per lane load
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
        const T* kr = cache.k + kv_index(sl_s[kk], g, d0, hkv, DH);
        const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(kr);
        float kv[VEC];
        unpack16<T>(raw, kv);
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
        for (int off = 1; off < LPK; off <<= 1) part[hh] += __shfl_xor(part[hh], off);
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
      float m = warp_max(ps[hh][tid]);
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
      const float sm = warp_sum(p);
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
        const T* vr = cache.v + kv_index(sl_s[kk], g, d0, hkv, DH);
        const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(vr);
        float vv[VEC];
        unpack16<T>(raw, vv);
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
        for (int off = LPK; off < 64; off <<= 1) acc[hh][e] += __shfl_xor(acc[hh][e], off);
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

template <typename T>
__global__ void attn_combine_kernel(const float* __restrict__ ws, int hq, int dh, int nchunks, T* __restrict__ o) {
  const int r = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  if (d >= dh) return;
  const int stride = dh + 2;
  const float* w = ws + ((int64_t)r * hq + h) * nchunks * stride;
  float m = -INFINITY;
  for (int c = 0; c < nchunks; ++c) m = fmaxf(m, w[c * stride]);
  float l = 0.f, acc = 0.f;
  for (int c = 0; c < nchunks; ++c) {
    float mc = w[c * stride];
    if (mc == -INFINITY) continue;
    float e = __expf(mc - m);
    l += w[c * stride + 1] * e;
    acc += w[c * stride + 2 + d] * e;
  }
  o[((int64_t)r * hq + h) * dh + d] = from_f32<T>(acc / l);
}

}  // namespace

hipError_t launch_attn_prefill_bf16(const bf16_t* q, CacheSlot<bf16_t> cache, const int32_t* cu_seqlens,
                                    const int32_t* block_tables, int max_blocks, int batch, int max_seqlen, int hq,
                                    bf16_t* o, hipStream_t stream) {
  if (batch <= 0 || max_seqlen <= 0) return hipSuccess;
  constexpr int QT = 1;
  const int rep = hq / cache.hkv;
  dim3 grid((max_seqlen + 32 * QT - 1) / (32 * QT), batch, hq / 4);
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)FA_DH);
  hipLaunchKernelGGL(attn_prefill_kernel<QT>, grid, dim3(256), 0, stream, q, cache, cu_seqlens, block_tables,
                     max_blocks, hq, rep, scale_log2, o);
  return hipGetLastError();
}

int64_t attn_rows_ws_elems(int rows, int max_ctx, int hq, int dh) {
  int nchunks = (max_ctx + RW_CH - 1) / RW_CH;
  return (int64_t)rows * hq * nchunks * (dh + 2);
}

template <typename T>
hipError_t launch_attn_rows(const T* q, CacheSlot<T> cache, const int32_t* row_seq, const int32_t* row_pos,
                            const int32_t* block_tables, int max_blocks, int rows, int max_ctx, int hq, float* ws,
                            T* o, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const int nchunks = (max_ctx + RW_CH - 1) / RW_CH;
  const float scale = 1.0f / sqrtf((float)cache.dh);
  const dim3 grid(rows, cache.hkv, nchunks);
  switch (cache.dh) {
    case 128:
      hipLaunchKernelGGL((attn_rows_kernel<T, 128>), grid, dim3(256), 0, stream, q, cache, row_seq, row_pos,
                         block_tables, max_blocks, hq, nchunks, scale, ws);
      break;
    case 64:
      hipLaunchKernelGGL((attn_rows_kernel<T, 64>), grid, dim3(256), 0, stream, q, cache, row_seq, row_pos,
                         block_tables, max_blocks, hq, nchunks, scale, ws);
      break;
    case 32:
      hipLaunchKernelGGL((attn_rows_kernel<T, 32>), grid, dim3(256), 0, stream, q, cache, row_seq, row_pos,
                         block_tables, max_blocks, hq, nchunks, scale, ws);
      break;
    default:
      return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel<T>, dim3(rows, hq), dim3(RW_MAXDH), 0, stream, ws, hq, cache.dh, nchunks, o);
  return hipGetLastError();
}

template hipError_t launch_attn_rows<float>(const float*, CacheSlot<float>, const int32_t*, const int32_t*,
                                            const int32_t*, int, int, int, int, float*, float*, hipStream_t);
template hipError_t launch_attn_rows<bf16_t>(const bf16_t*, CacheSlot<bf16_t>, const int32_t*, const int32_t*,
                                             const int32_t*, int, int, int, int, float*, bf16_t*, hipStream_t);
