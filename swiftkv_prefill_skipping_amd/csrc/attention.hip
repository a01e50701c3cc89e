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
//    O^T is transposed through LDS at the end and written 8 bytes per lane.
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

template <int QT>
__global__ __launch_bounds__(256, 1) void attn_prefill_kernel(const bf16_t* __restrict__ q, CacheSlot<bf16_t> cache,
                                                              const int32_t* __restrict__ cu,
                                                              const int32_t* __restrict__ bt, int max_blocks, int hq,
                                                              int rep, float scale_log2, bf16_t* __restrict__ o) {
  // double-buffered K and V tiles, [64 keys][128 dims] each
  __shared__ __attribute__((aligned(16))) bf16_t sK[2][FA_KT * FA_DH];
  __shared__ __attribute__((aligned(16))) bf16_t sV[2][FA_KT * FA_DH];

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
  const int wave = tid >> 6;
  const int hh = lane >> 5;
  const int h = blockIdx.z * 4 + wave;
  const int g = (blockIdx.z * 4) / rep;
  const int hkv = cache.hkv;
  const int dq = hq * FA_DH;

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

  const int kend = min(N, q0 + QB);
  const int ntiles = (kend + FA_KT - 1) / FA_KT;
  const int32_t* btb = bt + (int64_t)b * max_blocks;

  // tile loader: 4 blocks of 16 keys, each block a contiguous [16][128]
  // (key, dim) slab of K and of V; thread -> (key = tid/16, chunk = tid%16)
  u32x4_t rk[4], rv[4];
  auto gload = [&](int kt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int key0 = kt * FA_KT + r * 16;
      int blk = (key0 < N) ? btb[key0 / 16] : -1;
      if (blk >= 0) {
        const int64_t off = ((int64_t)blk * hkv + g) * (16 * FA_DH) + tid * 8;
        rk[r] = *reinterpret_cast<const u32x4_t*>(cache.k + off);
        // values of keys beyond the prompt (stale cache contents) are zeroed
        rv[r] = (key0 + (tid >> 4) < N) ? *reinterpret_cast<const u32x4_t*>(cache.v + off) : u32x4_t{0, 0, 0, 0};
      } else {
        rk[r] = u32x4_t{0, 0, 0, 0};
        rv[r] = u32x4_t{0, 0, 0, 0};
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int key = r * 16 + (tid >> 4);
      int ch = tid & 15;
      const int o = key * FA_DH + ((ch ^ (key & 15)) << 3);
      *reinterpret_cast<u32x4_t*>(&sK[buf][o]) = rk[r];
      *reinterpret_cast<u32x4_t*>(&sV[buf][o]) = rv[r];
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < ntiles) gload(kt + 1);
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

    // online softmax per query column
    bf16x8_t pf[QT][4];
#pragma unroll
    for (int s = 0; s < QT; ++s) {
      const int qi = q0 + s * 32 + (lane & 31);
      const bool need_mask = (k0 + FA_KT - 1 > q0 + s * 32) || (k0 + FA_KT > N);
      float mt = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float x = sacc[s][st][v] * scale_log2;
          if (need_mask) {
            int key = k0 + st * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
            if (key > qi || key >= N) x = -INFINITY;
          }
          sacc[s][st][v] = x;
          mt = fmaxf(mt, x);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float m_new = fmaxf(m_run[s], mt);
      const float alpha = exp2f(m_run[s] - m_new);
      m_run[s] = m_new;
      float ls = 0.f;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float p = exp2f(sacc[s][st][v] - m_new);
          sacc[s][st][v] = p;
          ls += p;
        }
      ls += __shfl_xor(ls, 32, 64);
      l_run[s] = l_run[s] * alpha + ls;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[s][dt][v] *= alpha;
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

    if (kt + 1 < ntiles) sstore(cur ^ 1);
    __syncthreads();
  }

  // normalise and write: O^T -> LDS [32 q][128 d] per wave (8-byte quads
  // swizzled by q) -> global rows
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
        *reinterpret_cast<u32x2_t*>(o + (int64_t)(tok0 + qi) * dq + h * FA_DH + u * 4) = w;
      }
    }
    __syncthreads();
  }
}

constexpr int RW_CH = 256;     // keys per chunk
constexpr int RW_MAXREP = 16;  // q heads per kv head
constexpr int RW_MAXDH = 128;

template <typename T>
__global__ __launch_bounds__(256) void attn_rows_kernel(const T* __restrict__ q, CacheSlot<T> cache,
                                                        const int32_t* __restrict__ row_seq,
                                                        const int32_t* __restrict__ row_pos,
                                                        const int32_t* __restrict__ bt, int max_blocks, int hq,
                                                        int nchunks, float scale, float* __restrict__ ws) {
  __shared__ float qs[RW_MAXREP][RW_MAXDH];
  __shared__ float ps[RW_MAXREP][RW_CH];
  __shared__ int sl_s[RW_CH];
  __shared__ float red[RW_MAXREP][4];
  __shared__ float opart[256 / 32][RW_MAXDH];  // 256 / head_dim key partitions (head_dim >= 32)

  const int r = blockIdx.x, g = blockIdx.y, c = blockIdx.z;
  const int tid = threadIdx.x;
  const int hkv = cache.hkv, dh = cache.dh;
  const int rep = hq / hkv;
  const int ctx = row_pos[r] + 1;
  const int seq = row_seq[r];
  const int kbeg = c * RW_CH;
  const int stride = dh + 2;
  float* wsr = ws + ((int64_t)r * hq + g * rep) * nchunks * stride;

  if (kbeg >= ctx) {  // empty chunk
    for (int hl = tid; hl < rep; hl += 256) {
      float* w = wsr + ((int64_t)hl * nchunks + c) * stride;
      w[0] = -INFINITY;
      w[1] = 0.f;
    }
    return;
  }
  for (int i = tid; i < rep * dh; i += 256) {
    int hl = i / dh, d = i % dh;
    qs[hl][d] = to_f32<T>(q[((int64_t)r * hq + g * rep + hl) * dh + d]);
  }
  const int key = kbeg + tid;
  const bool valid = key < ctx;
  int sl = -1;
  if (valid) {
    int blk = bt[(int64_t)seq * max_blocks + key / kBlockSize];
    sl = blk * kBlockSize + key % kBlockSize;
  }
  sl_s[tid] = sl;
  __syncthreads();

  float sc[RW_MAXREP];
#pragma unroll
  for (int hl = 0; hl < RW_MAXREP; ++hl) sc[hl] = 0.f;
  if (valid) {
    const T* kr = cache.k + kv_index(sl, g, 0, hkv, dh);
    for (int d = 0; d < dh; ++d) {
      float kv = to_f32<T>(kr[d]);
#pragma unroll
      for (int hl = 0; hl < RW_MAXREP; ++hl)
        if (hl < rep) sc[hl] = fmaf(qs[hl][d], kv, sc[hl]);
    }
  }
  const int w = tid >> 6;
  for (int hl = 0; hl < rep; ++hl) {
    float x = valid ? sc[hl] * scale : -INFINITY;
    float m = warp_max(x);
    if ((tid & 63) == 0) red[hl][w] = m;
    sc[hl] = x;
  }
  __syncthreads();
  float mh[RW_MAXREP];
  for (int hl = 0; hl < rep; ++hl) mh[hl] = fmaxf(fmaxf(red[hl][0], red[hl][1]), fmaxf(red[hl][2], red[hl][3]));
  __syncthreads();
  for (int hl = 0; hl < rep; ++hl) {
    float p = valid ? __expf(sc[hl] - mh[hl]) : 0.f;
    ps[hl][tid] = p;
    float s = warp_sum(p);
    if ((tid & 63) == 0) red[hl][w] = s;
  }
  __syncthreads();

  // P V: thread -> (dim d, part) with parts = 256 / dh key ranges
  const int parts = 256 / dh;
  const int d = tid % dh, part = tid / dh;
  const int span = RW_CH / parts;
  const int nk = min(RW_CH, ctx - kbeg);
  for (int hl = 0; hl < rep; ++hl) {
    float acc = 0.f;
    for (int j = part * span; j < min(nk, (part + 1) * span); ++j) {
      acc = fmaf(ps[hl][j], to_f32<T>(cache.v[kv_index(sl_s[j], g, d, hkv, dh)]), acc);
    }
    opart[part][d] = acc;
    __syncthreads();
    if (tid < dh) {
      float o = 0.f;
      for (int p = 0; p < parts; ++p) o += opart[p][tid];
      float* wp = wsr + ((int64_t)hl * nchunks + c) * stride;
      wp[2 + tid] = o;
      if (tid == 0) {
        wp[0] = mh[hl];
        wp[1] = red[hl][0] + red[hl][1] + red[hl][2] + red[hl][3];
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
  hipLaunchKernelGGL(attn_rows_kernel<T>, dim3(rows, cache.hkv, nchunks), dim3(256), 0, stream, q, cache, row_seq,
                     row_pos, block_tables, max_blocks, hq, nchunks, scale, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel<T>, dim3(rows, hq), dim3(RW_MAXDH), 0, stream, ws, hq, cache.dh, nchunks, o);
  return hipGetLastError();
}

template hipError_t launch_attn_rows<float>(const float*, CacheSlot<float>, const int32_t*, const int32_t*,
                                            const int32_t*, int, int, int, int, float*, float*, hipStream_t);
template hipError_t launch_attn_rows<bf16_t>(const bf16_t*, CacheSlot<bf16_t>, const int32_t*, const int32_t*,
                                             const int32_t*, int, int, int, int, float*, bf16_t*, hipStream_t);
