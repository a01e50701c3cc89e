// Memory-bound kernels: per-token metadata, embedding gather, RMSNorm, row
// gathers and the load-time weight repacking.  Rows are handled by one
// 256-thread workgroup with 16-byte (or 8-byte) contiguous accesses per
// thread so a wavefront reads whole 1 KB spans.
#include "common.h"
#include "epilogues.h"
#include "kernels.h"

namespace {

__global__ void meta_kernel(const int32_t* __restrict__ cu, const int32_t* __restrict__ ctx,
                            const int32_t* __restrict__ bt, int batch, int max_blocks, int num_blocks, int T,
                            int32_t* __restrict__ pos, int32_t* __restrict__ slot, int32_t* __restrict__ last_pos,
                            int32_t* __restrict__ last_row) {
  int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < T) {
    int lo = 0, hi = batch;  // cu[lo] <= t < cu[hi]
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (cu[mid] <= t)
        lo = mid;
      else
        hi = mid;
    }
    int p = (ctx ? ctx[lo] : 0) + t - cu[lo];
    pos[t] = p;
    int bi = p / kBlockSize;
    int blk = bi < max_blocks ? bt[(int64_t)lo * max_blocks + bi] : -1;
    slot[t] = (blk >= 0 && blk < num_blocks) ? blk * kBlockSize + (p % kBlockSize) : -1;
  }
  if (t < batch) {
    last_pos[t] = (ctx ? ctx[t] : 0) + cu[t + 1] - cu[t] - 1;
    last_row[t] = cu[t + 1] - 1;
  }
}

__global__ void token_seq_kernel(const int32_t* __restrict__ cu, int batch, int T, int32_t* __restrict__ seq) {
  int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  int lo = 0, hi = batch;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (cu[mid] <= t)
      lo = mid;
    else
      hi = mid;
  }
  seq[t] = lo;
}

template <typename T>
__global__ void embed_kernel(const int32_t* __restrict__ tok, const T* __restrict__ E, int vocab, int d,
                             float* __restrict__ x) {
  int t = blockIdx.x;
  int id = tok[t];
  float* xr = x + (int64_t)t * d;
  if (id < 0 || id >= vocab) {
    for (int c = threadIdx.x; c < d; c += blockDim.x) xr[c] = 0.f;
    return;
  }
  const T* er = E + (int64_t)id * d;
  for (int c = threadIdx.x; c < d; c += blockDim.x) xr[c] = to_f32<T>(er[c]);
}

template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x, const int32_t* __restrict__ idx,
                                                      const float* __restrict__ gamma, int d, float eps,
                                                      T* __restrict__ y) {
  __shared__ float red[4];
  const int r = blockIdx.x;
  const int src = idx ? idx[r] : r;
  const float* xr = x + (int64_t)src * d;
  float ss = 0.f;
  // d is a multiple of 4: float4 loads
  for (int c = threadIdx.x * 4; c < d; c += 1024) {
    float4 v = *reinterpret_cast<const float4*>(xr + c);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = warp_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = red[0] + red[1] + red[2] + red[3];
  float inv = 1.0f / sqrtf(tot / (float)d + eps);
  T* yr = y + (int64_t)r * d;
  for (int c = threadIdx.x * 4; c < d; c += 1024) {
    float4 v = *reinterpret_cast<const float4*>(xr + c);
    float g0 = 1.f, g1 = 1.f, g2 = 1.f, g3 = 1.f;
    if (gamma) {
      float4 g = *reinterpret_cast<const float4*>(gamma + c);
      g0 = g.x, g1 = g.y, g2 = g.z, g3 = g.w;
    }
    yr[c + 0] = from_f32<T>(v.x * inv * g0);
    yr[c + 1] = from_f32<T>(v.y * inv * g1);
    yr[c + 2] = from_f32<T>(v.z * inv * g2);
    yr[c + 3] = from_f32<T>(v.w * inv * g3);
  }
}

// GEMM input of a row before its RMSNorm factor, plus that factor: y =
// bf16(x * gamma) in the panel layout (gamma NULL = 1), r[row] = 1 /
// sqrt(mean(x^2) + eps).  One wave per row.  split: y has 2d columns, the
// split-bf16 parts of x * gamma (hi at column c, lo at column d + c).
__global__ __launch_bounds__(256) void rows_rms_panel_kernel(const float* __restrict__ x, const float* __restrict__ gamma,
                                                             int rows, int d, float eps, bool split,
                                                             bf16_t* __restrict__ y, float* __restrict__ r_out) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const float* xr = x + (int64_t)r * d;
  float ss = 0.f;
  for (int c = lane * 8; c < d; c += 512) {
    float v[8];
    load8(xr + c, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
    if (gamma) {
      float g[8];
      load8(gamma + c, g);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] *= g[e];
    }
    if (split) {
      store8(y + panel_off(r, c, 2 * d), v);
      store8_lo(y + panel_off(r, d + c, 2 * d), v);
    } else {
      store8(y + panel_off(r, c, d), v);
    }
  }
  ss = warp_sum(ss);
  if (lane == 0) r_out[r] = 1.0f / sqrtf(ss / (float)d + eps);
}

// r[row] = 1 / sqrt(sum of the row's `units` partial sums of squares / d + eps).
// One wave per row: lane l adds partials l, l+64, ... in order, then a fixed
// butterfly across lanes (deterministic).
__global__ __launch_bounds__(256) void rms_from_partials_kernel(const float* __restrict__ ss, int rows, int units,
                                                                int d, float eps, float* __restrict__ r_out) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;  // whole waves
  const float* p = ss + (int64_t)r * units;
  float t = 0.f;
  if (units % 256 == 0) {
    // a lane sums four consecutive partials per 256 (one 16-byte load each,
    // all issued before the adds), then the wave reduces
    for (int u0 = 0; u0 < units; u0 += 256) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(p + u0 + lane * 4);
      t += (v[0] + v[1]) + (v[2] + v[3]);
    }
  } else {
    for (int u = lane; u < units; u += 64) t += p[u];
  }
  t = warp_sum(t);
  if (lane == 0) r_out[r] = 1.0f / sqrtf(t / (float)d + eps);
}

// Row-major [rows, K] -> panel layout with panels of pr rows, eight
// elements (16 bytes) per thread in destination order; rows beyond `rows`
// (panel padding) become zero.
__global__ void to_panels_kernel(const bf16_t* __restrict__ W, int rows, int K, int pr, int64_t n8,
                                 bf16_t* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = i * 8;
    const int64_t blk = e / ((int64_t)pr * kPanelCols);
    const int within = (int)(e % ((int64_t)pr * kPanelCols));
    const int kbs = K / kPanelCols;
    const int r = (int)(blk / kbs) * pr + within / kPanelCols;
    const int k = (int)(blk % kbs) * kPanelCols + within % kPanelCols;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (r < rows) v = *reinterpret_cast<const u32x4_t*>(W + (int64_t)r * K + k);
    *reinterpret_cast<u32x4_t*>(out + e) = v;
  }
}

__global__ void gather_rows_kernel(const float* __restrict__ x, const int32_t* __restrict__ idx, int d,
                                   float* __restrict__ y) {
  int r = blockIdx.x;
  const float* xr = x + (int64_t)idx[r] * d;
  float* yr = y + (int64_t)r * d;
  for (int c = threadIdx.x; c < d; c += blockDim.x) yr[c] = xr[c];
}

// One row per workgroup; a half-wave (32 lanes x 4 values) covers one
// 128-column unit of the sums of squares.
__global__ __launch_bounds__(256) void rows_act_ss_kernel(const float* __restrict__ x, const int32_t* __restrict__ idx,
                                                          const float* __restrict__ gamma, int d,
                                                          float* __restrict__ y, bf16_t* __restrict__ act,
                                                          float* __restrict__ ss) {
  const int r = blockIdx.x;
  const float* xr = x + (int64_t)(idx ? idx[r] : r) * d;
  for (int c = threadIdx.x * 4; c < d; c += 1024) {
    const float4 v = *reinterpret_cast<const float4*>(xr + c);
    if (y) *reinterpret_cast<float4*>(y + (int64_t)r * d + c) = v;
    const float4 g = gamma ? *reinterpret_cast<const float4*>(gamma + c) : float4{1.f, 1.f, 1.f, 1.f};
    const u32x2_t packed{pack_bf16x2(v.x * g.x, v.y * g.y), pack_bf16x2(v.z * g.z, v.w * g.w)};
    *reinterpret_cast<u32x2_t*>(act + (int64_t)r * d + c) = packed;
    float q = v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) q += __shfl_xor(q, o, 64);
    if ((threadIdx.x & 31) == 0) ss[(int64_t)r * (d / 128) + c / 128] = q;
  }
}

template <typename T>
__global__ void fold_rows_kernel(const T* __restrict__ W, const T* __restrict__ gamma, int rows, int cols,
                                 T* __restrict__ out) {
  int64_t n = (int64_t)rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    int c = (int)(i % cols);
    out[i] = from_f32<T>(to_f32<T>(W[i]) * to_f32<T>(gamma[c]));
  }
}

template <typename T>
__global__ void interleave_kernel(const T* __restrict__ gate, const T* __restrict__ up, int f, int d, int P,
                                  T* __restrict__ out) {
  int64_t n = (int64_t)2 * f * d;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    int64_t row = i / d;
    int c = (int)(i % d);
    int blk = (int)(row / (2 * P));
    int w = (int)(row % (2 * P));
    int64_t src_row = (int64_t)blk * P + (w % P);
    out[i] = (w < P) ? gate[src_row * d + c] : up[src_row * d + c];
  }
}

template <typename T>
__global__ void to_f32_kernel(const T* __restrict__ in, int64_t n, float* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = to_f32<T>(in[i]);
}

int grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  return (int)(g > 65536 ? 65536 : (g < 1 ? 1 : g));
}

}  // namespace

hipError_t launch_meta(const int32_t* cu_seqlens, const int32_t* ctx_lens, const int32_t* block_tables, int batch,
                       int max_blocks, int num_blocks, int total_tokens, int32_t* pos, int32_t* slot,
                       int32_t* last_pos, int32_t* last_row, hipStream_t stream) {
  int n = total_tokens > batch ? total_tokens : batch;
  hipLaunchKernelGGL(meta_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, cu_seqlens, ctx_lens, block_tables,
                     batch, max_blocks, num_blocks, total_tokens, pos, slot, last_pos, last_row);
  return hipGetLastError();
}

hipError_t launch_token_seq(const int32_t* cu_seqlens, int batch, int total_tokens, int32_t* seq,
                            hipStream_t stream) {
  if (total_tokens <= 0) return hipSuccess;
  hipLaunchKernelGGL(token_seq_kernel, dim3((total_tokens + 255) / 256), dim3(256), 0, stream, cu_seqlens, batch,
                     total_tokens, seq);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_embed(const int32_t* tok, const T* E, int vocab, int d, int T_, float* x, hipStream_t stream) {
  if (T_ <= 0) return hipSuccess;
  hipLaunchKernelGGL(embed_kernel<T>, dim3(T_), dim3(256), 0, stream, tok, E, vocab, d, x);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_rmsnorm(const float* x, const int32_t* rows_idx, const float* gamma, int rows, int d, float eps,
                          T* y, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_kernel<T>, dim3(rows), dim3(256), 0, stream, x, rows_idx, gamma, d, eps, y);
  return hipGetLastError();
}

hipError_t launch_rows_rms_panel(const float* x, const float* gamma, int rows, int d, float eps, bool split, bf16_t* y,
                                 float* r, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (d % kPanelCols) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rows_rms_panel_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, x, gamma, rows, d, eps, split,
                     y, r);
  return hipGetLastError();
}

hipError_t launch_rms_from_partials(const float* ss, int rows, int d, float eps, float* r, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (d % 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rms_from_partials_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, ss, rows, d / 16, d, eps,
                     r);
  return hipGetLastError();
}

hipError_t launch_to_panels(const bf16_t* W, int rows, int K, int panel_rows, bf16_t* out, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (K % kPanelCols || (panel_rows != kPanelRows && panel_rows != kSkinnyPanelRows)) return hipErrorInvalidValue;
  const int64_t rows_pad = (int64_t)(rows + panel_rows - 1) / panel_rows * panel_rows;
  const int64_t n8 = rows_pad * K / 8;
  hipLaunchKernelGGL(to_panels_kernel, dim3(grid_for(n8)), dim3(256), 0, stream, W, rows, K, panel_rows, n8, out);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const float* x, const int32_t* rows_idx, int rows, int d, float* y,
                              hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(rows), dim3(256), 0, stream, x, rows_idx, d, y);
  return hipGetLastError();
}

hipError_t launch_rows_act_ss(const float* x, const int32_t* rows_idx, const float* gamma, int rows, int d, float* y,
                              bf16_t* act, float* ss, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (d % 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rows_act_ss_kernel, dim3(rows), dim3(256), 0, stream, x, rows_idx, gamma, d, y, act, ss);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_fold_rows(const T* W, const T* gamma, int rows, int cols, T* out, hipStream_t stream) {
  hipLaunchKernelGGL(fold_rows_kernel<T>, dim3(grid_for((int64_t)rows * cols)), dim3(256), 0, stream, W, gamma, rows,
                     cols, out);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_interleave(const T* gate, const T* up, int f, int d, int P, T* out, hipStream_t stream) {
  hipLaunchKernelGGL(interleave_kernel<T>, dim3(grid_for((int64_t)2 * f * d)), dim3(256), 0, stream, gate, up, f, d,
                     P, out);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_to_f32(const T* in, int64_t n, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(to_f32_kernel<T>, dim3(grid_for(n)), dim3(256), 0, stream, in, n, out);
  return hipGetLastError();
}

#define SKV_INST_T(T)                                                                                             \
  template hipError_t launch_embed<T>(const int32_t*, const T*, int, int, int, float*, hipStream_t);              \
  template hipError_t launch_rmsnorm<T>(const float*, const int32_t*, const float*, int, int, float, T*,          \
                                        hipStream_t);                                                             \
  template hipError_t launch_fold_rows<T>(const T*, const T*, int, int, T*, hipStream_t);                         \
  template hipError_t launch_interleave<T>(const T*, const T*, int, int, int, T*, hipStream_t);                   \
  template hipError_t launch_to_f32<T>(const T*, int64_t, float*, hipStream_t);
SKV_INST_T(float)
SKV_INST_T(bf16_t)
