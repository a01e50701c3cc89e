// fp32 GEMM on the vector ALUs for fp32 models: C[M,N] = A[M,K] B[N,K]^T.
// 32 x 2P output tile per 256-thread workgroup; thread (c, g) owns columns
// (c, c + P) of RPT consecutive rows, so epilogue pairs stay in one thread.
// Operands are staged through LDS in 32-wide k slices.
#include "common.h"
#include "epilogues.h"
#include "kernels.h"

namespace {

template <int P, class Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, const float* __restrict__ B,
                                                       int M, int N, int K, int lda, int ldb, Epi epi) {
  constexpr int BMf = 32, BNf = 2 * P, BKf = 32;
  constexpr int GROUPS = 256 / P;
  constexpr int RPT = BMf / GROUPS;
  __shared__ float As[BMf][BKf + 1];
  __shared__ float Bs[BNf][BKf + 1];
  const int m0 = blockIdx.y * BMf, n0 = blockIdx.x * BNf;
  const int tid = threadIdx.x;
  const int c = tid % P, rg = tid / P;
  float acc0[RPT], acc1[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) acc0[r] = acc1[r] = 0.f;

  for (int k0 = 0; k0 < K; k0 += BKf) {
    for (int idx = tid; idx < BMf * BKf; idx += 256) {
      int r = idx / BKf, kk = idx % BKf;
      int gr = m0 + r, gk = k0 + kk;
      As[r][kk] = (gr < M && gk < K) ? A[(int64_t)gr * lda + gk] : 0.f;
    }
    for (int idx = tid; idx < BNf * BKf; idx += 256) {
      int r = idx / BKf, kk = idx % BKf;
      int gr = n0 + r, gk = k0 + kk;
      Bs[r][kk] = (gr < N && gk < K) ? B[(int64_t)gr * ldb + gk] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < BKf; ++kk) {
      float b0 = Bs[c][kk], b1 = Bs[c + P][kk];
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        float a = As[rg * RPT + r][kk];
        acc0[r] = fmaf(a, b0, acc0[r]);
        acc1[r] = fmaf(a, b1, acc1[r]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    int row = m0 + rg * RPT + r;
    if (row < M) epi(row, n0 + c, acc0[r], acc1[r]);
  }
}

}  // namespace

template <int P, class Epi>
hipError_t launch_gemm_f32(const float* A, int lda, const float* B, int ldb, int M, int N, int K, const Epi& epi,
                           hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  dim3 grid(N / (2 * P), (M + 31) / 32);
  hipLaunchKernelGGL((gemm_f32_kernel<P, Epi>), grid, dim3(256), 0, stream, A, B, M, N, K, lda, ldb, epi);
  return hipGetLastError();
}

#define SKV_INST_F32(P, E)                                                                                   \
  template hipError_t launch_gemm_f32<P, E>(const float*, int, const float*, int, int, int, int, const E&, \
                                            hipStream_t);
#define SKV_INST_F32_ALL(P)          \
  SKV_INST_F32(P, EpiQKV<float>)     \
  SKV_INST_F32(P, EpiKVSkip<float>)  \
  SKV_INST_F32(P, EpiResidual)       \
  SKV_INST_F32(P, EpiSwiGLU<float>)  \
  SKV_INST_F32(P, EpiStore<float>)   \
  SKV_INST_F32(P, EpiStoreF32)
SKV_INST_F32_ALL(16)
SKV_INST_F32_ALL(32)
SKV_INST_F32_ALL(64)
