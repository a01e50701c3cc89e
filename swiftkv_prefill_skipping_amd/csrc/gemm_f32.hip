// fp32 GEMM on the matrix cores for fp32 models: C[M,N] = A[M,K] B[N,K]^T
// with v_mfma_f32_16x16x4f32 (fp32 operands, fp32 accumulation).  A
// 256-thread workgroup computes a 64 x 2P tile: wave w owns rows
// 16w .. 16w + 15 and all 2P columns as 2P/16 accumulator tiles.  The MFMA
// takes the B fragment as its first operand, so lane l holds output row
// l & 15 and columns 16j + 4(l >> 4) + v of tile j; the pair partner of
// column c < P sits in tile j + P/16 of the same lane, so the epilogue's
// pairs (c, c + P) stay in one thread.  Operands are staged through LDS in
// 32-wide k slices.
#include "common.h"
#include "epilogues.h"
#include "kernels.h"

namespace {

template <int P, class Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, const float* __restrict__ B,
                                                       int M, int N, int K, int lda, int ldb, Epi epi) {
  constexpr int BMf = 64, BNf = 2 * P, BKf = 32;
  constexpr int NT = BNf / 16;  // accumulator tiles per wave
  static_assert(P % 16 == 0, "pair distance");
  __shared__ float As[BMf][BKf + 1];
  __shared__ float Bs[BNf][BKf + 1];
  const int m0 = blockIdx.y * BMf, n0 = blockIdx.x * BNf;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, kq = lane >> 4;
  f32x4_t acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

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
#pragma unroll
    for (int kk = 0; kk < BKf; kk += 4) {
      const float a = As[w * 16 + r16][kk + kq];
#pragma unroll
      for (int j = 0; j < NT; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(Bs[j * 16 + r16][kk + kq], a, acc[j], 0, 0, 0);
    }
    __syncthreads();
  }
  const int row = m0 + w * 16 + r16;
  if (row >= M) return;
#pragma unroll
  for (int j = 0; j < NT / 2; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) epi(row, n0 + j * 16 + 4 * kq + v, acc[j][v], acc[j + NT / 2][v]);
}

}  // namespace

template <int P, class Epi>
hipError_t launch_gemm_f32(const float* A, int lda, const float* B, int ldb, int M, int N, int K, const Epi& epi,
                           hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  dim3 grid(N / (2 * P), (M + 63) / 64);
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
