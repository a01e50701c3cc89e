// Pure-MFMA throughput probe (a measurement aid, not part of the method):
// every workgroup runs 4 waves, each issuing back-to-back
// v_mfma_f32_16x16x32_bf16 (the GEMMs' instruction) on 64 independent
// accumulators (the same 8 x 8 arrangement the GEMM's waves use) from
// operands held in registers, with no memory traffic inside the loop.  Lane
// 0 of each workgroup records the shader clock (s_memtime) and the
// constant 100 MHz counter (s_memrealtime) around the loop, from which the
// host derives the clock the chip held.  With random operand bits the
// matrix cores alone reach the chip's power limit, so the result is the
// dense-bf16 ceiling for data like the random-init weights.
#include "common.h"
#include "kernels.h"

namespace {

// MFMAs per loop trip, each 16 x 16 x 32 (16384 FLOPs)
constexpr int kProbeMfmaPerIter = 64;

__global__ __launch_bounds__(256, 1) void mfma_probe_kernel(const bf16x8_t* __restrict__ in, int iters,
                                                            float* __restrict__ out,
                                                            unsigned long long* __restrict__ clk) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = in[i * 64 + lane];
    b[i] = in[(8 + i) * 64 + lane];
  }
  f32x4_t acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  // the sums keep the loop live
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) sum += acc[i][j][e];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
  if (threadIdx.x == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

int mfma_probe_per_iter() { return kProbeMfmaPerIter; }
int mfma_probe_flops_per_mfma() { return 2 * 16 * 16 * 32; }

hipError_t launch_mfma_probe(const bf16x8_t* in, int iters, int grid, float* out, unsigned long long* clk,
                             hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(grid), dim3(256), 0, stream, in, iters, out, clk);
  return hipGetLastError();
}
