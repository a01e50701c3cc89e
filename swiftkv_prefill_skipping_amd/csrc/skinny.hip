// Skinny bf16 products for the last-token path (at most 32 rows, one per
// prompt): the layer weights are streamed from HBM exactly once, so the
// kernel is laid out for bandwidth.  Each wave64 owns 64 output columns and
// one K split; A (activations, tiny and L2 resident) and B (weights) are
// read 16 bytes per lane straight into v_mfma_f32_16x16x32_bf16 operands.
// B is stored in panels of pr rows (64 for the last-token weights, 256 for
// the weights the prompt-token GEMMs also read) of [pr][32] blocks; the
// wave's 64 columns sit in one panel and each load instruction (16 rows x
// 32 k) reads 1 KB of contiguous memory.
// Split-K partial sums land in an fp32 buffer [splits, 32, N] and a second
// pass adds them in fixed split order (deterministic) and applies the
// epilogue on column pairs (col, col + 64).
#include <type_traits>

#include "common.h"
#include "epilogues.h"
#include "kernels.h"

namespace {

constexpr int SK_ROWS = kSkinnyMaxRows;

// U k-steps of 32 per loop trip: all U x 4 weight loads (and the few
// activation loads) are issued before the MFMAs that consume them, so each
// wave keeps U x 4 KB of weights in flight.
constexpr int SK_U = 4;

__global__ __launch_bounds__(256) void skinny_partial_kernel(const bf16_t* __restrict__ A, int lda,
                                                             const bf16_t* __restrict__ B, int K, int pr, int M,
                                                             int N, int kc, float* __restrict__ partial) {
  const int lane = threadIdx.x & 63;
  const int cb = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (cb * 64 >= N) return;
  const int s = blockIdx.y;
  const int kbeg = s * kc;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  const bool two = M > 16;

  f32x4_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0, 0, 0, 0};

  // columns cb*64 .. +64 sit in panel p at rows r0 ..; k-block kb of the
  // panel starts at (p * K/32 + kb) * pr * 32, row r at + r * 32
  const int64_t blk = (int64_t)pr * kPanelCols;
  const int p = cb * 64 / pr, r0 = cb * 64 - p * pr;
  const bf16_t* bpanel = B + ((int64_t)p * (K / kPanelCols) + kbeg / kPanelCols) * blk + r0 * kPanelCols;
  const bf16_t* bp[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) bp[j] = bpanel + (j * 16 + r16) * kPanelCols + kq;
  const bool a0ok = r16 < M, a1ok = (16 + r16) < M;
  const bf16_t* ap0 = A + (int64_t)r16 * lda + kbeg + kq;
  const bf16_t* ap1 = A + (int64_t)(16 + r16) * lda + kbeg + kq;

  for (int k = 0; k < kc; k += 32 * SK_U) {
    u32x4_t b[SK_U][4], a0[SK_U], a1[SK_U];
#pragma unroll
    for (int u = 0; u < SK_U; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) b[u][j] = *reinterpret_cast<const u32x4_t*>(bp[j] + (int64_t)(k / 32 + u) * blk);
#pragma unroll
    for (int u = 0; u < SK_U; ++u) {
      a0[u] = a0ok ? *reinterpret_cast<const u32x4_t*>(ap0 + k + u * 32) : u32x4_t{0, 0, 0, 0};
      a1[u] = (two && a1ok) ? *reinterpret_cast<const u32x4_t*>(ap1 + k + u * 32) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < SK_U; ++u) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0[u]), as_bf16x8(b[u][j]), acc[0][j], 0, 0, 0);
      if (two) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[1][j] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1[u]), as_bf16x8(b[u][j]), acc[1][j], 0, 0, 0);
      }
    }
  }
  // C layout of 16x16: row 4*(lane/16) + v, column lane % 16
  float* out = partial + (int64_t)s * SK_ROWS * N;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (i == 1 && !two) break;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        int row = i * 16 + 4 * (lane >> 4) + v;
        if (row < M) out[(int64_t)row * N + cb * 64 + j * 16 + r16] = acc[i][j][v];
      }
  }
}

template <class Epi>
__global__ void skinny_finalize_kernel(const float* __restrict__ partial, int M, int N, int nsplit, Epi epi,
                                       SkinnyRowNorm rn) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t half = N / 2;
  if (idx >= (int64_t)M * half) return;  // whole waves: half is a multiple of 64
  const int row = (int)(idx / half);
  const int j = (int)(idx % half);
  const int col = (j / 64) * 128 + (j % 64);
  const int lane = threadIdx.x & 63;
  // the row's RMSNorm partials (a wave's 64 threads share its row), loaded
  // with the splits
  float t = 0.f;
  if (rn.ss_in)
    for (int i = lane; i < rn.nparts; i += 64) t += rn.ss_in[(int64_t)row * rn.nparts + i];
  // splits summed in order; eight at a time so their loads are in flight together
  const float* p = partial + (int64_t)row * N + col;
  const int64_t ss = (int64_t)SK_ROWS * N;
  float v0 = 0.f, v1 = 0.f;
  int s = 0;
  for (; s + 8 <= nsplit; s += 8) {
    float a[8], b[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      a[u] = p[(s + u) * ss];
      b[u] = p[(s + u) * ss + 64];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      v0 += a[u];
      v1 += b[u];
    }
  }
  for (; s < nsplit; ++s) {
    v0 += p[s * ss];
    v1 += p[s * ss + 64];
  }
  if (rn.ss_in) {  // the input was bf16(x) with the gain in the weights: scale by 1 / rms(x)
    const float r = 1.0f / sqrtf(warp_sum(t) * rn.inv_d + rn.eps);
    v0 *= r;
    v1 *= r;
  }
  if constexpr (std::is_same<Epi, EpiResidualRow>::value) {
    const float q = warp_sum(epi(row, col, v0, v1));
    if (lane == 0) rn.ss_out[(int64_t)row * (N / 128) + col / 128] = q;
  } else {
    epi(row, col, v0, v1);
  }
}

// K splits (each a multiple of 256 columns): the fewest that still give
// about 768 waves (3 per CU).  Fewer, longer waves stream the weights
// faster than many short ones (each wave keeps 16 KB of loads in flight and
// writes a partial tile), and the partials to finalize shrink with them;
// measured on the 8B decode step: 5.50 ms at 2048 waves, 5.29 at 1024, 5.08
// at 768, 5.31 at 512.
int choose_splits(int N, int K) {
  const int units = K / 256;
  const int colblocks = N / 64;
  int best = units;
  for (int s = 1; s <= units; ++s)
    if (units % s == 0 && (int64_t)s * colblocks >= 768) {
      best = s;
      break;
    }
  return best;
}

}  // namespace

int64_t skinny_partial_elems(int N, int K) { return (int64_t)choose_splits(N, K) * SK_ROWS * N; }

template <class Epi>
hipError_t launch_skinny_bf16(const bf16_t* A, int lda, const bf16_t* B, int panel_rows, int M, int N, int K,
                              float* partial, int64_t partial_elems, const Epi& epi, hipStream_t stream,
                              SkinnyRowNorm rn) {
  if (M <= 0) return hipSuccess;
  if (M > SK_ROWS || K % 256 != 0 || N % 128 != 0 || (panel_rows != kSkinnyPanelRows && panel_rows != kPanelRows))
    return hipErrorInvalidValue;
  if (rn.ss_in && (rn.nparts <= 0 || !(rn.inv_d > 0.f))) return hipErrorInvalidValue;
  if (std::is_same<Epi, EpiResidualRow>::value && !rn.ss_out) return hipErrorInvalidValue;
  const int ns = choose_splits(N, K);
  if ((int64_t)ns * SK_ROWS * N > partial_elems) return hipErrorInvalidValue;
  const int kc = K / ns;
  dim3 grid((N / 64 + 3) / 4, ns);
  hipLaunchKernelGGL(skinny_partial_kernel, grid, dim3(256), 0, stream, A, lda, B, K, panel_rows, M, N, kc,
                     partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t work = (int64_t)M * (N / 2);
  hipLaunchKernelGGL(skinny_finalize_kernel<Epi>, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, stream, partial,
                     M, N, ns, epi, rn);
  return hipGetLastError();
}

template hipError_t launch_skinny_bf16<EpiQKV<bf16_t>>(const bf16_t*, int, const bf16_t*, int, int, int, int, float*,
                                                       int64_t, const EpiQKV<bf16_t>&, hipStream_t, SkinnyRowNorm);
template hipError_t launch_skinny_bf16<EpiResidual>(const bf16_t*, int, const bf16_t*, int, int, int, int, float*,
                                                    int64_t, const EpiResidual&, hipStream_t, SkinnyRowNorm);
template hipError_t launch_skinny_bf16<EpiSwiGLU<bf16_t>>(const bf16_t*, int, const bf16_t*, int, int, int, int,
                                                          float*, int64_t, const EpiSwiGLU<bf16_t>&, hipStream_t, SkinnyRowNorm);
template hipError_t launch_skinny_bf16<EpiStoreF32>(const bf16_t*, int, const bf16_t*, int, int, int, int, float*,
                                                    int64_t, const EpiStoreF32&, hipStream_t, SkinnyRowNorm);
template hipError_t launch_skinny_bf16<EpiKVSkip<bf16_t>>(const bf16_t*, int, const bf16_t*, int, int, int, int,
                                                          float*, int64_t, const EpiKVSkip<bf16_t>&, hipStream_t, SkinnyRowNorm);
template hipError_t launch_skinny_bf16<EpiStore<bf16_t>>(const bf16_t*, int, const bf16_t*, int, int, int, int,
                                                         float*, int64_t, const EpiStore<bf16_t>&, hipStream_t, SkinnyRowNorm);
template hipError_t launch_skinny_bf16<EpiResidualRow>(const bf16_t*, int, const bf16_t*, int, int, int, int, float*,
                                                       int64_t, const EpiResidualRow&, hipStream_t, SkinnyRowNorm);
