// bf16 MFMA GEMM for gfx950: C[M,N] = A[M,K] . B[N,K]^T with fp32
// accumulation, results handed to an epilogue functor as column pairs
// (col, col + 64).
//
// Tile 256 x 256 x 64, 256 threads = 4 wave64s in a 2 x 2 arrangement,
// each wave owning a 128 x 128 block as 4 x 4 tiles of
// v_mfma_f32_32x32x16_bf16.  A wave's 128 columns are 4 MFMA column tiles;
// tiles t and t+2 are 64 columns apart, which is the RoPE pair distance for
// head_dim 128 and the gate/up interleave distance, so every epilogue pair
// sits in one lane.
//
// Operand staging: global -> registers (16 B per load) -> LDS, double
// buffered (2 x 64 KB), one barrier per k-step.  LDS rows are 128 B (64
// bf16); the 16 B chunk c of row r is stored at chunk c ^ (r & 7) so that the
// 8 rows read by 8 consecutive lanes hit 8 distinct chunks.
//
// Workgroups are dispatched round robin over the 8 XCDs; the tile index is
// remapped so each XCD processes a contiguous run of tiles, and runs are
// ordered in groups of kGroupM row tiles so concurrently resident tiles share
// A rows and B columns in that XCD's L2.
#include "common.h"
#include "epilogues.h"
#include "kernels.h"

namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 256;
constexpr int kGroupM = 4;
constexpr int kXcds = 8;

SKV_DEV int xcd_remap(int wg, int n) {
  int q = n / kXcds, r = n % kXcds;
  int xcd = wg % kXcds, local = wg / kXcds;
  return (xcd < r) ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

template <class Epi>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(const bf16_t* __restrict__ A,
                                                                 const bf16_t* __restrict__ B, int M, int N,
                                                                 int K, int lda, int ldb, Epi epi) {
  __shared__ __attribute__((aligned(16))) bf16_t smem[2][(BM + BN) * BK];

  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + BN - 1) / BN;
  const int ntiles = tiles_m * tiles_n;
  const int tile = xcd_remap(blockIdx.x, ntiles);
  // grouped order: kGroupM row tiles walked down, then the next column tile
  const int per_group = kGroupM * tiles_n;
  const int grp = tile / per_group;
  const int first_m = grp * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int tm = first_m + (tile % per_group) % gsize;
  const int tn = (tile % per_group) / gsize;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  // global -> LDS mapping: thread loads chunk lc of rows lr + 32 i
  const int lr = tid >> 3, lc = tid & 7;
  const bf16_t* a_src[8];
  const bf16_t* b_src[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int ar = min(m0 + lr + 32 * i, M - 1);
    int br = min(n0 + lr + 32 * i, N - 1);
    a_src[i] = A + (int64_t)ar * lda + lc * 8;
    b_src[i] = B + (int64_t)br * ldb + lc * 8;
  }
  int st_off[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int r = lr + 32 * i;
    st_off[i] = r * BK + ((lc ^ (r & 7)) << 3);
  }

  u32x4_t ra[8], rb[8];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ra[i] = *reinterpret_cast<const u32x4_t*>(a_src[i] + k0);
      rb[i] = *reinterpret_cast<const u32x4_t*>(b_src[i] + k0);
    }
  };
  auto sstore = [&](int buf) {
    bf16_t* sa = smem[buf];
    bf16_t* sb = smem[buf] + BM * BK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *reinterpret_cast<u32x4_t*>(sa + st_off[i]) = ra[i];
      *reinterpret_cast<u32x4_t*>(sb + st_off[i]) = rb[i];
    }
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{0};

  // fragment addresses (elements) inside one buffer, without the k-chunk part
  const int frag_row = lane & 31;
  const int khalf = lane >> 5;
  const int swz = lane & 7;

  const int nk = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
    const bf16_t* sa = smem[cur] + (wm * 128 + frag_row) * BK;
    const bf16_t* sb = smem[cur] + BM * BK + (wn * 128 + frag_row) * BK;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int ch = ((ks * 2 + khalf) ^ swz) << 3;
      bf16x8_t af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(sa + i * 32 * BK + ch));
        bfr[i] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(sb + i * 32 * BK + ch));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds column (lane & 31) of each 32x32 tile and rows
  // 8*(v/4) + 4*(lane/32) + (v%4)
  const int col_base = n0 + wn * 128 + (lane & 31);
  const int row_base = m0 + wm * 128 + 4 * (lane >> 5);
#pragma clang loop unroll(full)
  for (int i = 0; i < 4; ++i) {
#pragma clang loop unroll(full)
    for (int j = 0; j < 2; ++j) {
      const int col = col_base + j * 32;
      if (col >= N) continue;
#pragma clang loop unroll(full)
      for (int v = 0; v < 16; ++v) {
        const int row = row_base + i * 32 + 8 * (v >> 2) + (v & 3);
        if (row < M) epi(row, col, acc[i][j][v], acc[i][j + 2][v]);
      }
    }
  }
}

}  // namespace

template <class Epi>
hipError_t launch_gemm_bf16(const bf16_t* A, int lda, const bf16_t* B, int ldb, int M, int N, int K, const Epi& epi,
                            hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL(gemm_bf16_kernel<Epi>, dim3(tiles), dim3(kThreads), 0, stream, A, B, M, N, K, lda, ldb, epi);
  return hipGetLastError();
}

template hipError_t launch_gemm_bf16<EpiQKV<bf16_t>>(const bf16_t*, int, const bf16_t*, int, int, int, int,
                                                     const EpiQKV<bf16_t>&, hipStream_t);
template hipError_t launch_gemm_bf16<EpiKVSkip<bf16_t>>(const bf16_t*, int, const bf16_t*, int, int, int, int,
                                                        const EpiKVSkip<bf16_t>&, hipStream_t);
template hipError_t launch_gemm_bf16<EpiResidual>(const bf16_t*, int, const bf16_t*, int, int, int, int,
                                                  const EpiResidual&, hipStream_t);
template hipError_t launch_gemm_bf16<EpiSwiGLU<bf16_t>>(const bf16_t*, int, const bf16_t*, int, int, int, int,
                                                        const EpiSwiGLU<bf16_t>&, hipStream_t);
template hipError_t launch_gemm_bf16<EpiStore<bf16_t>>(const bf16_t*, int, const bf16_t*, int, int, int, int,
                                                       const EpiStore<bf16_t>&, hipStream_t);
template hipError_t launch_gemm_bf16<EpiStoreF32>(const bf16_t*, int, const bf16_t*, int, int, int, int,
                                                  const EpiStoreF32&, hipStream_t);
