// bf16 MFMA GEMM for gfx950: C[M,N] = A[M,K] . B[N,K]^T with fp32
// accumulation, results handed to an epilogue functor as column pairs
// (col, col + 64).
//
// Tile 256 x 256, k-slices of 32.  512 threads = 8 wave64s, two per SIMD;
// wave w owns output rows 64*(w%4) .. +64 and columns 128*(w/4) .. +128 as
// 2 x 4 tiles of v_mfma_f32_32x32x16_bf16.  A wave's 128 columns are 4
// MFMA column tiles; tiles t and t+2 are 64 columns apart, which is the RoPE
// pair distance for head_dim 128 and the gate/up interleave distance, so
// every epilogue pair sits in one lane.
//
// Operand staging: global -> LDS directly (global_load_lds_dwordx4, no
// register round trip) into a ring of 4 k-slices (4 x 32 KB), loads issued 3
// slices ahead so HBM / infinity-cache latency is covered.  LDS rows are
// 64 B (32 bf16); the 16 B chunk c of row r is stored at chunk
// c ^ ((r >> 2) & 3).  gfx950's LDS serves a ds_read_b128 16 lanes (256 B,
// all 64 banks) per pass; with this swizzle the 16 rows read by one pass
// cover all 16 bank groups, so the reads are conflict free.
//
// The two waves of a SIMD alternate between a memory phase and an MFMA
// phase (ping-pong, separated by workgroup barriers), so the matrix core of
// every SIMD is fed by one wave while the other waits on LDS / VMEM.
//
// Workgroups are dispatched round robin over the 8 XCDs; the tile index is
// remapped so each XCD processes a contiguous run of tiles, and runs are
// ordered in groups of kGroupM row tiles so concurrently resident tiles share
// A rows and B columns in that XCD's L2.
#include "common.h"
#include "epilogues.h"
#include "kernels.h"

namespace {

constexpr int BM = 256, BN = 256, BK = 32;
constexpr int kStages = 4;  // LDS ring of k-slices; loads run kStages-1 slices ahead
constexpr int kThreads = 512;
constexpr int kGroupM = 4;
constexpr int kXcds = 8;

SKV_DEV int xcd_remap(int wg, int n) {
  int q = n / kXcds, r = n % kXcds;
  int xcd = wg % kXcds, local = wg / kXcds;
  return (xcd < r) ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// "s_waitcnt vmcnt(8) lgkmcnt(0); s_barrier" and a bare "s_barrier", written
// out because a workgroup fence (__syncthreads) would also wait for every
// outstanding direct load and empty the ring.  The memory clobber keeps the
// compiler from moving LDS accesses across them.
// sched_barrier(0) on both sides stops the scheduler from moving any
// instruction (MFMAs included) across, which is what keeps the phases apart.
SKV_DEV void wait_ring_and_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
SKV_DEV void barrier_only() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <class Epi>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(const bf16_t* __restrict__ A,
                                                                 const bf16_t* __restrict__ B, int M, int N,
                                                                 int K, int lda, int ldb, Epi epi) {
  __shared__ __attribute__((aligned(16))) bf16_t smem[kStages][(BM + BN) * BK];

  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + BN - 1) / BN;
  const int ntiles = tiles_m * tiles_n;
  const int tile = xcd_remap(blockIdx.x, ntiles);
  // grouped order: kGroupM row tiles walked down, then the next column tile
  const int per_group = kGroupM * tiles_n;
  const int grp_t = tile / per_group;
  const int first_m = grp_t * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int tm = first_m + (tile % per_group) % gsize;
  const int tn = (tile % per_group) / gsize;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7; SIMD = wave & 3
  const int pp = wave >> 2;                                   // ping-pong group
  const int wm = wave & 3, wn = pp;                           // 64 x 128 output block of this wave

  // Direct global -> LDS loads (global_load_lds_dwordx4): one instruction
  // moves 1 KB = 16 rows x 64 B and lane l's 16 bytes land at byte 16*l of
  // the destination, so the XOR swizzle is applied on the global side: lane
  // l fetches the logical chunk of row (l >> 2) that belongs at physical
  // chunk l & 3.  A k-slice is 16 row groups of A and 16 of B; wave w loads
  // groups 4w .. 4w+3 (A for w < 4, B otherwise).
  const bf16_t* gsrc_base;
  int gsrc_off[4];
  int lds_dst[4];
  {
    const int is_b = wave >> 2;
    gsrc_base = is_b ? B : A;
    const int ld = is_b ? ldb : lda;
    const int lim = is_b ? N - 1 : M - 1;
    const int r0 = is_b ? n0 : m0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int grp = (wave & 3) * 4 + i;
      const int row = grp * 16 + (lane >> 2);
      const int c = (lane & 3) ^ ((row >> 2) & 3);
      gsrc_off[i] = min(r0 + row, lim) * ld + c * 8;
      lds_dst[i] = (is_b ? BM * BK : 0) + grp * 16 * BK;
    }
  }
  auto gload = [&](int buf, int k0) {
    bf16_t* base = smem[buf];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds(gsrc_base + gsrc_off[i] + k0,
                                       (__attribute__((address_space(3))) void*)(base + lds_dst[i]), 16, 0, 0);
  };

  f32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{0};

  const int frag_row = lane & 31;
  const int khalf = lane >> 5;
  const int swz = (lane >> 2) & 3;  // (row >> 2) & 3 of the fragment row
  const int a_off = (wm * 64 + frag_row) * BK;
  const int b_off = BM * BK + (wn * 128 + frag_row) * BK;

  // operands of one k-slice: 2 substeps x (2 A + 4 B) fragments
  bf16x8_t af[2][2], bfr[2][4];
  auto fload = [&](int buf) {
    const bf16_t* sa = smem[buf] + a_off;
    const bf16_t* sb = smem[buf] + b_off;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ch = ((ks * 2 + khalf) ^ swz) << 3;
#pragma unroll
      for (int i = 0; i < 2; ++i) af[ks][i] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(sa + i * 32 * BK + ch));
#pragma unroll
      for (int j = 0; j < 4; ++j) bfr[ks][j] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(sb + j * 32 * BK + ch));
    }
  };

  // Ping-pong over the two waves of each SIMD.  Per k-slice every wave runs
  // a memory phase (read its operands of slice kt from LDS, issue its 4
  // direct loads of slice kt+3 into the ring, wait until slice kt+1 has
  // landed) and a compute phase (16 MFMAs), each closed by a workgroup
  // barrier.  Group 1 starts one barrier late, so at any time one wave of a
  // SIMD computes while the other does memory work.  Every wave passes the
  // same number of barriers (1 + 1 + 2 nk).  Slices past the end are dummy
  // loads of slice 0 into a buffer nothing reads again, keeping the
  // outstanding-load count uniform (vmcnt(8) = slices kt+2, kt+3).
  const int nk = K / BK;
#pragma unroll
  for (int st = 0; st < kStages - 1; ++st) gload(st, (st < nk ? st : 0) * BK);
  wait_ring_and_barrier();
  if (pp == 1) barrier_only();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & (kStages - 1);
    fload(cur);
    gload((kt + kStages - 1) & (kStages - 1), (kt + kStages - 1 < nk ? kt + kStages - 1 : 0) * BK);
    wait_ring_and_barrier();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks][i], bfr[ks][j], acc[i][j], 0, 0, 0);
    barrier_only();
  }
  if (pp == 0) barrier_only();

  // epilogue: lane holds column (lane & 31) of each 32x32 tile and rows
  // 8*(v/4) + 4*(lane/32) + (v%4)
  const int col_base = n0 + wn * 128 + (lane & 31);
  const int row_base = m0 + wm * 64 + 4 * (lane >> 5);
#pragma clang loop unroll(full)
  for (int i = 0; i < 2; ++i) {
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
