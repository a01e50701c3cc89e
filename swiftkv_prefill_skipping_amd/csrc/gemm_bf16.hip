// bf16 MFMA GEMM for gfx950: C[M,N] = A[M,K] . B[N,K]^T with fp32
// accumulation, results handed to an epilogue functor as column pairs
// (col, col + 64).
//
// Tile 256 x 256, k-stages of 64.  512 threads = 8 wave64s, two per SIMD;
// wave w owns output rows 64*(w%4) .. +64 and columns 128*(w/4) .. +128 as
// 2 x 4 tiles of v_mfma_f32_32x32x16_bf16.  A wave's 128 columns are 4
// MFMA column tiles; tiles t and t+2 are 64 columns apart, which is the RoPE
// pair distance for head_dim 128 and the gate/up interleave distance, so
// every epilogue pair sits in one lane.
//
// Operand staging: global -> LDS directly (global_load_lds_dwordx4, no
// register round trip) into two 64 KB stages.  LDS rows are 128 B (64
// bf16); the 16 B chunk c of row r is stored at chunk c ^ ((r >> 1) & 7).
// gfx950's LDS serves a ds_read_b128 16 lanes (256 B, all 64 banks) per
// pass; with this swizzle the 16 rows read by one pass cover all 16 bank
// groups, so the reads are conflict free.
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

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 512;
constexpr int kGroupM = 4;
constexpr int kXcds = 8;

SKV_DEV int xcd_remap(int wg, int n) {
  int q = n / kXcds, r = n % kXcds;
  int xcd = wg % kXcds, local = wg / kXcds;
  return (xcd < r) ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// Workgroup barriers written out: a workgroup fence (__syncthreads) would
// also wait for every outstanding direct load.  sched_barrier(0) on both
// sides keeps the scheduler from moving any instruction (MFMAs included)
// across, which is what keeps the ping-pong phases apart; the memory
// clobber keeps LDS accesses in place at the IR level.
SKV_DEV void barrier_only() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
SKV_DEV void wait_loads_and_reads() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Tile index -> (row tile, column tile) in grouped order: kGroupM row tiles
// walked down, then the next column tile.
SKV_DEV void tile_coords(int tile, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int per_group = kGroupM * tiles_n;
  const int first_m = (tile / per_group) * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  tm = first_m + (tile % per_group) % gsize;
  tn = (tile % per_group) / gsize;
}

// Work split of one launch.  The first dp_tiles tiles are computed whole
// (data parallel, grid blocks 0 .. dp_tiles-1, XCD remapped); each of the
// remaining tiles is split along K into `splits` ranges (stream-K tail),
// one grid block per range, whose fp32 partial tiles go to `ws` and are
// summed in fixed order by gemm_reduce_kernel.
struct SplitPlan {
  int dp_tiles;
  int splits;
  float* ws;
};

template <class Epi>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(const bf16_t* __restrict__ A,
                                                                 const bf16_t* __restrict__ B, int M, int N,
                                                                 int K, int lda, int ldb, SplitPlan plan, Epi epi) {
  __shared__ __attribute__((aligned(16))) bf16_t smem[2][(BM + BN) * BK];

  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + BN - 1) / BN;
  const int nk_all = K / BK;
  const int bid = blockIdx.x;
  const bool split = bid >= plan.dp_tiles;
  int tile, kb, ke, unit = 0;
  if (!split) {
    tile = xcd_remap(bid, plan.dp_tiles);
    kb = 0;
    ke = nk_all;
  } else {
    unit = bid - plan.dp_tiles;
    tile = plan.dp_tiles + unit / plan.splits;
    const int sp = unit % plan.splits;
    kb = sp * nk_all / plan.splits;
    ke = (sp + 1) * nk_all / plan.splits;
  }
  int tm, tn;
  tile_coords(tile, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7; SIMD = wave & 3
  const int pp = wave >> 2;                                   // ping-pong group
  const int wm = wave & 3, wn = pp;                           // 64 x 128 output block of this wave

  // Direct global -> LDS loads (global_load_lds_dwordx4): one instruction
  // moves 1 KB = 8 rows x 128 B (whole cache lines: the vector memory path
  // pays per line, so half-line row segments would halve its throughput)
  // and lane l's 16 bytes land at byte 16*l of the destination, so the XOR
  // swizzle is applied on the global side: lane l fetches the logical chunk
  // of row (l >> 3) that belongs at physical chunk l & 7.  A stage is 32 row
  // groups of A and 32 of B; group 0 loads A, group 1 loads B, 8
  // instructions per wave.
  const bf16_t* gsrc_base;
  int gsrc_off[8];
  int lds_dst[8];
  {
    const int is_b = pp;
    gsrc_base = is_b ? B : A;
    const int ld = is_b ? ldb : lda;
    const int lim = is_b ? N - 1 : M - 1;
    const int r0 = is_b ? n0 : m0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int grp = (wave & 3) * 8 + i;
      const int row = grp * 8 + (lane >> 3);
      const int c = (lane & 7) ^ ((row >> 1) & 7);
      gsrc_off[i] = min(r0 + row, lim) * ld + c * 8;
      lds_dst[i] = (is_b ? BM * BK : 0) + grp * 8 * BK;
    }
  }
  auto gload = [&](int buf, int k0) {
    bf16_t* base = smem[buf];
#pragma unroll
    for (int i = 0; i < 8; ++i)
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
  const int swz = (lane >> 1) & 7;  // (row >> 1) & 7 of the fragment row
  const int a_off = (wm * 64 + frag_row) * BK;
  const int b_off = BM * BK + (wn * 128 + frag_row) * BK;

  // operands of half a stage: 2 k-substeps x (2 A + 4 B) fragments
  bf16x8_t af[2][2], bfr[2][4];
  auto fload = [&](int buf, int half) {
    const bf16_t* sa = smem[buf] + a_off;
    const bf16_t* sb = smem[buf] + b_off;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ch = (((half * 2 + kk) * 2 + khalf) ^ swz) << 3;
#pragma unroll
      for (int i = 0; i < 2; ++i) af[kk][i] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(sa + i * 32 * BK + ch));
#pragma unroll
      for (int j = 0; j < 4; ++j) bfr[kk][j] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(sb + j * 32 * BK + ch));
    }
  };
  auto compute = [&]() {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk][i], bfr[kk][j], acc[i][j], 0, 0, 0);
  };

  // Ping-pong over the two waves of each SIMD: every wave runs the same
  // sequence of phases separated by workgroup barriers -- read the first
  // half of stage s from LDS (and issue its share of the loads of stage s+1
  // into the other buffer), multiply it (16 MFMAs), read the second half and
  // wait for its loads, multiply it -- and group 1 starts one barrier late,
  // so in every slot one wave of each SIMD is on the matrix core while the
  // other reads LDS.  Group 0 reads stage s in slots 4s and 4s+2, group 1 in
  // 4s+1 and 4s+3; the loads of stage s+1 go out in slots 4s / 4s+1, after
  // the last reads of that buffer (stage s-1, slot 4s-1), and each wave
  // waits for them at the end of its second read phase (slot 4s+2 / 4s+3),
  // before stage s+1 is first read in slot 4s+4.  Every wave passes
  // 2 + 4 nk barriers.
  const int nk = ke - kb;
  const int k_base = kb * BK;
  gload(0, k_base);
  wait_loads_and_reads();
  barrier_only();
  if (pp == 1) barrier_only();
  for (int s = 0; s < nk; ++s) {
    const int cur = s & 1;
    fload(cur, 0);
    if (s + 1 < nk) gload(cur ^ 1, k_base + (s + 1) * BK);
    barrier_only();
    compute();
    barrier_only();
    fload(cur, 1);
    wait_loads_and_reads();
    barrier_only();
    compute();
    barrier_only();
  }
  if (pp == 0) barrier_only();

  // epilogue: lane holds column (lane & 31) of each 32x32 tile and rows
  // 8*(v/4) + 4*(lane/32) + (v%4)
  if (split) {
    float* part = plan.ws + (int64_t)unit * (BM * BN);
    const int cl = wn * 128 + (lane & 31);
    const int rl = wm * 64 + 4 * (lane >> 5);
#pragma clang loop unroll(full)
    for (int i = 0; i < 2; ++i)
#pragma clang loop unroll(full)
      for (int j = 0; j < 4; ++j)
#pragma clang loop unroll(full)
        for (int v = 0; v < 16; ++v)
          part[(rl + i * 32 + 8 * (v >> 2) + (v & 3)) * BN + cl + j * 32] = acc[i][j][v];
    return;
  }
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

// Sum the split partial tiles in fixed order and apply the epilogue:
// thread -> (tail tile, row, column pair (c, c + 64)).
template <class Epi>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(int M, int N, SplitPlan plan, Epi epi) {
  const int tiles_n = (N + BN - 1) / BN;
  const int tiles_m = (M + BM - 1) / BM;
  const int r = blockIdx.y;  // tail tile
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;  // row * 128 + pair
  const int row = idx >> 7, pair = idx & 127;
  const int cl = (pair >> 6) * 128 + (pair & 63);
  int tm, tn;
  tile_coords(plan.dp_tiles + r, tiles_m, tiles_n, tm, tn);
  const int grow = tm * BM + row, gcol = tn * BN + cl;
  if (grow >= M || gcol >= N) return;
  const float* part = plan.ws + (int64_t)r * plan.splits * (BM * BN) + row * BN + cl;
  float v0 = 0.f, v1 = 0.f;
  for (int sp = 0; sp < plan.splits; ++sp) {
    v0 += part[(int64_t)sp * (BM * BN)];
    v1 += part[(int64_t)sp * (BM * BN) + 64];
  }
  epi(grow, gcol, v0, v1);
}

int num_cus() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
  }
  return n;
}

}  // namespace

int64_t gemm_bf16_ws_elems() { return (int64_t)num_cus() * BM * BN; }

template <class Epi>
hipError_t launch_gemm_bf16(const bf16_t* A, int lda, const bf16_t* B, int ldb, int M, int N, int K, const Epi& epi,
                            float* ws, int64_t ws_elems, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int P = num_cus();
  const int nk = K / BK;
  // a partly filled last wave of whole tiles is replaced by K-split units
  // that fill every CU (at least 2 k-stages per unit)
  SplitPlan plan{tiles, 1, ws};
  const int rem = tiles % P;
  if (ws != nullptr && tiles >= P && rem != 0) {
    const int splits = min(P / rem, nk / 2);
    if (splits >= 2 && (int64_t)rem * splits * BM * BN <= ws_elems) {
      plan.dp_tiles = tiles - rem;
      plan.splits = splits;
    }
  }
  const int grid = plan.dp_tiles + (tiles - plan.dp_tiles) * plan.splits;
  hipLaunchKernelGGL((gemm_bf16_kernel<Epi>), dim3(grid), dim3(kThreads), 0, stream, A, B, M, N, K, lda, ldb, plan,
                     epi);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.dp_tiles == tiles) return e;
  hipLaunchKernelGGL((gemm_reduce_kernel<Epi>), dim3(BM * 128 / 256, tiles - plan.dp_tiles), dim3(256), 0, stream, M,
                     N, plan, epi);
  return hipGetLastError();
}

#define SKV_INST_GEMM(E)                                                                                      \
  template hipError_t launch_gemm_bf16<E>(const bf16_t*, int, const bf16_t*, int, int, int, int, const E&, float*, \
                                          int64_t, hipStream_t);
SKV_INST_GEMM(EpiQKV<bf16_t>)
SKV_INST_GEMM(EpiKVSkip<bf16_t>)
SKV_INST_GEMM(EpiResidual)
SKV_INST_GEMM(EpiSwiGLU<bf16_t>)
SKV_INST_GEMM(EpiStore<bf16_t>)
SKV_INST_GEMM(EpiStoreF32)
