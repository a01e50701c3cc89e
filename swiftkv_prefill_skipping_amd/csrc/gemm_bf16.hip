// bf16 MFMA GEMM for gfx950: C[M,N] = A[M,K] . B[N,K]^T with fp32
// accumulation, results handed to an epilogue functor eight column pairs
// (col + e, col + 64 + e) at a time.
//
// Operands are in the panel layout (common.h): 256-row panels stored as
// contiguous [256][32] blocks, so the k-stage s of an output tile is one
// contiguous 16 KB block of A's panel and one of B's.
//
// Tile 256 x 256, k-stages of 32.  256 threads = 4 wave64s, one per SIMD;
// wave w owns output rows 128*(w&1) .. +128 and columns 128*(w>>1) .. +128
// as 8 x 8 tiles of v_mfma_f32_16x16x32_bf16 (256 accumulator registers).
// The 16x16x32 form rather than 32x32x16: with operands whose bits toggle
// like these weights', a CU full of back-to-back 32x32x16 MFMAs draws the
// chip to its power limit at ~1.83 GHz (1.84 PFLOP/s), while the same work
// as 16x16x32 MFMAs holds ~2.13 GHz (2.10 PFLOP/s); with constant operands
// both run at ~2.39 GHz.  The MFMA takes the B fragment as its first
// operand, so each lane ends up holding one output row (lane & 15) and runs
// of four consecutive columns.
//
// Operand staging: global -> LDS directly (global_load_lds_dwordx4, no
// register round trip) into a ring of kNBuf 32 KB stages, kNBuf - 1 of them
// in flight while one is multiplied.  LDS rows are 64 B (32 bf16); the 16 B
// chunk c of row r is stored at chunk c ^ ((r >> 1) & 3), which the
// bank-conflict counter shows conflict free for the fragment reads (see
// swizzle()).
//
// Schedule: each k-stage is 64 MFMAs in two halves (row tiles 0..3, then
// 4..7, every column tile).  The first half reads the second half's A
// fragments; the second half reads the next stage's fragments (A row tiles
// 0..3 into the registers the first half freed, the B fragments into a
// second set, the two sets alternating by stage parity), all early enough
// to land before the next stage needs them.  One workgroup barrier per
// stage, between the halves, publishes the next stage and frees the
// current buffer, whose next load goes out in two halves, one in each of
// the following two half-stages, between their MFMAs.
//
// Epilogue: the accumulators go through LDS (each wave stages 32 rows x 128
// columns of fp32 at a time in a padded, conflict-free layout), so the
// epilogue functor sees eight consecutive columns per call and every global
// store is a whole 16-byte run.  The SwiGLU epilogue skips the staging: a
// lane already holds each gate column next to its up partner.
//
// A partly filled last wave of tiles is split over K into units of a second
// launch; gemm_reduce_kernel sums their fp32 partial tiles in fixed order.
//
// Workgroups are dispatched round robin over the 8 XCDs; the tile index is
// remapped so each XCD processes a contiguous run of tiles, and runs are
// ordered in groups of kGroupM row tiles so concurrently resident tiles share
// A and B panels in that XCD's L2.
#include <type_traits>

#include "common.h"
#include "epilogues.h"
#include "kernels.h"

namespace {

constexpr int BM = 256, BN = 256;
constexpr int kNBuf = 4;  // LDS stages (32-column k-blocks) in flight
constexpr int kThreads = 256;
constexpr int kGroupM = 4;
constexpr int kXcds = 8;
// epilogue staging: 32 rows x 128 fp32 columns per wave, rows padded by 4
// floats so that both the column-run writes and the row reads are
// conflict free
constexpr int kStageLd = 132;
constexpr int kStageWave = 32 * kStageLd;  // floats

SKV_DEV int xcd_remap(int wg, int n) {
  int q = n / kXcds, r = n % kXcds;
  int xcd = wg % kXcds, local = wg / kXcds;
  return (xcd < r) ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
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

// Wait for this wave's direct loads (all but the N most recent) and LDS
// reads, then a workgroup barrier.  (__syncthreads would add a fence; the
// memory clobber and the scheduling barriers keep every LDS access and MFMA
// on its side.)
template <int N>
SKV_DEV void wait_vm_then_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
  __builtin_amdgcn_sched_barrier(0);
}
SKV_DEV void wait_lds_then_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
SKV_DEV void wait_lds() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Physical 16-byte chunk of logical chunk 0 in LDS row `row` (XOR
// swizzle).  A fragment read (ds_read_b128) has lane l read row l & 15 of
// a 16-row block at logical chunk l >> 4.  With 64-byte rows (4 chunks) the
// chunk is XORed with (row >> 1) & 3: the bank-conflict counter reads 0.00
// cycles per instruction for that pattern on gfx950, against 3.98 for
// (row >> 2) & 3 and for no swizzle (a probe of each address pattern alone,
// SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS).  With 8 chunks (128-byte rows),
// (row >> 1) & 7 measured conflict free as well.
template <int CH>
SKV_DEV int swizzle(int row) {
  return CH == 8 ? (row >> 1) & 7 : (row >> 1) & 3;
}

// Shape of one k-stage of BK columns: LDS rows are BK bf16 = CH chunks of
// 16 B; one direct load instruction moves RPI rows; each wave issues LPW of
// them per stage; a stage is NSUB k-substeps of 16.
template <int BK>
struct StageShape {
  static constexpr int CH = BK / 8;
  static constexpr int RPI = 64 / CH;
  static constexpr int LPW = (BM + BN) / RPI / 4;
  static constexpr int NSUB = BK / 16;
};

// What an epilogue reads, and when.  Every read is issued before the
// stores it would otherwise wait behind (one vector-memory counter covers
// loads and stores on gfx9):
//   Lane: per-lane constants (a lane's columns are the same in every
//         pass), read at the start of the epilogue;
//   Row:  per-row values of each of the lane's 16 rows, read at the start
//         of the epilogue;
//   Pre:  per-unit values, read one pass ahead (before the previous pass's
//         stores).
// The defaults read nothing.
template <class Epi>
struct EpiAhead {
  struct Lane {};
  struct Row {};
  struct Pre {};
  static SKV_DEV Lane lane(const Epi&, int) { return {}; }
  static SKV_DEV Row row(const Epi&, int) { return {}; }
  static SKV_DEV Pre load(const Epi&, int, int, const Row&) { return {}; }
  static SKV_DEV void apply(const Epi& e, int row, int col, const float* a, const float* b, const Lane&, const Row&,
                            const Pre&) {
    e.vec8(row, col, a, b);
  }
};
// RoPE / KV-cache epilogues: each row's RMSNorm factor, position and cache
// slot up front; a unit's RoPE rotation (q and k columns) one pass ahead.
template <class Epi>
struct EpiAheadRope {
  struct Lane {};
  using Row = RowInfo;
  struct Pre {
    float c[8], s[8];
  };
  static SKV_DEV Lane lane(const Epi&, int) { return {}; }
  static SKV_DEV Row row(const Epi& e, int r) { return e.row_info(r); }
  static SKV_DEV Pre load(const Epi& e, int, int col, const Row& ri) {
    Pre p;
    if (e.roped(col)) e.rope_tab(ri.pos, col, p.c, p.s);
    return p;
  }
  static SKV_DEV void apply(const Epi& e, int row, int col, const float* a, const float* b, const Lane&,
                            const Row& ri, const Pre& p) {
    e.vec8t(row, col, a, b, ri, p.c, p.s);
  }
};
template <>
struct EpiAhead<EpiQKV<bf16_t>> : EpiAheadRope<EpiQKV<bf16_t>> {};
template <>
struct EpiAhead<EpiKVSkip<bf16_t>> : EpiAheadRope<EpiKVSkip<bf16_t>> {};
// Residual add: the next RMSNorm's gains of the lane's columns up front,
// the residual values it updates one pass ahead.
template <>
struct EpiAhead<EpiResidual> {
  struct Lane {
    float g0[8], g1[8];
  };
  struct Row {};
  using Pre = EpiResidual::Pre;
  static SKV_DEV Lane lane(const EpiResidual& e, int col) {
    Lane l;
    e.gains8(col, l.g0, l.g1);
    return l;
  }
  static SKV_DEV Row row(const EpiResidual&, int) { return {}; }
  static SKV_DEV Pre load(const EpiResidual& e, int row, int col, const Row&) { return e.pre8(row, col); }
  static SKV_DEV void apply(const EpiResidual& e, int row, int col, const float* a, const float* b, const Lane& l,
                            const Row&, const Pre& p) {
    e.vec8g(row, col, a, b, p, l.g0, l.g1);
  }
};

// Epilogues with kFromRegisters take their column pairs straight from the
// accumulators (vec4x2s) instead of through the LDS staging.
template <class Epi, class = void>
struct FromRegisters {
  static constexpr bool value = false;
};
template <class Epi>
struct FromRegisters<Epi, decltype((void)Epi::kFromRegisters)> {
  static constexpr bool value = Epi::kFromRegisters;
};

// Work split of one GEMM.  The first dp_tiles tiles are computed whole
// (data parallel, one launch, XCD remapped); each of the remaining tiles is
// split along K into `splits` ranges (a partly filled last wave of tiles
// becomes K-split units that fill every CU), one workgroup per range in a
// second launch, whose fp32 partial tiles go to `ws` and are summed in
// fixed order by gemm_reduce_kernel.
struct SplitPlan {
  int dp_tiles;
  int splits;
  float* ws;
};

// SPLIT selects the launch: false = the whole tiles (grid dp_tiles, XCD
// remapped), true = the K-split units of the tail tiles (grid (tiles -
// dp_tiles) * splits), whose fp32 partial tiles go to plan.ws.  Separate
// kernels keep one epilogue per kernel, so neither path's register needs
// shape the other's.
template <int NBUF, class Epi, bool SPLIT>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(const bf16_t* __restrict__ A,
                                                                 const bf16_t* __restrict__ B, int M, int N,
                                                                 int K, SplitPlan plan, Epi epi) {
  constexpr int BK = kPanelCols;  // one k-stage = one 32-column block of a panel
  constexpr int CH = StageShape<BK>::CH, RPI = StageShape<BK>::RPI, LPW = StageShape<BK>::LPW;
  constexpr int NSUB = StageShape<BK>::NSUB;
  static_assert(NSUB % 2 == 0 && NBUF >= 2, "stage shape");
  __shared__ __attribute__((aligned(1024))) bf16_t smem[NBUF][(BM + BN) * BK];

  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + BN - 1) / BN;
  const int nk_all = K / BK;
  const int bid = blockIdx.x;
  constexpr bool split = SPLIT;
  int tile, kb, ke, unit = 0;
  if (!split) {
    tile = xcd_remap(bid, plan.dp_tiles);
    kb = 0;
    ke = nk_all;
  } else {
    unit = bid;
    tile = plan.dp_tiles + unit / plan.splits;
    const int sp = unit % plan.splits;
    // ranges in whole pairs of stages: every range has an even stage count
    kb = 2 * (sp * (nk_all / 2) / plan.splits);
    ke = 2 * ((sp + 1) * (nk_all / 2) / plan.splits);
  }
  int tm, tn;
  tile_coords(tile, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..3, one per SIMD
  const int wm = wave & 1, wn = wave >> 1;                    // 128 x 128 output block

  // Direct global -> LDS loads.  Stage s of row panel tm of A is the
  // contiguous 16 KB block a_panel + s * 8192 (likewise B), so every load
  // instruction moves one contiguous 1 KB run (RPI = 16 rows of 64 B).  Lane
  // l's 16 bytes land at byte 16*l of the instruction's LDS destination, so
  // the XOR swizzle of the LDS layout is applied on the global side: lane l
  // fetches the logical chunk of row l / CH that belongs at physical chunk
  // l % CH.  Wave w moves row groups w*LPW/2 .. +LPW/2 of both A and B.
  constexpr int LH = LPW / 2;
  const int nkb = K / BK;
  // (from stage kb on: the loads below count stages from the range start)
  const bf16_t* a_panel = A + ((int64_t)tm * nkb + kb) * (BM * BK);
  const bf16_t* b_panel = B + ((int64_t)tn * nkb + kb) * (BN * BK);
  int g_off[LH];
#pragma unroll
  for (int i = 0; i < LH; ++i) {
    const int row = (wave * LH + i) * RPI + lane / CH;
    g_off[i] = row * BK + (((lane % CH) ^ swizzle<CH>(row)) << 3);
  }
  // loads i0 .. i1-1 of stage stage_idx (two instructions each, A and B)
  auto gload_part = [&](int buf, int stage_idx, int i0, int i1) {
    typedef __attribute__((address_space(3))) void* lds_ptr;
    const int64_t so = (int64_t)stage_idx * (BM * BK);
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      const int grp = wave * LH + i;
      const bf16_t* sa = a_panel + so + g_off[i];
      const bf16_t* sb = b_panel + so + g_off[i];
      __builtin_amdgcn_global_load_lds(sa, (lds_ptr)(&smem[buf][grp * RPI * BK]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(sb, (lds_ptr)(&smem[buf][BM * BK + grp * RPI * BK]), 16, 0, 0);
    }
  };
  auto gload = [&](int buf, int stage_idx) { gload_part(buf, stage_idx, 0, LH); };

  f32x4_t acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // A fragment (16 rows x 32 k): lane l holds row l & 15, k-chunk l >> 4;
  // rows 16 apart share the swizzle
  const int frag_row = lane & 15;
  const int swz = swizzle<CH>(frag_row);
  const int fch = ((lane >> 4) ^ swz) << 3;
  const int a_off = (wm * 128 + frag_row) * BK + fch;
  const int b_off = BM * BK + (wn * 128 + frag_row) * BK + fch;

  // fragments: 8 A row tiles of the current stage, 8 B column tiles in
  // each of two sets (set = stage parity)
  bf16x8_t af[8], bfr[2][8];
  auto read_a = [&](int buf, int i) {
    af[i] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(smem[buf] + a_off + i * 16 * BK));
  };
  auto read_b = [&](int set, int buf, int j) {
    bfr[set][j] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(smem[buf] + b_off + j * 16 * BK));
  };
  // acc[i][j] (transposed tile): lane holds output row i*16 + (lane & 15),
  // columns j*16 + 4*(lane/16) + v
  auto mfma = [&](int set, int i, int j) {
    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[set][j], af[i], acc[i][j], 0, 0, 0);
  };

  // Epilogue geometry.  unit (pass i, it): row wm*128 + i*32 + it*8 + er,
  // columns lcol.. and lcol+64..  What the epilogue reads (residual values,
  // row factors) for pass i+1 is loaded before pass i's stores are issued:
  // the vector-memory counter covers stores too, so a load issued after
  // them would make its wait cover them as well.  (Loading pass 0 during the
  // last k-stages instead was measured slower: every CU reaches its epilogue
  // at the same time, so those loads only move the HBM burst earlier.)
  const int er = lane >> 3;       // row within a group of 8
  const int ec = (lane & 7) * 8;  // first of eight columns, 0..56
  const int lcol = wn * 128 + ec;
  const bool cols_ok = n0 + wn * 128 < N;
  using Ahead = EpiAhead<Epi>;
  typename Ahead::Lane lane_c;
  typename Ahead::Row rows[4][4];
  typename Ahead::Pre ahead[2][4];
  auto unit_row = [&](int i, int it) { return wm * 128 + i * 32 + it * 8 + er; };
  auto load_rows = [&]() {
    lane_c = Ahead::lane(epi, n0 + lcol);
#pragma clang loop unroll(full)
    for (int i = 0; i < 4; ++i)
#pragma clang loop unroll(full)
      for (int it = 0; it < 4; ++it)
        if (m0 + unit_row(i, it) < M) rows[i][it] = Ahead::row(epi, m0 + unit_row(i, it));
  };
  auto load_pass = [&](int i) {
#pragma clang loop unroll(full)
    for (int it = 0; it < 4; ++it)
      if (m0 + unit_row(i, it) < M) ahead[i & 1][it] = Ahead::load(epi, m0 + unit_row(i, it), n0 + lcol, rows[i][it]);
  };

  const int nk = ke - kb;
  static_assert(NSUB == 2 && LH % 2 == 0 && LH / 2 == 2, "32-deep stages, loads in two halves of 4");

  // Pipeline: all NBUF buffers are filled up front.  The barrier in the
  // middle of stage s publishes stage s+1 (every wave has landed its share)
  // and frees the buffer of stage s (its fragments are in registers by
  // then).  Stage s+NBUF then goes into that buffer in two halves: the
  // first during the second half of stage s, the second during the first
  // half of stage s+1, so each half-stage's 32 MFMAs carry LPW/2 direct
  // loads and the load issue never bunches up behind the barrier.  At the
  // barrier of stage s the loads issued after stage s+1's are those of
  // stages s+2 and s+3 (LPW each), whenever both exist; near the end the
  // wait drains all.  The flags are constants at each call site, so every
  // stage body is one straight-line block and the group barriers interleave
  // its loads and LDS reads with the MFMAs.
  //   load_a: first half of stage s+NBUF, after the barrier
  //   load_b: second half of stage s+NBUF-1, before the barrier
  auto stage = [&](auto parity, int s, bool load_a, bool load_b, bool next) {
    constexpr int P = decltype(parity)::value;
    const int cur = s % NBUF, nxt = (s + 1) % NBUF;
    // first half: row tiles 0..3; reads the A fragments of row tiles 4..7
    // and issues the second half of the previous stage's load
#pragma unroll
    for (int i = 4; i < 8; ++i) read_a(cur, i);
    if (load_b) gload_part((s + NBUF - 1) % NBUF, s + NBUF - 1, LH / 2, LH);
    // A fragment outer: eight MFMAs in a row share their second operand
    // (measured 0.3-1.2 % faster per call than B outer, 4 alternating runs
    // on one box, on every shape of the step)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) mfma(P, i, j);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    if (load_b) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
    } else {
      __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (next) {
      if (load_a || load_b) wait_vm_then_barrier<2 * LPW>();
      else wait_vm_then_barrier<0>();
    }
    // second half: row tiles 4..7; reads the next stage's fragments (A
    // row tiles 0..3, the other B set) and issues the first half of stage
    // s+NBUF into the freed buffer
    if (next) {
#pragma unroll
      for (int i = 0; i < 4; ++i) read_a(nxt, i);
#pragma unroll
      for (int j = 0; j < 8; ++j) read_b(1 - P, nxt, j);
    }
    if (load_a) gload_part(cur, s + NBUF, 0, LH / 2);
#pragma unroll
    for (int i = 4; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) mfma(P, i, j);
    if (next) {
#pragma unroll
      for (int g = 0; g < 12; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    if (load_a) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // every range has at least NBUF stages: fill the ring, wait for stage 0
  for (int p = 0; p < NBUF; ++p) gload(p, p);
  wait_vm_then_barrier<(NBUF - 1) * LPW>();
#pragma unroll
  for (int j = 0; j < 8; ++j) read_b(0, 0, j);
#pragma unroll
  for (int i = 0; i < 4; ++i) read_a(0, i);
  __builtin_amdgcn_sched_barrier(0);
  // Stage s of nk (nk even and >= 6, so every call site knows its parity):
  //   load_a = s < nk - NBUF, load_b = 1 <= s <= nk - NBUF, next = s < nk - 1
  using Even = std::integral_constant<int, 0>;
  using Odd = std::integral_constant<int, 1>;
  static_assert(NBUF == 4, "stage sequence written for four buffers");
  stage(Even{}, 0, true, false, true);
  for (int s = 1; s < nk - 5; s += 2) {
    stage(Odd{}, s, true, true, true);
    stage(Even{}, s + 1, true, true, true);
  }
  stage(Odd{}, nk - 5, true, true, true);
  stage(Even{}, nk - 4, false, true, true);
  stage(Odd{}, nk - 3, false, false, true);
  stage(Even{}, nk - 2, false, false, true);
  stage(Odd{}, nk - 1, false, false, false);

  // Epilogues that take their pairs from registers (SwiGLU: a lane's gate
  // columns j*16 + 4*(lane/16) + v and their up partners sit in acc[i][j]
  // and acc[i][j+4] for j < 4) skip the LDS staging; each call takes two
  // adjacent column blocks of a row block.  The row bound is the same for
  // lanes l and l + 16, which the call's lane exchange pairs.
  if constexpr (FromRegisters<Epi>::value && !SPLIT) {
    {
      if (!cols_ok) return;
      const int row0 = m0 + wm * 128 + (lane & 15);
      const int col0 = n0 + wn * 128;
      const int rg = lane >> 4;
      float sr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) sr[i] = row0 + i * 16 < M ? epi.scale(row0 + i * 16) : 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (row0 + i * 16 < M) {
#pragma unroll
          for (int j = 0; j < 4; j += 2) {
            const float g0[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
            const float u0[4] = {acc[i][j + 4][0], acc[i][j + 4][1], acc[i][j + 4][2], acc[i][j + 4][3]};
            const float g1[4] = {acc[i][j + 1][0], acc[i][j + 1][1], acc[i][j + 1][2], acc[i][j + 1][3]};
            const float u1[4] = {acc[i][j + 5][0], acc[i][j + 5][1], acc[i][j + 5][2], acc[i][j + 5][3]};
            epi.vec4x2s(row0 + i * 16, col0 + j * 16, g0, u0, g1, u1, sr[i], rg);
          }
        }
        // one row block at a time: bounds the values copied out of the
        // accumulators that are live at once
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
  }

  // Epilogue through LDS.  Every stage load has landed (the last barrier
  // waited for all of them); after this barrier every wave has also finished
  // reading the last stage, so the stage buffers can be reused.
  wait_lds_then_barrier();
  float* stg = reinterpret_cast<float*>(&smem[0][0]) + wave * kStageWave;
  if (!split && cols_ok) {
    load_rows();
    load_pass(0);
  }
#pragma clang loop unroll(full)
  for (int i = 0; i < 4; ++i) {
    // stage rows i*32 .. +32 of this wave's block: tile (2i+h, j) value v
    // is column j*16 + 4*(lane/16) + v of staged row h*16 + (lane & 15)
#pragma clang loop unroll(full)
    for (int h = 0; h < 2; ++h)
#pragma clang loop unroll(full)
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<f32x4_t*>(stg + (h * 16 + (lane & 15)) * kStageLd + j * 16 + 4 * (lane >> 4)) =
            acc[2 * i + h][j];
    wait_lds();
    if (!split && cols_ok && i < 3) load_pass(i + 1);
#pragma clang loop unroll(full)
    for (int it = 0; it < 4; ++it) {
      const int r = it * 8 + er;
      float a[8], b[8];
      load8(stg + r * kStageLd + ec, a);
      load8(stg + r * kStageLd + ec + 64, b);
      const int lrow = unit_row(i, it);
      if (split) {
        float* part = plan.ws + (int64_t)unit * (BM * BN) + lrow * BN + lcol;
        store8(part, a);
        store8(part + 64, b);
      } else if (cols_ok) {
        if (m0 + lrow < M) Ahead::apply(epi, m0 + lrow, n0 + lcol, a, b, lane_c, rows[i][it], ahead[i & 1][it]);
      }
    }
    wait_lds();
  }
}

// Sum the split partial tiles in fixed order and apply the epilogue:
// thread -> (tail tile, row, eight column pairs).
template <class Epi>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(int M, int N, SplitPlan plan, Epi epi) {
  const int tiles_n = (N + BN - 1) / BN;
  const int tiles_m = (M + BM - 1) / BM;
  const int r = blockIdx.y;                               // tail tile
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;  // row * 16 + unit
  const int row = idx >> 4, u = idx & 15;
  const int cl = (u >> 3) * 128 + (u & 7) * 8;  // first column of the unit (pair at +64)
  int tm, tn;
  tile_coords(plan.dp_tiles + r, tiles_m, tiles_n, tm, tn);
  const int grow = tm * BM + row, gcol = tn * BN + cl;
  if (grow >= M || gcol >= N) return;
  const float* part = plan.ws + (int64_t)r * plan.splits * (BM * BN) + row * BN + cl;
  float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, b[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < plan.splits; ++sp) {
    float pa[8], pb[8];
    load8(part + (int64_t)sp * (BM * BN), pa);
    load8(part + (int64_t)sp * (BM * BN) + 64, pb);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] += pa[e];
      b[e] += pb[e];
    }
  }
  epi.vec8(grow, gcol, a, b);
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

// room for 2 partial tiles per CU (128 MB on 256 CUs)
int64_t gemm_bf16_ws_elems() { return (int64_t)2 * num_cus() * BM * BN; }

template <int NBUF, class Epi>
hipError_t launch_gemm_cfg(const bf16_t* A, const bf16_t* B, int M, int N, int K, const Epi& epi, float* ws,
                           int64_t ws_elems, hipStream_t stream) {
  constexpr int BK = kPanelCols;
  if (M <= 0) return hipSuccess;
  // whole pairs of 32-column stages, at least six per tile (and per K-split
  // unit, below)
  if (K % (2 * BK) != 0 || K < 6 * BK || N % 128 != 0) return hipErrorInvalidValue;
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int P = num_cus();
  const int nk = K / BK;
  // A partly filled last wave of whole tiles (or a launch of fewer tiles
  // than CUs) is replaced by K-split units.  The split count s minimises the
  // tail's time in units of one whole tile: waves of units ceil(rem*s/P),
  // each unit taking 1/s of the tile plus a fixed cost (pipeline fill and
  // the fp32 partial-tile store, ~10 % of a tile at K = 4096), plus the
  // summing pass over all rem*s partial tiles (~13 % of a tile per P of
  // them at K = 4096); measured on the MI355X at K = 4096 and 14336.  At
  // least 6 k-stages per unit; partial tiles must fit the workspace.
  SplitPlan plan{tiles, 1, ws};
  const int rem = tiles % P;
  if (ws != nullptr && rem != 0) {
    const double fixed = 0.10 * 4096.0 / K, sum = 0.13 * 4096.0 / K;
    double best = 1.0;
    int best_s = 1;
    const int64_t cap = ws_elems / ((int64_t)BM * BN);
    for (int s = 2; s <= nk / 6 && (int64_t)rem * s <= cap; ++s) {
      const double cost = (double)((rem * s + P - 1) / P) * (1.0 / s + fixed) + sum * rem * s / P;
      if (cost < best) {
        best = cost;
        best_s = s;
      }
    }
    if (best_s >= 2) {
      plan.dp_tiles = tiles - rem;
      plan.splits = best_s;
    }
  }
  if (plan.dp_tiles > 0) {
    hipLaunchKernelGGL((gemm_bf16_kernel<NBUF, Epi, false>), dim3(plan.dp_tiles), dim3(kThreads), 0, stream, A, B, M,
                       N, K, plan, epi);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (plan.dp_tiles == tiles) return hipSuccess;
  hipLaunchKernelGGL((gemm_bf16_kernel<NBUF, Epi, true>), dim3((tiles - plan.dp_tiles) * plan.splits), dim3(kThreads),
                     0, stream, A, B, M, N, K, plan, epi);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gemm_reduce_kernel<Epi>), dim3(BM * 16 / 256, tiles - plan.dp_tiles), dim3(256), 0, stream, M,
                     N, plan, epi);
  return hipGetLastError();
}

template <class Epi>
hipError_t launch_gemm_bf16(const bf16_t* A, const bf16_t* B, int M, int N, int K, const Epi& epi, float* ws,
                            int64_t ws_elems, hipStream_t stream) {
  return launch_gemm_cfg<kNBuf>(A, B, M, N, K, epi, ws, ws_elems, stream);
}

#define SKV_INST_GEMM(E)                                                                                      \
  template hipError_t launch_gemm_bf16<E>(const bf16_t*, const bf16_t*, int, int, int, const E&, float*, int64_t, \
                                          hipStream_t);
SKV_INST_GEMM(EpiQKV<bf16_t>)
SKV_INST_GEMM(EpiKVSkip<bf16_t>)
SKV_INST_GEMM(EpiResidual)
SKV_INST_GEMM(EpiSwiGLU<bf16_t>)
SKV_INST_GEMM(EpiSwiGLUPanel)
SKV_INST_GEMM(EpiStore<bf16_t>)
SKV_INST_GEMM(EpiStoreF32)
