// Host-side launchers of the gfx950 kernels (internal to libswiftkv).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "epilogues.h"
#include "fp8.h"

// C[M,N] = A[M,K] B[N,K]^T on MFMA (bf16 in, fp32 accumulate), pair distance 64.
// A and B are in the panel layout (panel_off; row counts rounded up to 256,
// padding rows are read but their results are never stored).  Requires
// K % 64 == 0, K >= 192, N % 128 == 0.  ws (gemm_bf16_ws_elems() floats, or NULL)
// holds the split partial tiles of a partly filled last wave.
template <class Epi>
hipError_t launch_gemm_bf16(const bf16_t* A, const bf16_t* B, int M, int N, int K, const Epi& epi, float* ws,
                            int64_t ws_elems, hipStream_t stream);
int64_t gemm_bf16_ws_elems();

// Same product in fp32 on the matrix cores (v_mfma_f32_16x16x4f32, fp32
// models), pair distance P
// (P in {16, 32, 64}); requires N % (2P) == 0.
template <int P, class Epi>
hipError_t launch_gemm_f32(const float* A, int lda, const float* B, int ldb, int M, int N, int K, const Epi& epi,
                           hipStream_t stream);

// Rows one skinny product takes at most.
constexpr int kSkinnyMaxRows = 32;

// Skinny bf16 product for the last-token path (M <= 32 rows): split-K MFMA
// partial sums into `partial` [splits, 32, N] fp32, then a finalize pass
// that reduces them in fixed order and applies the epilogue (pair distance
// 64).  A is row-major [M, lda]; B [N, K] is in the panel layout with
// panels of panel_rows (kSkinnyPanelRows or kPanelRows) rows.  Requires
// K % 256 == 0, N % 128 == 0.
//
// Row RMSNorm applied by the product (rn.ss_in != NULL): A holds
// bf16(x * gain) of the rows, and rn.ss_in [M, nparts] holds partial sums
// of squares of x; the finalize scales each row's products by
// 1 / sqrt(sum * inv_d + eps) before the epilogue.  EpiResidualRow writes
// the new rows' partials (one per 128 columns) to rn.ss_out [M, N / 128].
struct SkinnyRowNorm {
  const float* ss_in = nullptr;
  int nparts = 0;
  float inv_d = 0.f;
  float eps = 0.f;
  float* ss_out = nullptr;
};
template <class Epi>
hipError_t launch_skinny_bf16(const bf16_t* A, int lda, const bf16_t* B, int panel_rows, int M, int N, int K,
                              float* partial, int64_t partial_elems, const Epi& epi, hipStream_t stream,
                              SkinnyRowNorm rn = SkinnyRowNorm{});
int64_t skinny_partial_elems(int N, int K);

// Per-token metadata of a batch whose sequence b already holds ctx_b cached
// positions (ctx_lens NULL: all zero) and brings the tokens cu[b]..cu[b+1]:
// pos[t] = ctx_b + t - cu[b], slot[t] = its cache slot, and
// last_pos[b] = ctx_b + len_b - 1, last_row[b] = cu[b+1] - 1.
hipError_t launch_meta(const int32_t* cu_seqlens, const int32_t* ctx_lens, const int32_t* block_tables, int batch,
                       int max_blocks, int num_blocks, int total_tokens, int32_t* pos, int32_t* slot,
                       int32_t* last_pos, int32_t* last_row, hipStream_t stream);

// x[t, :] = E[tok[t], :] as fp32.
template <typename T>
hipError_t launch_embed(const int32_t* tok, const T* E, int vocab, int d, int T_, float* x, hipStream_t stream);

// y[r, :] = x[r, :] / sqrt(mean(x^2) + eps) * gamma  (gamma NULL -> 1), fp32 math.
// rows_idx (optional) gathers input rows: input row = rows_idx[r].
template <typename T>
hipError_t launch_rmsnorm(const float* x, const int32_t* rows_idx, const float* gamma, int rows, int d, float eps,
                          T* y, hipStream_t stream);

// Input of the next projection before its RMSNorm factor: y = bf16(x *
// gamma) in the panel layout (d columns, d % 32 == 0; gamma NULL = 1) and
// r[row] = 1 / sqrt(mean x^2 + eps).  split: y is the split-bf16 form of
// x * gamma with 2d columns, hi at column c and lo at column d + c.
hipError_t launch_rows_rms_panel(const float* x, const float* gamma, int rows, int d, float eps, bool split, bf16_t* y,
                                 float* r, hipStream_t stream);
// r[row] from the d/16 partial sums of squares per row that EpiResidual
// writes (summed in a fixed order); d % 16 == 0.
hipError_t launch_rms_from_partials(const float* ss, int rows, int d, float eps, float* r, hipStream_t stream);

// y[r, :] = x[rows_idx[r], :]  (fp32 rows)
hipError_t launch_gather_rows(const float* x, const int32_t* rows_idx, int rows, int d, float* y,
                              hipStream_t stream);
// The skinny products' input before its RMSNorm factor: act[r, :] =
// bf16(x[src, :] * gamma) (gamma NULL = 1) and ss[r, c] = sum of x[src,
// 128 c .. 128 c + 128]^2, with src = rows_idx[r] (rows_idx NULL: src = r);
// y (optional) receives a copy of the fp32 row.  d % 128 == 0.
hipError_t launch_rows_act_ss(const float* x, const int32_t* rows_idx, const float* gamma, int rows, int d, float* y,
                              bf16_t* act, float* ss, hipStream_t stream);

// Causal GQA flash attention for prompt tokens (bf16, MFMA): q [T, hq, dh],
// K/V from one cache slot, o [T, hq * dh] in the panel layout (panel_off with
// hq * dh columns).  Sequence b's tokens cu[b]..cu[b+1] sit at positions
// ctx_b.. (ctx_lens NULL: 0) and attend to every cached position up to their
// own.  max_new = the longest cu run.  head_dim 128, hq/hkv % 4 == 0.
hipError_t launch_attn_prefill_bf16(const bf16_t* q, CacheSlot<bf16_t> cache, const int32_t* cu_seqlens,
                                    const int32_t* ctx_lens, const int32_t* block_tables, int max_blocks, int batch,
                                    int max_new, int hq, bf16_t* o, hipStream_t stream);

// The same attention in split-bf16 form: q / q_lo, the cache slot's K/V and
// their low parts in `lo` (same geometry) are the two parts of each
// operand; o gets 2 hq * dh columns, the output's high parts at column c and
// low parts at hq * dh + c.
hipError_t launch_attn_prefill_split(const bf16_t* q, const bf16_t* q_lo, CacheSlot<bf16_t> cache,
                                     CacheSlot<bf16_t> lo, const int32_t* cu_seqlens, const int32_t* ctx_lens,
                                     const int32_t* block_tables, int max_blocks, int batch, int max_new, int hq,
                                     bf16_t* o, hipStream_t stream);

// The same attention with K/V from a per-token FP8 cache slot.
hipError_t launch_attn_prefill_fp8(const bf16_t* q, Fp8Slot cache, const int32_t* cu_seqlens, const int32_t* ctx_lens,
                                   const int32_t* block_tables, int max_blocks, int batch, int max_new, int hq,
                                   bf16_t* o, hipStream_t stream);

// Attention for a list of query rows, each attending to positions
// [0, ctx) of its prompt (ctx = pos + 1), split over key chunks with a
// combine pass.  Used for the last-token path and for fp32 prompt tokens.
// rows: number of query rows; q [rows, hq, dh]; row_seq[r] = prompt index;
// row_pos[r] = position (ctx = pos + 1).  Workspace: attn_ws_elems floats.
template <typename T>
hipError_t launch_attn_rows(const T* q, CacheSlot<T> cache, const int32_t* row_seq, const int32_t* row_pos,
                            const int32_t* block_tables, int max_blocks, int rows, int max_ctx, int hq, float* ws,
                            T* o, hipStream_t stream);
int64_t attn_rows_ws_elems(int rows, int max_ctx, int hq, int dh, bool bf16_rows);
// The same with K/V from a per-token FP8 cache slot (bf16 queries, dh 128).
hipError_t launch_attn_rows_fp8(const bf16_t* q, Fp8Slot cache, const int32_t* row_seq, const int32_t* row_pos,
                                const int32_t* block_tables, int max_blocks, int rows, int max_ctx, int hq, float* ws,
                                bf16_t* o, hipStream_t stream);

// For fp32 prompt-token attention: row_seq[t] for every token.
hipError_t launch_token_seq(const int32_t* cu_seqlens, int batch, int total_tokens, int32_t* seq,
                            hipStream_t stream);

// Per-token FP8 quantisation of T new tokens' K/V rows.  stage: bf16 rows in
// the cache layout with physical slot = token index (group g's K at
// stage + g * stage_group_stride, V at + stage_v_offset); ngroups
// destination slots dst0, dst0 + 1 slot, ... (codes dst_slot_stride bytes
// apart, scales dst_scale_stride floats apart); slot[t] = the token's
// physical slot (-1: skipped).  hkv * dh <= 1024, dh % 16 == 0.
hipError_t launch_kv_quant(const bf16_t* stage, int64_t stage_group_stride, int64_t stage_v_offset, int T,
                           int ngroups, const int32_t* slot, Fp8Slot dst0, int64_t dst_slot_stride,
                           int64_t dst_scale_stride, hipStream_t stream);

// Weight repacking at load time.
template <typename T>
hipError_t launch_fold_rows(const T* W, const T* gamma, int rows, int cols, T* out, hipStream_t stream);
template <typename T>
hipError_t launch_interleave(const T* gate, const T* up, int f, int d, int P, T* out, hipStream_t stream);
// Row-major W [rows, K] -> panel layout with panels of panel_rows rows
// (kPanelRows or kSkinnyPanelRows), rows rounded up to a whole panel
// (padding rows zero); K % 32 == 0.
hipError_t launch_to_panels(const bf16_t* W, int rows, int K, int panel_rows, bf16_t* out, hipStream_t stream);
template <typename T>
hipError_t launch_to_f32(const T* in, int64_t n, float* out, hipStream_t stream);

// Pure-MFMA throughput probe (calib.hip): `grid` workgroups of 4 waves, each
// wave issuing mfma_probe_per_iter() 16x16x32 bf16 MFMAs (of
// mfma_probe_flops_per_mfma() FLOPs) per iteration from the 16 x 64 bf16x8
// operands in `in`; clk[2g] / clk[2g+1] = shader-clock cycles / 100 MHz
// ticks of workgroup g's loop.  out: grid * 256 floats.
int mfma_probe_per_iter();
int mfma_probe_flops_per_mfma();
hipError_t launch_mfma_probe(const bf16x8_t* in, int iters, int grid, float* out, unsigned long long* clk,
                             hipStream_t stream);
