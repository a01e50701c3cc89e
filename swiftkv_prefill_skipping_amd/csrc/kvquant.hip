// Per-token FP8 quantisation of freshly computed K/V rows into the paged
// FP8 cache (fp8.h gives the format and the rounding).
//
// The GEMM epilogues write the new tokens' K/V (RoPE applied, bf16) into a
// staging area laid out like a cache slot whose "physical slot" is the token
// index t; one wave then takes one (token, group, K-or-V) row of hkv * dh
// values, finds max|x|, and writes 16 codes per lane plus the row's scale at
// the token's physical slot of the destination cache slot.
#include "fp8.h"
#include "kernels.h"

namespace {

constexpr int kQuantMaxRow = 64 * 16;  // hkv * dh handled by one wave, 16 values per lane

__global__ __launch_bounds__(256) void kv_quant_kernel(const bf16_t* __restrict__ stage, int64_t stage_group_stride,
                                                       int64_t stage_v_offset, int T, int ngroups, int hkv, int dh,
                                                       const int32_t* __restrict__ slot, Fp8Slot dst0,
                                                       int64_t dst_slot_stride, int64_t dst_scale_stride) {
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  const int row = hkv * dh;
  const int t = wave / (2 * ngroups);
  if (t >= T) return;
  const int rest = wave - t * 2 * ngroups;
  const int grp = rest >> 1, is_v = rest & 1;
  const int sl = slot[t];
  if (sl < 0) return;
  const int c0 = lane * 16;  // this lane's 16 values of the row (head c0 / dh, dims c0 % dh ..)
  const bool live = c0 < row;
  const int h = c0 / dh, d = c0 % dh;
  const bf16_t* src = stage + grp * stage_group_stride + (is_v ? stage_v_offset : 0);
  float x[16];
  float amax = 0.f;
  if (live) {
    const bf16_t* p = src + kv_index(t, h, d, hkv, dh);
    unpack16<bf16_t>(*reinterpret_cast<const u32x4_t*>(p), x);
    unpack16<bf16_t>(*reinterpret_cast<const u32x4_t*>(p + 8), x + 8);
#pragma unroll
    for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(x[e]));
  }
  amax = warp_max(amax);
  const float scale = amax / 448.0f;
  const float inv = scale > 0.f ? 1.0f / scale : 0.f;
  if (live) {
    u32x4_t w = {0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float y = fminf(fmaxf(x[e] * inv, -448.0f), 448.0f);
      w[e >> 2] |= f32_to_e4m3(y) << (8 * (e & 3));
    }
    uint8_t* dst = (is_v ? dst0.v : dst0.k) + grp * dst_slot_stride;
    *reinterpret_cast<u32x4_t*>(dst + kv_index(sl, h, d, hkv, dh)) = w;
  }
  if (lane == 0) (is_v ? dst0.vs : dst0.ks)[grp * dst_scale_stride + sl] = scale;
}

}  // namespace

hipError_t launch_kv_quant(const bf16_t* stage, int64_t stage_group_stride, int64_t stage_v_offset, int T,
                           int ngroups, const int32_t* slot, Fp8Slot dst0, int64_t dst_slot_stride,
                           int64_t dst_scale_stride, hipStream_t stream) {
  if (T <= 0 || ngroups <= 0) return hipSuccess;
  if (dst0.hkv * dst0.dh > kQuantMaxRow || dst0.dh % 16) return hipErrorInvalidValue;
  const int64_t waves = (int64_t)T * ngroups * 2;
  hipLaunchKernelGGL(kv_quant_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, stage,
                     stage_group_stride, stage_v_offset, T, ngroups, dst0.hkv, dst0.dh, slot, dst0, dst_slot_stride,
                     dst_scale_stride);
  return hipGetLastError();
}
