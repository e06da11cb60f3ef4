// Gather-form combine: y[t] = bf16(sum_j w[t,j] O[pos(t, j)]), j ascending, one thread per
// 16-byte output slice, no atomics. elementwise.hip launches it as a kernel; the single-launch
// forward (fused.hip) runs the same code inside its persistent kernel.
//
// The combine is the local half of the pages' forward combine (MarkTechPost, "Three design
// decisions that matter").
#pragma once

#include "common.h"

namespace moe {

// Rows of a token are gathered in groups of kGather: all loads of a group are issued before its
// first FMA, so each thread keeps up to kGather 16-byte loads in flight. Sums still run in
// ascending j.
constexpr int kGather = 8;

// Token of slice i (vpr slices per row). WAVE_TOKEN: vpr is a multiple of the wave size, so
// the 64 slices of a wave belong to one token; saying so lets the token's row indices, weights
// and expert ids arrive through scalar loads, once per wave instead of once per lane.
template <bool WAVE_TOKEN>
MOE_DEV int slice_token(int i, int vpr) {
  return WAVE_TOKEN ? __builtin_amdgcn_readfirstlane(i / vpr) : i / vpr;
}

// y[t] = bf16( sum_{j=0..k-1} w[t,j] * O[tk_row[t*k+j]] ), fp32 fma with j ascending.
// One thread per 16-byte slice (t, v) of y, no loop: the token's row indices and weights are
// loaded first, then its gathered slices (kGather at a time), so every thread of the grid has
// its loads in flight at once.
// Slice i of y (i < T * d / 8).
template <bool WAVE_TOKEN>
MOE_DEV void combine_slice(int i, const uint16_t* __restrict__ O,
                           const int32_t* __restrict__ tk_row, const float* __restrict__ topk_w,
                           int k, int d, uint16_t* __restrict__ y) {
  const int vpr = d / 8;
  const int t = slice_token<WAVE_TOKEN>(i, vpr), v = i % vpr;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < k; j0 += kGather) {
    int pos[kGather];
    float w[kGather];
    uint4 o[kGather];
#pragma unroll
    for (int jj = 0; jj < kGather; ++jj) {
      const int j = j0 + jj;
      pos[jj] = j < k ? tk_row[(size_t)t * k + j] : -1;
      w[jj] = j < k ? topk_w[(size_t)t * k + j] : 0.f;
    }
#pragma unroll
    for (int jj = 0; jj < kGather; ++jj)
      o[jj] = pos[jj] >= 0 ? nt_load16(O + (size_t)pos[jj] * d + v * 8) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int jj = 0; jj < kGather; ++jj) {
      if (pos[jj] < 0) continue;
      const uint32_t ow[4] = {o[jj].x, o[jj].y, o[jj].z, o[jj].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = __builtin_fmaf(w[jj], bf2f_lo(ow[q]), acc[2 * q]);
        acc[2 * q + 1] = __builtin_fmaf(w[jj], bf2f_hi(ow[q]), acc[2 * q + 1]);
      }
    }
  }
  uint4 out;
  out.x = pack_bf2(acc[0], acc[1]);
  out.y = pack_bf2(acc[2], acc[3]);
  out.z = pack_bf2(acc[4], acc[5]);
  out.w = pack_bf2(acc[6], acc[7]);
  *reinterpret_cast<uint4*>(y + (size_t)t * d + v * 8) = out;
}

}  // namespace moe
