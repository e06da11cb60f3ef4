// Router device code: fp32 logits in one fixed summation order, then a wavefront-level top-k
// with ties going to the lower expert index, then the softmax weights renormalised over the
// selected k. router.hip launches them as kernels; the single-launch forward (fused.hip) runs
// the same code inside its persistent kernel.
//
// The toknow.ai summary says an MoE sends each input to a few experts; the pages define no
// gate beyond that. This router is the plain top-k softmax gate.
#pragma once

#include "common.h"

namespace moe {

// Logits: one lane per token and one expert per wave (RE = 1), so a wave covers 64 tokens x 1
// expert and a block of RW waves the same 64 tokens x RW experts. For every (token, expert) a
// single fp32 accumulator gains x[i] * w[i] for i = 0, 1, ..., d-1 in ascending order with one
// rounding per step. The bf16 x bf16 products are exact in fp32, so fma(x, w, acc) equals
// fl(acc + x * w). The router rows, widened to fp32 beforehand (exactly), are the same for the
// whole wave: they arrive through scalar loads straight into FMA operands. What sets the rate is
// how many waves hide those scalar loads' latency: with one expert per wave the grid holds
// T/64 x E waves (8 per SIMD at T = 2048, E = 256); 4 experts per wave gave 2 per SIMD and ran
// 1.5x slower, although each x value then fed 4 FMAs. The block's 64 token rows go through
// LDS, RSTEP hidden elements at a time (double-buffered, each row one whole 128-byte line per
// step, staged by the first four waves), so the RW waves share one read of them.
constexpr int RE = 1;       // experts per wave
constexpr int RW = 8;       // waves per block
constexpr int RSTEP = 64;   // hidden elements per step (staged in LDS)
constexpr int RHALF = 32;   // hidden elements per FMA pass (bounds the scalar registers)
constexpr int RLD = RSTEP + 8;  // LDS row pitch (144 bytes: a lane group's 16-byte reads miss
                                // each other's banks)

// The router weight widened to fp32 (exact), four values per call: i is a multiple of 4.
MOE_DEV void widen_router_item(const uint16_t* __restrict__ wr, float* __restrict__ w32,
                               long long i) {
  const uint2 v = *reinterpret_cast<const uint2*>(wr + i);
  *reinterpret_cast<float4*>(w32 + i) =
      make_float4(bf2f_lo(v.x), bf2f_hi(v.x), bf2f_lo(v.y), bf2f_hi(v.y));
}

// The logits of block (bx, by): tokens [64 bx, 64 bx + 64) x experts [RWN by, RWN by + RWN),
// with RWN waves (at least four, which stage the token rows) and xs the block's LDS stage pair
// (2 x 64 x RLD bf16).
template <int RWN>
MOE_DEV void router_logits_block(int bx, int by, const uint16_t* __restrict__ x,
                                 const float* __restrict__ w32, float* __restrict__ logits, int T,
                                 int d, int E, uint16_t* __restrict__ xs_base) {
  static_assert(RWN >= 4, "four waves stage the token rows");
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int e0 = (by * RWN + wave) * RE;
  // waves past E still load and meet every barrier; they only skip the FMAs and the store
  const int ecount = max(0, min(RE, E - e0));
  const int t0 = bx * kWave;
  // this thread's two 16-byte pieces of each step: token row tid / 4 (a clamped copy of the last
  // row past T), columns 16 (tid % 4) .. + 16
  const int lt = (threadIdx.x / 4) % kWave, lc = (threadIdx.x % 4) * 16;
  const bool stager = threadIdx.x < 256;  // four waves stage the tile
  const uint16_t* xr = x + (size_t)min(t0 + lt, T - 1) * d + lc;
  const float* w0 = w32 + (size_t)min(e0, E - 1) * d;
  float acc[RE];
#pragma unroll
  for (int q = 0; q < RE; ++q) acc[q] = 0.f;
  uint4 p0 = make_uint4(0, 0, 0, 0), p1 = p0;
  if (stager) {
    p0 = *reinterpret_cast<const uint4*>(xr);
    p1 = *reinterpret_cast<const uint4*>(xr + 8);
  }
  int buf = 0;
  for (int i0 = 0; i0 < d; i0 += RSTEP) {
    if (stager) {
      *reinterpret_cast<uint4*>(xs_base + buf * (kWave * RLD) + lt * RLD + lc) = p0;
      *reinterpret_cast<uint4*>(xs_base + buf * (kWave * RLD) + lt * RLD + lc + 8) = p1;
    }
    __syncthreads();
    if (stager && i0 + RSTEP < d) {
      p0 = *reinterpret_cast<const uint4*>(xr + i0 + RSTEP);
      p1 = *reinterpret_cast<const uint4*>(xr + i0 + RSTEP + 8);
    }
    const uint16_t* row = xs_base + buf * (kWave * RLD) + lane * RLD;
#pragma unroll
    for (int h = 0; h < RSTEP; h += RHALF) {
      float xv[RHALF];
#pragma unroll
      for (int v = 0; v < RHALF / 8; ++v) {
        const uint4 q4 = *reinterpret_cast<const uint4*>(row + h + 8 * v);
        const uint32_t xw[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          xv[8 * v + 2 * q] = bf2f_lo(xw[q]);
          xv[8 * v + 2 * q + 1] = bf2f_hi(xw[q]);
        }
      }
#pragma unroll
      for (int ee = 0; ee < RE; ++ee) {
        if (ee >= ecount) break;  // wave-uniform
        const float* wp = w0 + (size_t)ee * d + i0 + h;
#pragma unroll
        for (int q = 0; q < RHALF; ++q) acc[ee] = __builtin_fmaf(xv[q], wp[q], acc[ee]);
      }
    }
    buf ^= 1;
  }
  const int t = t0 + lane;
  if (t < T) {
#pragma unroll
    for (int ee = 0; ee < RE; ++ee)
      if (ee < ecount) logits[(size_t)t * E + e0 + ee] = acc[ee];
  }
}

// One wave per token. Lane l holds the logits of experts l, l+64, ... Each of the k rounds takes
// the lane-local best unselected expert, then a butterfly reduction over the wave. The order
// is: larger logit first, equal logits lower index first. Round j's winner is kept by lane j.
// The weights are w_j = exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0), with the sum taken in
// ascending j.
// Token t's top-k on the calling wave (every lane calls it; no block barrier inside).
MOE_DEV void router_topk_token(int t, const float* __restrict__ logits, int E, int k,
                               int32_t* __restrict__ idx, float* __restrict__ w) {
  constexpr int MAXQ = 1024 / kWave;
  const int lane = threadIdx.x % kWave;
  const float* row = logits + (size_t)t * E;
  float v[MAXQ];
#pragma unroll
  for (int q = 0; q < MAXQ; ++q) {
    const int e = lane + kWave * q;
    v[q] = e < E ? row[e] : -INFINITY;
  }
  uint32_t taken = 0;
  float my_v = -INFINITY;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < MAXQ; ++q) {
      const int e = lane + kWave * q;
      if (e < E && !((taken >> q) & 1u) && (v[q] > bv || (v[q] == bv && e < be))) {
        bv = v[q];
        be = e;
      }
    }
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oe = __shfl_xor(be, off);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be % kWave) == lane) taken |= 1u << (be / kWave);
    if (lane == j) {
      my_v = bv;
      my_e = be;
    }
  }
  const float l0 = __shfl(my_v, 0);
  const float z = lane < k ? expf(my_v - l0) : 0.f;
  float s = 0.f;
  for (int j = 0; j < k; ++j) s += __shfl(z, j);
  if (lane < k) {
    idx[(size_t)t * k + lane] = my_e;
    w[(size_t)t * k + lane] = z / s;
  }
}

}  // namespace moe
