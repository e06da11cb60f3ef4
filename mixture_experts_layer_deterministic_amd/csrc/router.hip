// Router: fp32 logits in one fixed summation order, then a wavefront-level top-k with ties
// going to the lower expert index, then the softmax weights renormalised over the selected k.
//
// The toknow.ai summary says an MoE sends each input to a few experts; the pages define no
// gate beyond that. This router is the plain top-k softmax gate.
#include "common.h"
#include "kernels.h"

namespace moe {

// One thread per expert (256 experts per workgroup), TT tokens per workgroup. For every
// (token, expert) a single fp32 accumulator gains x[i] * w[i] for i = 0, 1, ..., d-1 in
// ascending order with one rounding per step. The bf16 x bf16 products are exact in fp32, so
// fma(x, w, acc) equals fl(acc + x * w). Tokens are staged in LDS as fp32 (read as lane-uniform
// broadcasts); router rows are staged as bf16 with 16 bytes of padding per row, so the 64 lanes'
// 16-byte reads of 64 different rows are bank-conflict free.
template <int TT, int CH>
__global__ void __launch_bounds__(256) router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ wr,
                                                            float* __restrict__ logits, int T,
                                                            int d, int E) {
  __shared__ float xs[TT][CH];
  __shared__ __align__(16) uint16_t ws[256][CH + 8];
  const int t0 = blockIdx.x * TT;
  const int e0 = blockIdx.y * 256;
  const int tid = threadIdx.x;
  float acc[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) acc[tt] = 0.f;

  for (int i0 = 0; i0 < d; i0 += CH) {
    for (int v = tid; v < TT * CH; v += 256) {
      const int tt = v / CH, ii = v % CH, t = t0 + tt;
      xs[tt][ii] = t < T ? bf2f(x[(size_t)t * d + i0 + ii]) : 0.f;
    }
    for (int v = tid; v < 256 * (CH / 8); v += 256) {
      const int row = v / (CH / 8), cv = v % (CH / 8), e = e0 + row;
      const uint4 val = e < E ? *reinterpret_cast<const uint4*>(wr + (size_t)e * d + i0 + cv * 8)
                              : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(&ws[row][cv * 8]) = val;
    }
    __syncthreads();
#pragma unroll 2
    for (int ii = 0; ii < CH; ii += 8) {
      const uint4 wv = *reinterpret_cast<const uint4*>(&ws[tid][ii]);
      const float w8[8] = {bf2f_lo(wv.x), bf2f_hi(wv.x), bf2f_lo(wv.y), bf2f_hi(wv.y),
                           bf2f_lo(wv.z), bf2f_hi(wv.z), bf2f_lo(wv.w), bf2f_hi(wv.w)};
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) acc[tt] = __builtin_fmaf(xs[tt][ii + q], w8[q], acc[tt]);
    }
    __syncthreads();
  }
  const int e = e0 + tid;
  if (e < E) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
      if (t0 + tt < T) logits[(size_t)(t0 + tt) * E + e] = acc[tt];
  }
}

// One wave per token. Lane l holds the logits of experts l, l+64, ... Each of the k rounds takes
// the lane-local best unselected expert, then a butterfly reduction over the wave. The order
// is: larger logit first, equal logits lower index first. Round j's winner is kept by lane j.
// The weights are w_j = exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0), with the sum taken in
// ascending j.
__global__ void __launch_bounds__(256) router_topk_kernel(const float* __restrict__ logits, int T,
                                                          int E, int k, int32_t* __restrict__ idx,
                                                          float* __restrict__ w) {
  constexpr int MAXQ = 1024 / kWave;
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;  // whole wave leaves together; no block barrier below
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

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* wr, float* logits, int T,
                                int d, int E, hipStream_t s) {
  constexpr int TT = 8, CH = 64;
  dim3 grid((T + TT - 1) / TT, (E + 255) / 256);
  {
    TraceScope trace("router_logits", s);
    hipLaunchKernelGGL((router_logits_kernel<TT, CH>), grid, dim3(256), 0, s, x, wr, logits, T, d,
                       E);
  }
  return hipGetLastError();
}

hipError_t launch_router_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                              hipStream_t s) {
  {
    TraceScope trace("router_topk", s);
    hipLaunchKernelGGL(router_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, idx,
                       w);
  }
  return hipGetLastError();
}

}  // namespace moe
