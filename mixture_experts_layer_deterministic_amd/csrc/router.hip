// Router kernels: fp32 logits in one fixed summation order, then a wavefront-level top-k with
// ties going to the lower expert index, then the softmax weights renormalised over the selected
// k. The device code is in router.h.
#include "common.h"
#include "kernels.h"
#include "router.h"

namespace moe {

__global__ void __launch_bounds__(256) widen_router_kernel(const uint16_t* __restrict__ wr,
                                                           float* __restrict__ w32, long long n) {
  const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  widen_router_item(wr, w32, i);
}

__global__ void __launch_bounds__(RW * 64) router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ w32,
                                                            float* __restrict__ logits, int T,
                                                            int d, int E) {
  __shared__ __align__(16) uint16_t xs[2 * kWave * RLD];
  router_logits_block<RW>(blockIdx.x, blockIdx.y, x, w32, logits, T, d, E, xs);
}

__global__ void __launch_bounds__(256) router_topk_kernel(const float* __restrict__ logits, int T,
                                                          int E, int k, int32_t* __restrict__ idx,
                                                          float* __restrict__ w) {
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;  // whole wave leaves together; no block barrier below
  router_topk_token(t, logits, E, k, idx, w);
}

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* wr, float* w32, float* logits,
                                int T, int d, int E, hipStream_t s) {
  const long long n = (long long)E * d;
  {
    TraceScope trace("widen_router", s);
    hipLaunchKernelGGL(widen_router_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, s,
                       wr, w32, n);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  dim3 grid((T + kWave - 1) / kWave, (E + RW * RE - 1) / (RW * RE));
  {
    TraceScope trace("router_logits", s);
    hipLaunchKernelGGL(router_logits_kernel, grid, dim3(RW * 64), 0, s, x, w32, logits, T, d, E);
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
