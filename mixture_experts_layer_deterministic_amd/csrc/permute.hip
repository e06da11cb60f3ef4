// Deterministic expert permutation into a ring slot: per-block histograms, an exclusive scan,
// then a stable placement of every row and the copy of its token into the slot.
//
// The ring token buffer of the MarkTechPost page ("Three design decisions that matter") has a
// fixed size, drops no tokens and keeps the CPU out of the loop. Here the slot holds T*k rows,
// the worst case, so no expert imbalance can overflow it. The counts stay on the device.
// Row r = t*k + j of expert e lands at offsets[e] + (rows r' < r of expert e), so segments
// ascend by r.
#include <mutex>

#include "common.h"
#include "kernels.h"
#include "permute.h"

namespace moe {

// Fixed scratch of the permutation for callers that cannot allocate (moe_permute_static): one
// copy per GPU, held until the process ends. Host code never passes this name to a kernel (on
// the host it is only a stand-in); it passes the device address that static_perm_scratch()
// fetched with hipGetSymbolAddress on that device.
static __device__ __align__(256) unsigned char scratch[kStaticPermScratchBytes];

hipError_t static_perm_scratch(void** ptr) {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static void* addr[kMaxDev] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

__global__ void __launch_bounds__(kPermRows) perm_hist_kernel(const int32_t* __restrict__ idx,
                                                              int Tk, int E,
                                                              int32_t* __restrict__ blk_cnt,
                                                              int32_t* __restrict__ rank,
                                                              int32_t* __restrict__ blk_flag) {
  __shared__ int sh_e[kPermRows];
  __shared__ int sh_cnt[1024];
  perm_hist_block(blockIdx.x, idx, Tk, E, blk_cnt, rank, blk_flag, sh_e, sh_cnt);
}

// One workgroup: column-wise exclusive scan of the block counts (block order), expert totals,
// an exclusive scan over experts, and the per-block base positions.
__global__ void __launch_bounds__(1024) perm_scan_kernel(int32_t* __restrict__ blk_cnt, int nb,
                                                         int E, const int32_t* __restrict__ blk_flag,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ status) {
  __shared__ int sc[1024];
  const int e = threadIdx.x;
  constexpr int U = 16;  // block counts loaded together before their running sum
  int total = 0;
  if (e < E) {
    for (int b0 = 0; b0 < nb; b0 += U) {
      int c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) c[u] = b0 + u < nb ? blk_cnt[(size_t)(b0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (b0 + u < nb) blk_cnt[(size_t)(b0 + u) * E + e] = total;
        total += c[u];
      }
    }
    counts[e] = total;
  }
  sc[e] = total;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = e >= off ? sc[e - off] : 0;
    __syncthreads();
    sc[e] += v;
    __syncthreads();
  }
  const int excl = sc[e] - total;
  if (e < E) {
    offsets[e] = excl;
    for (int b0 = 0; b0 < nb; b0 += U) {
      int c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) c[u] = b0 + u < nb ? blk_cnt[(size_t)(b0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (b0 + u < nb) blk_cnt[(size_t)(b0 + u) * E + e] = c[u] + excl;
    }
  }
  if (e == 1023) offsets[E] = sc[1023];
  int f = 0;
  for (int b = e; b < nb; b += 1024) f |= blk_flag[b];
  f = __syncthreads_or(f);
  if (e == 0) status[0] = f ? 1 : 0;
}

template <int Q>
__global__ void __launch_bounds__(256) perm_place_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ rank,
    const int32_t* __restrict__ blk_base, int T, int E, int k, int32_t* __restrict__ row_src,
    int32_t* __restrict__ tk_row, const uint16_t* __restrict__ x, uint16_t* __restrict__ xp,
    uint8_t* __restrict__ xp8, uint8_t* __restrict__ xps, int d, int tpb) {
  __shared__ int sh_pos[256];
  perm_place_block<Q>(blockIdx.x, idx, rank, blk_base, T, E, k, row_src, tk_row, x, xp, xp8,
                       xps, d, tpb, sh_pos);
}

hipError_t launch_perm_hist(const int32_t* idx, int Tk, int E, int32_t* blk_cnt, int32_t* rank,
                            int32_t* blk_flag, hipStream_t s) {
  const int nb = (Tk + kPermRows - 1) / kPermRows;
  {
    TraceScope trace("perm_hist", s);
    hipLaunchKernelGGL(perm_hist_kernel, dim3(nb), dim3(kPermRows), 0, s, idx, Tk, E, blk_cnt, rank,
                       blk_flag);
  }
  return hipGetLastError();
}

hipError_t launch_perm_scan(int32_t* blk_cnt, int nb, int E, const int32_t* blk_flag,
                            int32_t* counts, int32_t* offsets, int32_t* status, hipStream_t s) {
  {
    TraceScope trace("perm_scan", s);
    hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(1024), 0, s, blk_cnt, nb, E, blk_flag, counts,
                       offsets, status);
  }
  return hipGetLastError();
}

hipError_t launch_perm_place(const int32_t* idx, const int32_t* rank, const int32_t* blk_base,
                             int Tk, int E, int k, int32_t* row_src, int32_t* tk_row,
                             const uint16_t* x, uint16_t* xp, uint8_t* xp8, uint8_t* xps, int d,
                             int fbits, hipStream_t s) {
  const int T = Tk / k;
  // about 1024 slices of 16 bytes per block, and at most 256 rows
  int tpb = 1024 / (d / 8);
  if (tpb < 1) tpb = 1;
  if (tpb > 256 / k) tpb = 256 / k;
  const int grid = (T + tpb - 1) / tpb;
  {
    TraceScope trace("perm_place", s);
    if (xp8 && fbits == 4)
      hipLaunchKernelGGL(perm_place_kernel<4>, dim3(grid), dim3(256), 0, s, idx, rank, blk_base,
                         T, E, k, row_src, tk_row, x, xp, xp8, xps, d, tpb);
    else if (xp8)
      hipLaunchKernelGGL(perm_place_kernel<8>, dim3(grid), dim3(256), 0, s, idx, rank, blk_base,
                         T, E, k, row_src, tk_row, x, xp, xp8, xps, d, tpb);
    else
      hipLaunchKernelGGL(perm_place_kernel<0>, dim3(grid), dim3(256), 0, s, idx, rank,
                         blk_base, T, E, k, row_src, tk_row, x, xp, xp8, xps, d, tpb);
  }
  return hipGetLastError();
}

}  // namespace moe
