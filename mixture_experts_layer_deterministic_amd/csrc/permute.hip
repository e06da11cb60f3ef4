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

// Block b owns rows [256 b, 256 b + 256): per-expert counts of the block, and each row's rank
// among the block's earlier rows of the same expert (a direct count, so it is stable).
__global__ void __launch_bounds__(kPermRows) perm_hist_kernel(const int32_t* __restrict__ idx,
                                                              int Tk, int E,
                                                              int32_t* __restrict__ blk_cnt,
                                                              int32_t* __restrict__ rank,
                                                              int32_t* __restrict__ blk_flag) {
  __shared__ int sh_e[kPermRows];
  __shared__ int sh_cnt[1024];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int r = b * kPermRows + tid;
  for (int i = tid; i < E; i += kPermRows) sh_cnt[i] = 0;
  int e = -1;
  int bad = 0;
  if (r < Tk) {
    e = idx[r];
    if (e < 0 || e >= E) {
      bad = 1;
      e = -1;
    }
  }
  sh_e[tid] = e;
  __syncthreads();
  if (e >= 0) atomicAdd(&sh_cnt[e], 1);  // integer counts: the result is order independent
  int rk = 0;
  for (int j = 0; j < tid; ++j) rk += (sh_e[j] == e);
  const int any_bad = __syncthreads_or(bad);
  if (r < Tk) rank[r] = e >= 0 ? rk : -1;
  for (int i = tid; i < E; i += kPermRows) blk_cnt[(size_t)b * E + i] = sh_cnt[i];
  if (tid == 0) blk_flag[b] = any_bad;
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

// Block b owns tokens [tpb b, tpb b + tpb) and their rows r = t*k + j (tpb*k <= 256). It
// places every row, then copies each token slice ONCE from x and stores it to the token's k
// positions: Xp[pos(t*k+j)] = x[t]. With MX the stored image is the token's MXFP8 form: E4M3
// codes xp8 [T*k, d] and one scale per 32 along d in xps [T*k, d/32]. Four consecutive lanes
// own one 32-block (d is a multiple of 32, so blocks never straddle rows), and every lane runs
// the shuffles.
template <bool MX>
__global__ void __launch_bounds__(256) perm_place_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ rank,
    const int32_t* __restrict__ blk_base, int T, int E, int k, int32_t* __restrict__ row_src,
    int32_t* __restrict__ tk_row, const uint16_t* __restrict__ x, uint16_t* __restrict__ xp,
    uint8_t* __restrict__ xp8, uint8_t* __restrict__ xps, int d, int tpb) {
  __shared__ int sh_pos[256];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * tpb;
  const int Tk = T * k;
  const int nr = tpb * k;
  if (tid < nr) {
    const int r = t0 * k + tid;
    int pos = -1;
    if (r < Tk) {
      const int rk = rank[r];
      if (rk >= 0) {
        pos = blk_base[(size_t)(r / kPermRows) * E + idx[r]] + rk;
        row_src[pos] = r;
      }
      tk_row[r] = pos;
    }
    sh_pos[tid] = pos;
  }
  __syncthreads();
  const int vpr = d / 8;
  const int n = tpb * vpr;
  if constexpr (!MX) {
    // U token slices loaded together, then each stored to its k positions
    constexpr int U = 4;
    for (int i0 = 0; i0 < n; i0 += 256 * U) {
      uint4 val[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + 256 * u + tid;
        const int t = t0 + i / vpr;
        val[u] = i < n && t < T
                     ? *reinterpret_cast<const uint4*>(x + (size_t)t * d + (i % vpr) * 8)
                     : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + 256 * u + tid;
        const int tt = i / vpr, v = i % vpr;
        if (i >= n || t0 + tt >= T) continue;
        for (int j = 0; j < k; ++j) {
          const int pos = sh_pos[tt * k + j];
          if (pos >= 0) *reinterpret_cast<uint4*>(xp + (size_t)pos * d + v * 8) = val[u];
        }
      }
    }
    return;
  }
  for (int i0 = 0; i0 < n; i0 += 256) {
    const int i = i0 + tid;
    const int tt = i / vpr, v = i % vpr;
    const int t = t0 + tt;
    const bool live = i < n && t < T;
    const uint4 val =
        live ? *reinterpret_cast<const uint4*>(x + (size_t)t * d + v * 8) : make_uint4(0, 0, 0, 0);
    const uint32_t xw[4] = {val.x, val.y, val.z, val.w};
    float f[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f[2 * q] = bf2f_lo(xw[q]);
      f[2 * q + 1] = bf2f_hi(xw[q]);
    }
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(f[j]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    const uint32_t code = mx_scale_code(amax);
    const float inv = mx_inv_scale(code);
    uint2 o;
    o.x = e4m3x2(f[0] * inv, f[1] * inv) | (e4m3x2(f[2] * inv, f[3] * inv) << 16);
    o.y = e4m3x2(f[4] * inv, f[5] * inv) | (e4m3x2(f[6] * inv, f[7] * inv) << 16);
    if (!live) continue;
    for (int j = 0; j < k; ++j) {
      const int pos = sh_pos[tt * k + j];
      if (pos < 0) continue;
      *reinterpret_cast<uint2*>(xp8 + (size_t)pos * d + v * 8) = o;
      if ((v & 3) == 0) xps[(size_t)pos * (d / 32) + v / 4] = static_cast<uint8_t>(code);
    }
  }
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
                             hipStream_t s) {
  const int T = Tk / k;
  // about 1024 slices of 16 bytes per block, and at most 256 rows
  int tpb = 1024 / (d / 8);
  if (tpb < 1) tpb = 1;
  if (tpb > 256 / k) tpb = 256 / k;
  const int grid = (T + tpb - 1) / tpb;
  {
    TraceScope trace("perm_place", s);
    if (xp8)
      hipLaunchKernelGGL(perm_place_kernel<true>, dim3(grid), dim3(256), 0, s, idx, rank, blk_base,
                         T, E, k, row_src, tk_row, x, xp, xp8, xps, d, tpb);
    else
      hipLaunchKernelGGL(perm_place_kernel<false>, dim3(grid), dim3(256), 0, s, idx, rank,
                         blk_base, T, E, k, row_src, tk_row, x, xp, xp8, xps, d, tpb);
  }
  return hipGetLastError();
}

}  // namespace moe
