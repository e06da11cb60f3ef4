// Gather-form combine and its backward companions. Every output is written by exactly one
// thread, which sums in a fixed order: atomic-free and bitwise reproducible.
//
// The combine is the local half of the pages' forward combine; the backward un-permute is the
// local half of their reverse dispatch (MarkTechPost, "Three design decisions that matter").
#include "combine.h"
#include "common.h"
#include "kernels.h"

namespace moe {

template <bool WAVE_TOKEN>
__global__ void __launch_bounds__(256) combine_kernel(const uint16_t* __restrict__ O,
                                                      const int32_t* __restrict__ tk_row,
                                                      const float* __restrict__ topk_w, int T,
                                                      int k, int d, uint16_t* __restrict__ y) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= T * (d / 8)) return;
  combine_slice<WAVE_TOKEN>(i, O, tk_row, topk_w, k, d, y);
}

// One wave per token, lane j for its row j (k <= 64): dw_j is the sum of that row's per-tile
// partials from the down-dgrad epilogue, in ascending tile order -> d_topk_w; and, when the
// layer routed itself, the top-k softmax backward dl_j = w_j (dw_j - sum_i w_i dw_i) stored per
// position, the sum taken in ascending i by every lane alike.
__global__ void __launch_bounds__(256) dw_router_kernel(const float* __restrict__ dwpart, int nIt,
                                                        const int32_t* __restrict__ tk_row,
                                                        const float* __restrict__ topk_w, int T,
                                                        int k, float* __restrict__ d_topk_w,
                                                        float* __restrict__ dl_pos, int routed) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
  if (t >= T) return;  // whole wave
  const bool live = lane < k;
  const size_t r = (size_t)t * k + lane;
  const int pos = live ? tk_row[r] : -1;
  const float w = live ? topk_w[r] : 0.f;
  float dw = 0.f;
  if (pos >= 0)
    for (int it = 0; it < nIt; ++it) dw += dwpart[(size_t)pos * nIt + it];
  if (live) d_topk_w[r] = dw;
  if (!routed) return;
  float s = 0.f;
  for (int j = 0; j < k; ++j) s = __builtin_fmaf(__shfl(w, j), __shfl(dw, j), s);
  if (pos >= 0) dl_pos[pos] = w * (dw - s);
}

// dx[t] = bf16( sum_j dXp[tk_row[t*k+j]] + sum_j dl_j * Wr[e_j] ), j ascending, fp32; the
// router term only when wr is given. One thread per 16-byte slice (t, v) of dx, no loop.
// ONE_GROUP (k <= kGather): the row indices and expert indices are loaded first, then every dXp
// row, router row and dl together, so a token costs two round trips to memory; the sums keep
// the order above.
template <bool ONE_GROUP, bool WAVE_TOKEN>
__global__ void __launch_bounds__(256) uncombine_kernel(
    const uint16_t* __restrict__ dXp, const int32_t* __restrict__ tk_row,
    const int32_t* __restrict__ topk_idx, const float* __restrict__ dl_pos,
    const uint16_t* __restrict__ wr, int T, int k, int d, uint16_t* __restrict__ dx) {
  const int vpr = d / 8;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= T * vpr) return;
  const int t = slice_token<WAVE_TOKEN>(i, vpr), v = i % vpr;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if constexpr (ONE_GROUP) {
    int pos[kGather], e[kGather];
#pragma unroll
    for (int j = 0; j < kGather; ++j) {
      pos[j] = j < k ? tk_row[(size_t)t * k + j] : -1;
      e[j] = wr && j < k ? topk_idx[(size_t)t * k + j] : 0;
    }
    uint4 g[kGather], h[kGather];
    float dl[kGather];
#pragma unroll
    for (int j = 0; j < kGather; ++j) {
      const bool live = pos[j] >= 0;
      g[j] = live ? nt_load16(dXp + (size_t)pos[j] * d + v * 8) : make_uint4(0, 0, 0, 0);
      h[j] = wr && live ? *reinterpret_cast<const uint4*>(wr + (size_t)e[j] * d + v * 8)
                        : make_uint4(0, 0, 0, 0);
      dl[j] = wr && live ? dl_pos[pos[j]] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kGather; ++j) {
      if (pos[j] < 0) continue;
      const uint32_t gw[4] = {g[j].x, g[j].y, g[j].z, g[j].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += bf2f_lo(gw[q]);
        acc[2 * q + 1] += bf2f_hi(gw[q]);
      }
    }
    if (wr) {
#pragma unroll
      for (int j = 0; j < kGather; ++j) {
        if (pos[j] < 0) continue;
        const uint32_t hw[4] = {h[j].x, h[j].y, h[j].z, h[j].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = __builtin_fmaf(dl[j], bf2f_lo(hw[q]), acc[2 * q]);
          acc[2 * q + 1] = __builtin_fmaf(dl[j], bf2f_hi(hw[q]), acc[2 * q + 1]);
        }
      }
    }
    uint4 out;
    out.x = pack_bf2(acc[0], acc[1]);
    out.y = pack_bf2(acc[2], acc[3]);
    out.z = pack_bf2(acc[4], acc[5]);
    out.w = pack_bf2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(dx + (size_t)t * d + v * 8) = out;
    return;
  }
  for (int j0 = 0; j0 < k; j0 += kGather) {
    int pos[kGather];
    uint4 g[kGather];
#pragma unroll
    for (int jj = 0; jj < kGather; ++jj) {
      const int j = j0 + jj;
      pos[jj] = j < k ? tk_row[(size_t)t * k + j] : -1;
      g[jj] = pos[jj] >= 0 ? nt_load16(dXp + (size_t)pos[jj] * d + v * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int jj = 0; jj < kGather; ++jj) {
      if (pos[jj] < 0) continue;
      const uint32_t gw[4] = {g[jj].x, g[jj].y, g[jj].z, g[jj].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += bf2f_lo(gw[q]);
        acc[2 * q + 1] += bf2f_hi(gw[q]);
      }
    }
  }
  if (wr) {
    for (int j0 = 0; j0 < k; j0 += kGather) {
      int pos[kGather];
      uint4 g[kGather];
#pragma unroll
      for (int jj = 0; jj < kGather; ++jj) {
        const int j = j0 + jj;
        pos[jj] = j < k ? tk_row[(size_t)t * k + j] : -1;
        const int e = pos[jj] >= 0 ? topk_idx[(size_t)t * k + j] : 0;
        g[jj] = pos[jj] >= 0 ? *reinterpret_cast<const uint4*>(wr + (size_t)e * d + v * 8)
                             : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int jj = 0; jj < kGather; ++jj) {
        if (pos[jj] < 0) continue;
        const float dl = dl_pos[pos[jj]];
        const uint32_t gw[4] = {g[jj].x, g[jj].y, g[jj].z, g[jj].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = __builtin_fmaf(dl, bf2f_lo(gw[q]), acc[2 * q]);
          acc[2 * q + 1] = __builtin_fmaf(dl, bf2f_hi(gw[q]), acc[2 * q + 1]);
        }
      }
    }
  }
  uint4 out;
  out.x = pack_bf2(acc[0], acc[1]);
  out.y = pack_bf2(acc[2], acc[3]);
  out.z = pack_bf2(acc[4], acc[5]);
  out.w = pack_bf2(acc[6], acc[7]);
  *reinterpret_cast<uint4*>(dx + (size_t)t * d + v * 8) = out;
}

// dWr[e, c] = sum over positions p of expert e of dl_pos[p] * Xp[p, c] (fp32). Block (cx, e)
// covers columns [512 cx, 512 cx + 512); each lane owns 8 columns. The expert's positions are
// split into four contiguous quarters, one per wave, each summed in ascending p; the quarters
// are then added in order ((q0 + q1) + q2) + q3, so the result is the same on every run. F = 8
// reads Xp as its MXFP8 image (E4M3 codes xp8, one scale per 32 columns in xps), F = 4 as its
// MXFP4 image (E2M1 codes, two a byte), F = 0 as bf16 rows xp.
template <int F>
__global__ void __launch_bounds__(256) dwr_kernel(const float* __restrict__ dl_pos,
                                                  const uint16_t* __restrict__ xp,
                                                  const uint8_t* __restrict__ xp8,
                                                  const uint8_t* __restrict__ xps,
                                                  const int32_t* __restrict__ offsets, int d,
                                                  float* __restrict__ dwr, int accumulate) {
  __shared__ float part[3][8][64];
  const int e = blockIdx.y;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int c0 = (blockIdx.x * 64 + lane) * 8;
  const bool col = c0 < d;
  const int p0 = offsets[e], p1 = offsets[e + 1];
  const int quarter = (p1 - p0 + 3) / 4;
  const int q0 = min(p1, p0 + wave * quarter), q1 = min(p1, q0 + quarter);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // positions in groups of U: the group's loads are issued before its FMAs (p ascending)
  constexpr int U = 8;
  for (int pg = q0; pg < q1; pg += U) {
    float dl[U];
    uint4 raw[U];
    uint32_t sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = pg + u;
      const bool live = col && p < q1;
      dl[u] = live ? dl_pos[p] : 0.f;
      if constexpr (F == 8) {
        typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
        const u32x2 q2 = live ? __builtin_nontemporal_load(
                                    reinterpret_cast<const u32x2*>(xp8 + (size_t)p * d + c0))
                              : u32x2{0u, 0u};
        const uint2 q = make_uint2(q2[0], q2[1]);
        raw[u] = make_uint4(q.x, q.y, 0, 0);
        sc[u] = live ? xps[(size_t)p * (d / 32) + c0 / 32] : 0u;
      } else if constexpr (F == 4) {
        const uint32_t q = live ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(
                                      xp8 + (size_t)p * (d / 2) + c0 / 2))
                                : 0u;
        raw[u] = make_uint4(q, 0, 0, 0);
        sc[u] = live ? xps[(size_t)p * (d / 32) + c0 / 32] : 0u;
      } else {
        raw[u] = live ? nt_load16(xp + (size_t)p * d + c0) : make_uint4(0, 0, 0, 0);
        sc[u] = 0u;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (pg + u >= q1) break;
      float xv[8];
      if constexpr (F == 8) {
        const float s = mx_scale(sc[u]);
        float f[4], g[4];
        e4m3x4_to_f32(raw[u].x, f);
        e4m3x4_to_f32(raw[u].y, g);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          xv[q4] = f[q4] * s;
          xv[4 + q4] = g[q4] * s;
        }
      } else if constexpr (F == 4) {
        const float s = mx_scale(sc[u]);
        const float2 f0 = e2m1x2_to_f32<0>(raw[u].x), f1 = e2m1x2_to_f32<1>(raw[u].x),
                     f2 = e2m1x2_to_f32<2>(raw[u].x), f3 = e2m1x2_to_f32<3>(raw[u].x);
        xv[0] = f0.x * s, xv[1] = f0.y * s, xv[2] = f1.x * s, xv[3] = f1.y * s;
        xv[4] = f2.x * s, xv[5] = f2.y * s, xv[6] = f3.x * s, xv[7] = f3.y * s;
      } else {
        const uint32_t gw[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          xv[2 * q] = bf2f_lo(gw[q]);
          xv[2 * q + 1] = bf2f_hi(gw[q]);
        }
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(dl[u], xv[q], acc[q]);
    }
  }
  if (wave > 0)
#pragma unroll
    for (int q = 0; q < 8; ++q) part[wave - 1][q][lane] = acc[q];
  __syncthreads();
  if (wave > 0 || !col) return;
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] += part[w][q][lane];
  float4* dst = reinterpret_cast<float4*>(dwr + (size_t)e * d + c0);
  float4 a = make_float4(acc[0], acc[1], acc[2], acc[3]);
  float4 b = make_float4(acc[4], acc[5], acc[6], acc[7]);
  if (accumulate) {
    const float4 oa = dst[0], ob = dst[1];
    a.x += oa.x; a.y += oa.y; a.z += oa.z; a.w += oa.w;
    b.x += ob.x; b.y += ob.y; b.z += ob.z; b.w += ob.w;
  }
  dst[0] = a;
  dst[1] = b;
}

hipError_t launch_combine(const uint16_t* O, const int32_t* tk_row, const float* topk_w, int T,
                          int k, int d, uint16_t* y, hipStream_t s) {
  const int grid = (T * (d / 8) + 255) / 256;
  {
    TraceScope trace("combine", s);
    if ((d / 8) % kWave == 0)
      hipLaunchKernelGGL(combine_kernel<true>, dim3(grid), dim3(256), 0, s, O, tk_row, topk_w, T,
                         k, d, y);
    else
      hipLaunchKernelGGL(combine_kernel<false>, dim3(grid), dim3(256), 0, s, O, tk_row, topk_w, T,
                         k, d, y);
  }
  return hipGetLastError();
}

hipError_t launch_dw_router(const float* dwpart, int nIt, const int32_t* tk_row,
                            const float* topk_w, int T, int k, float* d_topk_w, float* dl_pos,
                            int routed, hipStream_t s) {
  {
    TraceScope trace("dw_router", s);
    const int tokens_per_block = 256 / kWave;
    hipLaunchKernelGGL(dw_router_kernel, dim3((T + tokens_per_block - 1) / tokens_per_block),
                       dim3(256), 0, s, dwpart, nIt, tk_row, topk_w, T, k, d_topk_w, dl_pos,
                       routed);
  }
  return hipGetLastError();
}

hipError_t launch_uncombine(const uint16_t* dXp, const int32_t* tk_row, const int32_t* topk_idx,
                            const float* dl_pos, const uint16_t* wr, int T, int k, int d,
                            uint16_t* dx, hipStream_t s) {
  {
    TraceScope trace("uncombine", s);
    const dim3 grid((T * (d / 8) + 255) / 256);
    const bool wt = (d / 8) % kWave == 0;
    if (k <= kGather && wt)
      hipLaunchKernelGGL((uncombine_kernel<true, true>), grid, dim3(256), 0, s, dXp, tk_row,
                         topk_idx, dl_pos, wr, T, k, d, dx);
    else if (k <= kGather)
      hipLaunchKernelGGL((uncombine_kernel<true, false>), grid, dim3(256), 0, s, dXp, tk_row,
                         topk_idx, dl_pos, wr, T, k, d, dx);
    else if (wt)
      hipLaunchKernelGGL((uncombine_kernel<false, true>), grid, dim3(256), 0, s, dXp, tk_row,
                         topk_idx, dl_pos, wr, T, k, d, dx);
    else
      hipLaunchKernelGGL((uncombine_kernel<false, false>), grid, dim3(256), 0, s, dXp, tk_row,
                         topk_idx, dl_pos, wr, T, k, d, dx);
  }
  return hipGetLastError();
}

hipError_t launch_dwr(const float* dl_pos, const uint16_t* xp, const uint8_t* xp8,
                      const uint8_t* xps, int fbits, const int32_t* offsets, int E, int d,
                      float* dwr, int accumulate, hipStream_t s) {
  {
    TraceScope trace("dwr", s);
    const dim3 grid((d + 511) / 512, E);
    if (xp8 && fbits == 4)
      hipLaunchKernelGGL(dwr_kernel<4>, grid, dim3(256), 0, s, dl_pos, xp, xp8, xps, offsets, d,
                         dwr, accumulate);
    else if (xp8)
      hipLaunchKernelGGL(dwr_kernel<8>, grid, dim3(256), 0, s, dl_pos, xp, xp8, xps, offsets, d,
                         dwr, accumulate);
    else
      hipLaunchKernelGGL(dwr_kernel<0>, grid, dim3(256), 0, s, dl_pos, xp, xp8, xps, offsets, d,
                         dwr, accumulate);
  }
  return hipGetLastError();
}

}  // namespace moe
