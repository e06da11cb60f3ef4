// Permutation device code: per-block expert histograms with stable in-block ranks, and the
// placement of every row plus the copy of its token into the ring slot. permute.hip launches
// them as kernels; the single-launch forward (fused.hip) runs the same code inside its
// persistent kernel.
//
// The ring token buffer of the MarkTechPost page ("Three design decisions that matter") has a
// fixed size, drops no tokens and keeps the CPU out of the loop.
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

// Block b owns rows [256 b, 256 b + 256): per-expert counts of the block, and each row's rank
// among the block's earlier rows of the same expert (a direct count, so it is stable). Run by
// kPermRows threads; sh_e [kPermRows] and sh_cnt [1024] are the block's LDS.
MOE_DEV void perm_hist_block(int b, const int32_t* __restrict__ idx, int Tk, int E,
                             int32_t* __restrict__ blk_cnt, int32_t* __restrict__ rank,
                             int32_t* __restrict__ blk_flag, int* sh_e, int* sh_cnt) {
  const int tid = threadIdx.x;
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

// Block b owns tokens [tpb b, tpb b + tpb) and their rows r = t*k + j (tpb*k <= 256). It
// places every row, then copies each token slice ONCE from x and stores it to the token's k
// positions: Xp[pos(t*k+j)] = x[t]. With MX (Q = 8 or 4) the stored image is the token's MX
// form: codes xp8 [T*k, d] (E4M3 bytes, Q = 8, or E2M1 nibbles two a byte, Q = 4) and one scale
// per 32 along d in xps [T*k, d/32]. Four consecutive lanes own one 32-block (d is a multiple
// of 32, so blocks never straddle rows), and every lane runs the shuffles.
// Run by 256 threads; sh_pos [256] is the block's LDS.
template <int Q>
MOE_DEV void perm_place_block(int blk, const int32_t* __restrict__ idx,
                              const int32_t* __restrict__ rank,
                              const int32_t* __restrict__ blk_base, int T, int E, int k,
                              int32_t* __restrict__ row_src, int32_t* __restrict__ tk_row,
                              const uint16_t* __restrict__ x, uint16_t* __restrict__ xp,
                              uint8_t* __restrict__ xp8, uint8_t* __restrict__ xps, int d, int tpb,
                              int* sh_pos) {
  const int tid = threadIdx.x;
  const int t0 = blk * tpb;
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
  if constexpr (Q == 0) {
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
    const uint32_t code = Q == 8 ? mx_scale_code(amax) : mx4_scale_code(amax);
    const float inv = mx_inv_scale(code);
    uint2 o;
    if constexpr (Q == 8) {
      o.x = e4m3x2(f[0] * inv, f[1] * inv) | (e4m3x2(f[2] * inv, f[3] * inv) << 16);
      o.y = e4m3x2(f[4] * inv, f[5] * inv) | (e4m3x2(f[6] * inv, f[7] * inv) << 16);
    } else {
      o.x = e2m1x4(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv) |
            (e2m1x4(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv) << 16);
    }
    if (!live) continue;
    for (int j = 0; j < k; ++j) {
      const int pos = sh_pos[tt * k + j];
      if (pos < 0) continue;
      if constexpr (Q == 8)
        *reinterpret_cast<uint2*>(xp8 + (size_t)pos * d + v * 8) = o;
      else
        *reinterpret_cast<uint32_t*>(xp8 + (size_t)pos * (d / 2) + v * 4) = o.x;
      if ((v & 3) == 0) xps[(size_t)pos * (d / 32) + v / 4] = static_cast<uint8_t>(code);
    }
  }
}

}  // namespace moe
