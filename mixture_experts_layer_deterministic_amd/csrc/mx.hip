// MXFP8 (OCP Microscaling) quantisation kernels for the layer's MXFP8 mode: E4M3 elements with
// one E8M0 scale per 32 consecutive elements along the reduction axis of the GEMM that reads them.
//
// The MarkTechPost page on Mixture-of-Kittens (MoK), closing paragraph of "Three design
// decisions that matter", names BF16 and MXFP8 precision modes. Scale code of a block:
// floor(log2 amax) - 8 + 127, clamped to 0..254 (0 for an all-zero block). Elements:
// round to nearest even of v / 2^(code - 127), saturated to +-448.
#include "common.h"
#include "kernels.h"

namespace moe {

// Rows of bf16 quantised along the row: thread v handles elements [8 v, 8 v + 8) of the
// flattened array; four consecutive threads (lanes 4q..4q+3 of a wave) make one 32-block.
// Requires the row length to be a multiple of 32.
__global__ void __launch_bounds__(256) quant_rows_kernel(const uint16_t* __restrict__ src,
                                                         uint8_t* __restrict__ dst,
                                                         uint8_t* __restrict__ sc,
                                                         long long nvec) {
  const long long v = (long long)blockIdx.x * 256 + threadIdx.x;
  const bool live = v < nvec;
  const uint4 x = live ? reinterpret_cast<const uint4*>(src)[v] : make_uint4(0, 0, 0, 0);
  const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
  float f[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f[2 * q] = bf2f_lo(xw[q]);
    f[2 * q + 1] = bf2f_hi(xw[q]);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const uint32_t code = mx_scale_code(amax);
  const float inv = mx_inv_scale(code);
  uint2 o;
  o.x = e4m3x2(f[0] * inv, f[1] * inv) | (e4m3x2(f[2] * inv, f[3] * inv) << 16);
  o.y = e4m3x2(f[4] * inv, f[5] * inv) | (e4m3x2(f[6] * inv, f[7] * inv) << 16);
  if (live) {
    reinterpret_cast<uint2*>(dst)[v] = o;
    if ((v & 3) == 0) sc[v >> 2] = static_cast<uint8_t>(code);
  }
}

// Both MXFP8 copies of a weight src [B][R][C] bf16 in one pass over it:
//  * along C (the forward GEMM's reduction axis): dq [B][R][C] codes, dqs [B][R][C/32] scales;
//  * along R, transposed (the dgrad's reduction axis): tq [B][C][R] codes, tqs [B][C][R/32].
// One workgroup of 256 threads per 128 x 128 tile (R and C are multiples of 128). The tile is
// read once: each row's 32-blocks are quantised from registers as they arrive, and the tile goes
// to LDS, where wave w quantises rows [32 w, 32 w + 32) of every column. The column codes are
// then staged in the same LDS (about 33 KB per workgroup in all, so four fit on a CU) and each
// column's 128 codes leave as 128 contiguous bytes. Scale codes leave four bytes at a time.
constexpr int kQT = 128;
__global__ void __launch_bounds__(256) quant_weight_kernel(const uint16_t* __restrict__ src,
                                                           uint8_t* __restrict__ dq,
                                                           uint8_t* __restrict__ dqs,
                                                           uint8_t* __restrict__ tq,
                                                           uint8_t* __restrict__ tqs, int R,
                                                           int C) {
  constexpr int TP = kQT / 2 + 1;  // tile pitch in words (bf16 pairs)
  constexpr int OP = kQT / 4 + 1;  // pitch of the staged column codes in words
  static_assert(kQT * OP <= kQT * TP, "column codes fit in the tile's LDS");
  __shared__ uint32_t tile[kQT * TP];
  __shared__ uint32_t scT[kQT];  // the column's four scale codes, one per byte
  // Tiles in diagonal order: workgroups adjacent in launch order differ in both tile row and
  // tile column, so those in flight at once neither write the transposed codes at one column
  // of rows R bytes apart nor the row codes at one column of rows C bytes apart.
  const int b = blockIdx.z, nx = gridDim.x, ny = gridDim.y;
  const int lin = blockIdx.y * nx + blockIdx.x;
  const int ty = lin % ny, tx = (lin / ny + ty) % nx;
  const int r0 = ty * kQT, c0 = tx * kQT;
  const int t = threadIdx.x;
  const uint16_t* s = src + ((size_t)b * R + r0) * C + c0;
  // Phase 1: sixteen lanes per row, eight elements per lane; lanes 4q..4q+3 make one 32-block.
  const int cv = t % 16;
  uint4 x[kQT / 16];
#pragma unroll
  for (int j = 0; j < kQT / 16; ++j)
    x[j] = *reinterpret_cast<const uint4*>(s + (size_t)(t / 16 + 16 * j) * C + cv * 8);
#pragma unroll
  for (int j = 0; j < kQT / 16; ++j) {
    const int r = t / 16 + 16 * j;
    tile[r * TP + cv * 4 + 0] = x[j].x;
    tile[r * TP + cv * 4 + 1] = x[j].y;
    tile[r * TP + cv * 4 + 2] = x[j].z;
    tile[r * TP + cv * 4 + 3] = x[j].w;
    const uint32_t xw[4] = {x[j].x, x[j].y, x[j].z, x[j].w};
    float f[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f[2 * q] = bf2f_lo(xw[q]);
      f[2 * q + 1] = bf2f_hi(xw[q]);
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    const uint32_t code = mx_scale_code(amax);
    const float inv = mx_inv_scale(code);
    uint2 o;
    o.x = e4m3x2(f[0] * inv, f[1] * inv) | (e4m3x2(f[2] * inv, f[3] * inv) << 16);
    o.y = e4m3x2(f[4] * inv, f[5] * inv) | (e4m3x2(f[6] * inv, f[7] * inv) << 16);
    const size_t row = (size_t)b * R + r0 + r;
    *reinterpret_cast<uint2*>(dq + row * C + c0 + cv * 8) = o;
    // the row's four block scales (lanes cv = 0, 4, 8, 12 of its group) as one word
    const int g0 = (t % kWave) & ~15;
    const uint32_t w4 = __shfl(code, g0) | (__shfl(code, g0 + 4) << 8) |
                        (__shfl(code, g0 + 8) << 16) | (__shfl(code, g0 + 12) << 24);
    if (cv == 0) *reinterpret_cast<uint32_t*>(dqs + row * (C / 32) + c0 / 32) = w4;
  }
  __syncthreads();
  // Phase 2: wave w takes rows [32 w, 32 w + 32); lane l the column pair (2 l, 2 l + 1).
  const int w = t / kWave, l = t % kWave;
  uint32_t clo[8], chi[8];
  {
    float lo[32], hi[32];
    float alo = 0.f, ahi = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t v = tile[(w * 32 + i) * TP + l];
      lo[i] = bf2f_lo(v);
      hi[i] = bf2f_hi(v);
      alo = fmaxf(alo, fabsf(lo[i]));
      ahi = fmaxf(ahi, fabsf(hi[i]));
    }
    const uint32_t slo = mx_scale_code(alo), shi = mx_scale_code(ahi);
    const float ilo = mx_inv_scale(slo), ihi = mx_inv_scale(shi);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      clo[q] = e4m3x2(lo[4 * q] * ilo, lo[4 * q + 1] * ilo) |
               (e4m3x2(lo[4 * q + 2] * ilo, lo[4 * q + 3] * ilo) << 16);
      chi[q] = e4m3x2(hi[4 * q] * ihi, hi[4 * q + 1] * ihi) |
               (e4m3x2(hi[4 * q + 2] * ihi, hi[4 * q + 3] * ihi) << 16);
    }
    reinterpret_cast<uint8_t*>(scT)[(2 * l) * 4 + w] = static_cast<uint8_t>(slo);
    reinterpret_cast<uint8_t*>(scT)[(2 * l + 1) * 4 + w] = static_cast<uint8_t>(shi);
  }
  __syncthreads();  // every wave has read the tile: its LDS now holds the column codes
  uint32_t* outT = tile;  // [kQT][OP]
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    outT[(2 * l) * OP + w * 8 + q] = clo[q];
    outT[(2 * l + 1) * OP + w * 8 + q] = chi[q];
  }
  __syncthreads();
  // Phase 3: each column's 128 codes as eight 16-byte stores, and its four scales as one word.
#pragma unroll
  for (int j = 0; j < kQT * 8 / 256; ++j) {
    const int idx = t + 256 * j, c = idx / 8, part = idx % 8;
    const uint4 v = make_uint4(outT[c * OP + part * 4], outT[c * OP + part * 4 + 1],
                               outT[c * OP + part * 4 + 2], outT[c * OP + part * 4 + 3]);
    *reinterpret_cast<uint4*>(tq + ((size_t)b * C + c0 + c) * R + r0 + part * 16) = v;
  }
  if (t < kQT)
    *reinterpret_cast<uint32_t*>(tqs + ((size_t)b * C + c0 + t) * (R / 32) + r0 / 32) = scT[t];
}

// dyw[pos] = bf16(w[r] * dy[r / k]) for every row r placed at pos = tk_row[r]: the down
// wgrad's left operand in position order. One thread per 16-byte slice (t, v) of dy: the slice
// is loaded once, together with the token's row positions and weights, and stored scaled to
// each of its k positions. Rows that were not placed (tk_row < 0) store nothing.
// WAVE_TOKEN: the 64 slices of a wave belong to one token (vpr a multiple of 64), so its row
// positions and weights arrive through scalar loads.
constexpr int kSgGroup = 8;
template <bool WAVE_TOKEN>
__global__ void __launch_bounds__(256) scale_gather_kernel(const uint16_t* __restrict__ dy,
                                                           const int32_t* __restrict__ tk_row,
                                                           const float* __restrict__ topk_w,
                                                           int T, int k, int d,
                                                           uint16_t* __restrict__ dyw) {
  const int vpr = d / 8;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= T * vpr) return;
  const int t = WAVE_TOKEN ? __builtin_amdgcn_readfirstlane(i / vpr) : i / vpr, v = i % vpr;
  const uint4 x = *reinterpret_cast<const uint4*>(dy + (size_t)t * d + v * 8);
  for (int j0 = 0; j0 < k; j0 += kSgGroup) {
    int pos[kSgGroup];
    float w[kSgGroup];
#pragma unroll
    for (int jj = 0; jj < kSgGroup; ++jj) {
      const int j = j0 + jj;
      pos[jj] = j < k ? tk_row[(size_t)t * k + j] : -1;
      w[jj] = j < k ? topk_w[(size_t)t * k + j] : 0.f;
    }
#pragma unroll
    for (int jj = 0; jj < kSgGroup; ++jj) {
      if (pos[jj] < 0) continue;
      const float wu = w[jj];
      uint4 o;
      o.x = pack_bf2(bf2f_lo(x.x) * wu, bf2f_hi(x.x) * wu);
      o.y = pack_bf2(bf2f_lo(x.y) * wu, bf2f_hi(x.y) * wu);
      o.z = pack_bf2(bf2f_lo(x.z) * wu, bf2f_hi(x.z) * wu);
      o.w = pack_bf2(bf2f_lo(x.w) * wu, bf2f_hi(x.w) * wu);
      *reinterpret_cast<uint4*>(dyw + (size_t)pos[jj] * d + v * 8) = o;
    }
  }
}

hipError_t launch_quant_rows(const uint16_t* src, long long rows, int cols, uint8_t* dst,
                             uint8_t* sc, const char* name, hipStream_t s) {
  const long long nvec = rows * cols / 8;
  if (nvec == 0) return hipSuccess;
  {
    TraceScope trace(name, s);
    hipLaunchKernelGGL(quant_rows_kernel, dim3((unsigned)((nvec + 255) / 256)), dim3(256), 0, s,
                       src, dst, sc, nvec);
  }
  return hipGetLastError();
}

hipError_t launch_quant_weight(const uint16_t* src, int B, int R, int C, uint8_t* dq,
                               uint8_t* dqs, uint8_t* tq, uint8_t* tqs, const char* name,
                               hipStream_t s) {
  if (R % kQT != 0 || C % kQT != 0) return hipErrorInvalidValue;
  if (B == 0) return hipSuccess;
  {
    TraceScope trace(name, s);
    hipLaunchKernelGGL(quant_weight_kernel, dim3(C / kQT, R / kQT, B), dim3(256), 0, s, src, dq,
                       dqs, tq, tqs, R, C);
  }
  return hipGetLastError();
}

hipError_t launch_scale_gather(const uint16_t* dy, const int32_t* tk_row, const float* topk_w,
                               int T, int k, int d, uint16_t* dyw, hipStream_t s) {
  const long long nvec = (long long)T * d / 8;
  if (nvec == 0) return hipSuccess;
  {
    TraceScope trace("scale_gather", s);
    const dim3 grid((unsigned)((nvec + 255) / 256));
    if ((d / 8) % 64 == 0)
      hipLaunchKernelGGL(scale_gather_kernel<true>, grid, dim3(256), 0, s, dy, tk_row, topk_w, T,
                         k, d, dyw);
    else
      hipLaunchKernelGGL(scale_gather_kernel<false>, grid, dim3(256), 0, s, dy, tk_row, topk_w, T,
                         k, d, dyw);
  }
  return hipGetLastError();
}

}  // namespace moe
