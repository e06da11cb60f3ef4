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

// src [B][R][C] bf16 quantised along R (blocks of 32 rows per column) and written transposed:
// dst [B][C][R] fp8, sc [B][C][R/32]. One workgroup of 128 threads per 32 x 128 tile; thread c
// owns column c of the tile and writes its 32 codes contiguously.
__global__ void __launch_bounds__(128) quant_cols_t_kernel(const uint16_t* __restrict__ src,
                                                           uint8_t* __restrict__ dst,
                                                           uint8_t* __restrict__ sc, int R,
                                                           int C) {
  __shared__ uint16_t tile[32][128 + 2];
  const int b = blockIdx.z, r0 = blockIdx.y * 32, c0 = blockIdx.x * 128;
  const uint16_t* s = src + ((size_t)b * R + r0) * C + c0;
  for (int i = threadIdx.x; i < 32 * 16; i += 128) {  // 32 rows x 16 vectors of 8
    const int r = i / 16, cv = i % 16;
    const uint4 x = *reinterpret_cast<const uint4*>(s + (size_t)r * C + cv * 8);
    const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      tile[r][cv * 8 + 2 * q] = static_cast<uint16_t>(xw[q] & 0xffffu);
      tile[r][cv * 8 + 2 * q + 1] = static_cast<uint16_t>(xw[q] >> 16);
    }
  }
  __syncthreads();
  const int c = threadIdx.x;
  float f[32];
  float amax = 0.f;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    f[r] = bf2f(tile[r][c]);
    amax = fmaxf(amax, fabsf(f[r]));
  }
  const uint32_t code = mx_scale_code(amax);
  const float inv = mx_inv_scale(code);
  uint32_t w[8];
#pragma unroll
  for (int q = 0; q < 8; ++q)
    w[q] = e4m3x2(f[4 * q] * inv, f[4 * q + 1] * inv) |
           (e4m3x2(f[4 * q + 2] * inv, f[4 * q + 3] * inv) << 16);
  uint8_t* d = dst + ((size_t)b * C + c0 + c) * R + r0;
  reinterpret_cast<uint4*>(d)[0] = make_uint4(w[0], w[1], w[2], w[3]);
  reinterpret_cast<uint4*>(d)[1] = make_uint4(w[4], w[5], w[6], w[7]);
  sc[((size_t)b * C + c0 + c) * (R / 32) + r0 / 32] = static_cast<uint8_t>(code);
}

// dyw[pos] = bf16(w[row_src[pos]] * dy[row_src[pos] / k]): the down wgrad's left operand in
// position order. Thread v handles 8 elements of one position's row.
__global__ void __launch_bounds__(256) scale_gather_kernel(const uint16_t* __restrict__ dy,
                                                           const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ row_src,
                                                           const float* __restrict__ topk_w,
                                                           int E, int k, int d,
                                                           uint16_t* __restrict__ dyw,
                                                           long long nvec) {
  const long long v = (long long)blockIdx.x * 256 + threadIdx.x;
  if (v >= nvec) return;
  const int vpr = d / 8;
  const long long pos = v / vpr;
  if (pos >= offsets[E]) return;  // rows skipped for a bad expert index
  const int c = static_cast<int>(v % vpr) * 8;
  const int r = row_src[pos];
  const float w = topk_w[r];
  const uint4 x = *reinterpret_cast<const uint4*>(dy + (size_t)(r / k) * d + c);
  uint4 o;
  o.x = pack_bf2(bf2f_lo(x.x) * w, bf2f_hi(x.x) * w);
  o.y = pack_bf2(bf2f_lo(x.y) * w, bf2f_hi(x.y) * w);
  o.z = pack_bf2(bf2f_lo(x.z) * w, bf2f_hi(x.z) * w);
  o.w = pack_bf2(bf2f_lo(x.w) * w, bf2f_hi(x.w) * w);
  *reinterpret_cast<uint4*>(dyw + (size_t)pos * d + c) = o;
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

hipError_t launch_quant_cols_t(const uint16_t* src, int B, int R, int C, uint8_t* dst,
                               uint8_t* sc, const char* name, hipStream_t s) {
  {
    TraceScope trace(name, s);
    hipLaunchKernelGGL(quant_cols_t_kernel, dim3(C / 128, R / 32, B), dim3(128), 0, s, src, dst,
                       sc, R, C);
  }
  return hipGetLastError();
}

hipError_t launch_scale_gather(const uint16_t* dy, const int32_t* offsets, const int32_t* row_src,
                               const float* topk_w, int E, int k, int d, int Tk, uint16_t* dyw,
                               hipStream_t s) {
  const long long nvec = (long long)Tk * d / 8;
  {
    TraceScope trace("scale_gather", s);
    hipLaunchKernelGGL(scale_gather_kernel, dim3((unsigned)((nvec + 255) / 256)), dim3(256), 0, s,
                       dy, offsets, row_src, topk_w, E, k, d, dyw, nvec);
  }
  return hipGetLastError();
}

}  // namespace moe
