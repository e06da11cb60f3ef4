// MX (OCP Microscaling) quantisation kernels for the layer's MXFP8 and MXFP4 modes: E4M3 (F = 8)
// or E2M1 (F = 4, two codes a byte) elements with one E8M0 scale per 32 consecutive elements
// along the reduction axis of the GEMM that reads them.
//
// The MarkTechPost page on Mixture-of-Kittens (MoK), closing paragraph of "Three design
// decisions that matter", names BF16 and MXFP8 precision modes, and its section "MoE layer as the
// bottleneck" names 4-bit (NVFP4) training kernels. Scale code of a block: floor(log2 amax) -
// emax + 127 with emax 8 (E4M3) or 2 (E2M1), clamped to 0..254 (0 for an all-zero block).
// Elements: round to nearest even of v / 2^(code - 127), saturated to +-448 or +-6.
#include "common.h"
#include "kernels.h"

namespace moe {

// The scale code of a block with max magnitude amax, and the codes of eight scaled values: 8
// bytes (E4M3) or 4 bytes (E2M1) in element order.
template <int F>
MOE_DEV uint32_t mxf_scale_code(float amax) {
  return F == 8 ? mx_scale_code(amax) : mx4_scale_code(amax);
}
template <int F>
MOE_DEV uint2 mxf_encode8(const float (&f)[8], float inv) {
  if constexpr (F == 8) {
    return make_uint2(e4m3x2(f[0] * inv, f[1] * inv) | (e4m3x2(f[2] * inv, f[3] * inv) << 16),
                      e4m3x2(f[4] * inv, f[5] * inv) | (e4m3x2(f[6] * inv, f[7] * inv) << 16));
  } else {
    return make_uint2(e2m1x4(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv) |
                          (e2m1x4(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv) << 16),
                      0u);
  }
}
// Stores the codes of eight elements (element offset `e`, a multiple of 8) into a code array.
template <int F>
MOE_DEV void mxf_store8(uint8_t* base, size_t e, uint2 codes) {
  if constexpr (F == 8)
    *reinterpret_cast<uint2*>(base + e) = codes;
  else
    *reinterpret_cast<uint32_t*>(base + e / 2) = codes.x;
}

// Rows of bf16 quantised along the row: thread v handles elements [8 v, 8 v + 8) of the
// flattened array; four consecutive threads (lanes 4q..4q+3 of a wave) make one 32-block.
// Requires the row length to be a multiple of 32.
template <int F>
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
  const uint32_t code = mxf_scale_code<F>(amax);
  const uint2 o = mxf_encode8<F>(f, mx_inv_scale(code));
  if (live) {
    mxf_store8<F>(dst, (size_t)v * 8, o);
    if ((v & 3) == 0) sc[v >> 2] = static_cast<uint8_t>(code);
  }
}

// Both MX copies of a weight src [B][R][C] bf16 in one pass over it:
//  * along C (the forward GEMM's reduction axis): dq [B][R][C] codes, dqs [B][R][C/32] scales;
//  * along R, transposed (the dgrad's reduction axis): tq [B][C][R] codes, tqs [B][C][R/32].
// One workgroup of 256 threads per 128 x 128 tile (R and C are multiples of 128). The tile is
// read once: each row's 32-blocks are quantised from registers as they arrive, and the tile goes
// to LDS, where wave w quantises rows [32 w, 32 w + 32) of every column. The column codes are
// then staged in the same LDS (about 33 KB per workgroup in all, so four fit on a CU) and each
// column's 128 codes leave as 128 (E2M1: 64) contiguous bytes. Scale codes leave four bytes at
// a time.
constexpr int kQT = 128;
template <int F>
__global__ void __launch_bounds__(256) quant_weight_kernel(const uint16_t* __restrict__ src,
                                                           uint8_t* __restrict__ dq,
                                                           uint8_t* __restrict__ dqs,
                                                           uint8_t* __restrict__ tq,
                                                           uint8_t* __restrict__ tqs, int R,
                                                           int C) {
  constexpr int TP = kQT / 2 + 1;        // tile pitch in words (bf16 pairs)
  constexpr int WPC = kQT * F / 32;      // code words of one column's 128 elements
  constexpr int WPB = 32 * F / 32;       // code words of one column's 32-row block
  constexpr int OP = WPC + 1;            // pitch of the staged column codes in words
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
    const uint32_t code = mxf_scale_code<F>(amax);
    const uint2 o = mxf_encode8<F>(f, mx_inv_scale(code));
    const size_t row = (size_t)b * R + r0 + r;
    mxf_store8<F>(dq, row * C + c0 + cv * 8, o);
    // the row's four block scales (lanes cv = 0, 4, 8, 12 of its group) as one word
    const int g0 = (t % kWave) & ~15;
    const uint32_t w4 = __shfl(code, g0) | (__shfl(code, g0 + 4) << 8) |
                        (__shfl(code, g0 + 8) << 16) | (__shfl(code, g0 + 12) << 24);
    if (cv == 0) *reinterpret_cast<uint32_t*>(dqs + row * (C / 32) + c0 / 32) = w4;
  }
  __syncthreads();
  // Phase 2: wave w takes rows [32 w, 32 w + 32); lane l the column pair (2 l, 2 l + 1).
  const int w = t / kWave, l = t % kWave;
  uint32_t clo[WPB], chi[WPB];
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
    const uint32_t slo = mxf_scale_code<F>(alo), shi = mxf_scale_code<F>(ahi);
    const float ilo = mx_inv_scale(slo), ihi = mx_inv_scale(shi);
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // 8 rows each
      const float vl[8] = {lo[8 * q], lo[8 * q + 1], lo[8 * q + 2], lo[8 * q + 3],
                           lo[8 * q + 4], lo[8 * q + 5], lo[8 * q + 6], lo[8 * q + 7]};
      const float vh[8] = {hi[8 * q], hi[8 * q + 1], hi[8 * q + 2], hi[8 * q + 3],
                           hi[8 * q + 4], hi[8 * q + 5], hi[8 * q + 6], hi[8 * q + 7]};
      const uint2 cl = mxf_encode8<F>(vl, ilo), ch = mxf_encode8<F>(vh, ihi);
      if constexpr (F == 8) {
        clo[2 * q] = cl.x;
        clo[2 * q + 1] = cl.y;
        chi[2 * q] = ch.x;
        chi[2 * q + 1] = ch.y;
      } else {
        clo[q] = cl.x;
        chi[q] = ch.x;
      }
    }
    reinterpret_cast<uint8_t*>(scT)[(2 * l) * 4 + w] = static_cast<uint8_t>(slo);
    reinterpret_cast<uint8_t*>(scT)[(2 * l + 1) * 4 + w] = static_cast<uint8_t>(shi);
  }
  __syncthreads();  // every wave has read the tile: its LDS now holds the column codes
  uint32_t* outT = tile;  // [kQT][OP]
#pragma unroll
  for (int q = 0; q < WPB; ++q) {
    outT[(2 * l) * OP + w * WPB + q] = clo[q];
    outT[(2 * l + 1) * OP + w * WPB + q] = chi[q];
  }
  __syncthreads();
  // Phase 3: each column's 128 codes as 16-byte stores (eight, or four for E2M1), and its four
  // scales as one word.
  constexpr int PPC = WPC / 4;  // 16-byte pieces per column
#pragma unroll
  for (int j = 0; j < kQT * PPC / 256; ++j) {
    const int idx = t + 256 * j, c = idx / PPC, part = idx % PPC;
    const uint4 v = make_uint4(outT[c * OP + part * 4], outT[c * OP + part * 4 + 1],
                               outT[c * OP + part * 4 + 2], outT[c * OP + part * 4 + 3]);
    *reinterpret_cast<uint4*>(tq + (((size_t)b * C + c0 + c) * R + r0) * F / 8 + part * 16) = v;
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

// ------------------------------------------------------------------------------------------
// MXFP8 weight gradients: both operands quantised along the positions of each expert segment.
//
// Segment layout: expert e's positions are stored from poff[e] on, padded to npad_e = the count
// rounded up to 128 (one scaled-MFMA K step), so poff is the exclusive scan of npad. One
// workgroup of 1024 threads (E <= 1024).
__global__ void __launch_bounds__(1024) seg_offsets_kernel(const int32_t* __restrict__ offsets,
                                                           int E, int32_t* __restrict__ poff) {
  __shared__ int scan[1024];
  const int e = threadIdx.x;
  const int c = e < E ? offsets[e + 1] - offsets[e] : 0;
  const int np = (c + kSegK - 1) / kSegK * kSegK;
  scan[e] = np;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int u = e >= off ? scan[e - off] : 0;
    __syncthreads();
    scan[e] += u;
    __syncthreads();
  }
  if (e < E) poff[e] = scan[e] - np;
  if (e == 1023) poff[E] = scan[1023];
}

// Q [C][P]: column c of an operand S [T*k, C] (position-major), expert by expert, quantised
// along the positions in blocks of 32 from each segment's first position; codes past a
// segment's count are zero (an all-padding block gets scale code 0). QS [C][P / 32] holds the
// scale codes. S is read as
//  * SRC_BF16: bf16 rows src [T*k, C];
//  * SRC_FP8: the MXFP8 image (codes src8, per-32 scales src8s along C), expanded exactly;
//  * SRC_WDY: w * dY[t] in fp32 for the row r = row_src[pos] of position pos, w = topk_w[r]
//    and t = r / k (dY bf16 [T, C]): the down weight gradient's left operand, quantised from
//    its fp32 value (no bf16 rounding in between).
// Block (q, y): padded positions [128 q, 128 q + 128) (one expert, found by binary search over
// poff) x columns [64 y, 64 y + 64). The 128 x 64 tile goes through LDS as fp32, then thread t
// quantises column t / 4, rows [32 (t % 4), +32), and writes the block's 32 codes as two
// 16-byte stores.
enum SegSrc { SRC_BF16, SRC_FP8, SRC_WDY };
template <int SRC>
__global__ void __launch_bounds__(256) quant_seg_kernel(const uint16_t* __restrict__ src,
                                                        const uint8_t* __restrict__ src8,
                                                        const uint8_t* __restrict__ src8s,
                                                        const int32_t* __restrict__ row_src,
                                                        const float* __restrict__ topk_w, int k,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ poff, int E,
                                                        int C, int P, uint8_t* __restrict__ q,
                                                        uint8_t* __restrict__ qs) {
  constexpr int LD = 64 + 1;  // fp32 LDS row pitch: column reads of 32 rows spread over banks
  __shared__ float tile[kSegK * LD];
  const int pstart = blockIdx.x * kSegK;
  if (pstart >= poff[E]) return;  // whole workgroup
  int lo = 0, hi = E;  // largest e with poff[e] <= pstart
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (poff[mid] <= pstart) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int rel = pstart - poff[e];
  const int nvalid = min(kSegK, offsets[e + 1] - offsets[e] - rel);
  const size_t row0 = (size_t)offsets[e] + rel;
  const int c0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = tid + 256 * j, r = i / 8, pc = i % 8;  // row r, 8-column piece pc
    float f[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (r < nvalid) {
      const size_t row = row0 + r;
      if constexpr (SRC == SRC_FP8) {
        const uint2 c8 = *reinterpret_cast<const uint2*>(src8 + row * C + c0 + pc * 8);
        const float sc = mx_scale(src8s[row * (C / 32) + (c0 + pc * 8) / 32]);
        float a[4], b[4];
        e4m3x4_to_f32(c8.x, a);
        e4m3x4_to_f32(c8.y, b);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          f[h] = a[h] * sc;
          f[4 + h] = b[h] * sc;
        }
      } else {
        float w = 1.f;
        size_t srow = row;
        if constexpr (SRC == SRC_WDY) {
          const int rr = row_src[row];
          w = topk_w[rr];
          srow = (size_t)(rr / k);
        }
        const uint4 v = *reinterpret_cast<const uint4*>(src + srow * C + c0 + pc * 8);
        const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          f[2 * h] = w * bf2f_lo(vw[h]);
          f[2 * h + 1] = w * bf2f_hi(vw[h]);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < 8; ++h) tile[r * LD + pc * 8 + h] = f[h];
  }
  __syncthreads();
  const int c = tid / 4, b = tid % 4;
  float f[32];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    f[i] = tile[(32 * b + i) * LD + c];
    amax = fmaxf(amax, fabsf(f[i]));
  }
  const uint32_t code = mx_scale_code(amax);
  const float inv = mx_inv_scale(code);
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    o[i] = e4m3x2(f[4 * i] * inv, f[4 * i + 1] * inv) |
           (e4m3x2(f[4 * i + 2] * inv, f[4 * i + 3] * inv) << 16);
  uint8_t* dst = q + (size_t)(c0 + c) * P + pstart + 32 * b;
  *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
  *reinterpret_cast<uint4*>(dst + 16) = make_uint4(o[4], o[5], o[6], o[7]);
  qs[(size_t)(c0 + c) * (P / 32) + pstart / 32 + b] = static_cast<uint8_t>(code);
}

hipError_t launch_seg_offsets(const int32_t* offsets, int E, int32_t* poff, hipStream_t s) {
  {
    TraceScope trace("seg_offsets", s);
    hipLaunchKernelGGL(seg_offsets_kernel, dim3(1), dim3(1024), 0, s, offsets, E, poff);
  }
  return hipGetLastError();
}

hipError_t launch_quant_seg(const SegOperand& x, const int32_t* offsets, const int32_t* poff,
                            int E, int C, int P, uint8_t* q, uint8_t* qs, const char* name,
                            hipStream_t s) {
  const dim3 grid(P / kSegK, C / 64);
  {
    TraceScope trace(name, s);
    if (x.src8)
      hipLaunchKernelGGL(quant_seg_kernel<SRC_FP8>, grid, dim3(256), 0, s, x.src, x.src8,
                         x.src8s, x.row_src, x.topk_w, x.k, offsets, poff, E, C, P, q, qs);
    else if (x.row_src)
      hipLaunchKernelGGL(quant_seg_kernel<SRC_WDY>, grid, dim3(256), 0, s, x.src, x.src8,
                         x.src8s, x.row_src, x.topk_w, x.k, offsets, poff, E, C, P, q, qs);
    else
      hipLaunchKernelGGL(quant_seg_kernel<SRC_BF16>, grid, dim3(256), 0, s, x.src, x.src8,
                         x.src8s, x.row_src, x.topk_w, x.k, offsets, poff, E, C, P, q, qs);
  }
  return hipGetLastError();
}

hipError_t launch_quant_rows(const uint16_t* src, long long rows, int cols, uint8_t* dst,
                             uint8_t* sc, int fbits, const char* name, hipStream_t s) {
  const long long nvec = rows * cols / 8;
  if (nvec == 0) return hipSuccess;
  {
    TraceScope trace(name, s);
    const dim3 grid((unsigned)((nvec + 255) / 256));
    if (fbits == 4)
      hipLaunchKernelGGL(quant_rows_kernel<4>, grid, dim3(256), 0, s, src, dst, sc, nvec);
    else
      hipLaunchKernelGGL(quant_rows_kernel<8>, grid, dim3(256), 0, s, src, dst, sc, nvec);
  }
  return hipGetLastError();
}

hipError_t launch_quant_weight(const uint16_t* src, int B, int R, int C, uint8_t* dq,
                               uint8_t* dqs, uint8_t* tq, uint8_t* tqs, int fbits,
                               const char* name, hipStream_t s) {
  if (R % kQT != 0 || C % kQT != 0) return hipErrorInvalidValue;
  if (B == 0) return hipSuccess;
  {
    TraceScope trace(name, s);
    const dim3 grid(C / kQT, R / kQT, B);
    if (fbits == 4)
      hipLaunchKernelGGL(quant_weight_kernel<4>, grid, dim3(256), 0, s, src, dq, dqs, tq, tqs, R,
                         C);
    else
      hipLaunchKernelGGL(quant_weight_kernel<8>, grid, dim3(256), 0, s, src, dq, dqs, tq, tqs, R,
                         C);
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
