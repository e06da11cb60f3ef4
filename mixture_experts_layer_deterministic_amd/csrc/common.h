// Device-side helpers shared by the MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_DEV __device__ __forceinline__

namespace moe {

constexpr int kWave = 64;
constexpr int kXcds = 8;  // MI355X: workgroups are dealt round-robin over 8 XCDs

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// bfloat16 <-> fp32. The widening is exact; the narrowing rounds to nearest, ties to even
// (finite inputs; the layer never produces NaN or Inf from finite data of its scale).
MOE_DEV float bf2f(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }
MOE_DEV float bf2f_lo(uint32_t w) { return __uint_as_float(w << 16); }
MOE_DEV float bf2f_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
MOE_DEV uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
MOE_DEV uint32_t pack_bf2(float lo, float hi) { return f2bf(lo) | (f2bf(hi) << 16); }

// One v_mfma_f32_16x16x32_bf16. Lane l of each operand holds 8 K-values of the M (or N) index
// l % 16; the K slot of an element is fixed by (l / 16, element), identically for both operands.
// Passing the B fragment first computes the transposed product, so lane l ends up holding
// C[m = l % 16][n = 4 * (l / 16) + r], r = 0..3: four consecutive output columns of one row.
MOE_DEV f32x4 mfma16(const uint4& bfrag, const uint4& afrag, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bfrag),
                                                 __builtin_bit_cast(bf16x8, afrag), acc, 0, 0, 0);
}

MOE_DEV float silu(float g) { return g / (1.0f + __expf(-g)); }
MOE_DEV float sigmoid(float g) { return 1.0f / (1.0f + __expf(-g)); }

// Transpose an 8x8 block of 16-bit values held as 8 rows of 8 (uint4 each): out[c] holds column
// c of the input, i.e. out[c] element p = in[p] element c.
MOE_DEV void transpose8x8_b16(const uint4 (&in)[8], uint4 (&out)[8]) {
  const uint32_t* iw[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) iw[r] = reinterpret_cast<const uint32_t*>(&in[r]);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t a = iw[2 * p][c >> 1];
      const uint32_t b = iw[2 * p + 1][c >> 1];
      o[p] = (c & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
    out[c] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// Workgroup id remapped so that each XCD gets one contiguous range of logical tiles. The
// hardware deals workgroup b to XCD b % 8; the logical id (b % 8) * R + b / 8 gives XCD x the
// range [x R, (x+1) R). `total` must be rounded up to a multiple of 8 by the launch.
MOE_DEV int xcd_contiguous(int b, int total8) {
  const int R = total8 / kXcds;
  return (b % kXcds) * R + b / kXcds;
}

}  // namespace moe
