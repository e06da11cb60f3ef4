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
typedef __attribute__((ext_vector_type(8))) int i32x8;

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

// MXFP8 (OCP MX): E4M3 elements sharing one E8M0 scale per 32 along the reduction axis.
// Scale code of a block with max magnitude amax: floor(log2 amax) - 8 + 127, clamped to 0..254;
// 0 for an all-zero block. The fp32 exponent field is floor(log2 amax) + 127 for normal amax and
// 0 for zero or subnormal amax, so code = clamp(field - 8, 0, 254).
MOE_DEV uint32_t mx_scale_code(float amax) {
  const int e = static_cast<int>((__float_as_uint(amax) >> 23) & 0xffu);
  return static_cast<uint32_t>(min(max(e - 8, 0), 254));
}
// 2^(127 - code): multiplying by it maps a block onto the E4M3 range (fp32 amax keeps
// code <= 246, so the result is a normal float).
MOE_DEV float mx_inv_scale(uint32_t code) { return __uint_as_float((254u - code) << 23); }
// 2^(code - 127); code 0 is the fp32 subnormal 2^-127.
MOE_DEV float mx_scale(uint32_t code) {
  return code ? __uint_as_float(code << 23) : __uint_as_float(0x00400000u);
}
// Two scaled fp32 values to two E4M3 codes (low 16 bits): saturate to +-448, then the
// hardware conversion rounds to nearest even (it does not saturate by itself).
MOE_DEV uint32_t e4m3x2(float a, float b) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xffffu;
}
// Four E4M3 codes packed in a dword to fp32 (exact).
MOE_DEV void e4m3x4_to_f32(uint32_t w, float (&f)[4]) {
  typedef __attribute__((ext_vector_type(2))) float f32x2;
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
  const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
  f[0] = lo[0];
  f[1] = lo[1];
  f[2] = hi[0];
  f[3] = hi[1];
}

// MXFP4 (OCP MX): E2M1 elements (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) sharing one E8M0 scale
// per 32, packed two to a byte with element 2i in the low nibble. The scale code is
// floor(log2 amax) - 2 + 127 (2 being E2M1's largest exponent), clamped to 0..254, 0 for an
// all-zero block; mx_inv_scale and mx_scale read it as for MXFP8.
MOE_DEV uint32_t mx4_scale_code(float amax) {
  const int e = static_cast<int>((__float_as_uint(amax) >> 23) & 0xffu);
  return static_cast<uint32_t>(min(max(e - 2, 0), 254));
}
// Four scaled fp32 values to four E2M1 codes in the low 16 bits (value i in bits 4 i .. 4 i + 3)
// by gfx950's scaled conversion with a unit scale, which rounds to the nearest magnitude, a tie
// to the even code, saturates magnitudes past 6 to 6 and keeps the value's sign bit (so a
// negative value that rounds to zero gives -0, code 8): the format's rounding. Measured
// against a comparison chain of that rule on every multiple of 1/128 in [-16, 16] (every tie and
// its neighbours) and on huge, tiny and subnormal values: no difference.
MOE_DEV uint32_t e2m1x4(float a, float b, float c, float d) {
  const uint32_t lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, c, d, 1.0f, 1);
}
// The values of the two E2M1 codes in byte SEL of w (exact in fp32), low nibble first.
template <int SEL>
MOE_DEV float2 e2m1x2_to_f32(uint32_t w) {
  const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
  return make_float2(v[0], v[1]);
}

// 16 bytes read once: a non-temporal load, so a single-use stream does not push reused data
// (router rows, index arrays) out of the caches. Measured on the un-permute at the DeepSeek-V3
// shape: 89-103 -> 58 us.
MOE_DEV uint4 nt_load16(const void* p) {
  typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Four consecutive fp32 weight-gradient values stored at p; with ACC added to what p holds.
template <bool ACC>
MOE_DEV void store_dw4(float* p, const f32x4& v) {
  float4 o = make_float4(v[0], v[1], v[2], v[3]);
  if (ACC) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    o.x += q.x;
    o.y += q.y;
    o.z += q.z;
    o.w += q.w;
  }
  *reinterpret_cast<float4*>(p) = o;
}

// Two side-by-side 16 x 16 MFMA output blocks (columns c0 .. c0 + 31) stored as bf16, with ACC
// added in fp32 to what is stored. Lane l holds row l % 16, columns c0 + 4 (l / 16) .. + 3 of
// lo and c0 + 16 + 4 (l / 16) .. + 3 of hi. Lanes l and l ^ 16 swap one block's values so that
// each lane holds 8 consecutive columns and the four lanes of a row cover its 64 contiguous
// bytes: the memory system then takes one 64-byte write per row, where the blocks' own 8-byte
// pieces made two of 32 bytes (write requests, not bytes, set the rate of a bf16 dW store).
// row: this lane's row at column c0 (64-byte aligned).
template <bool ACC>
MOE_DEV void store_dw8_bf16(uint16_t* row, const f32x4& lo, const f32x4& hi, int lane) {
  const int g = lane / 16;
  const bool even = (g & 1) == 0;
  float send[4], recv[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) send[q] = even ? hi[q] : lo[q];
#pragma unroll
  for (int q = 0; q < 4; ++q) recv[q] = __shfl_xor(send[q], 16);
  float o[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    o[q] = even ? lo[q] : recv[q];
    o[4 + q] = even ? recv[q] : hi[q];
  }
  // even g: columns 4 g .. 4 g + 7; odd g: 16 + 4 (g - 1) .. + 7
  uint4* p = reinterpret_cast<uint4*>(row + (even ? 4 * g : 12 + 4 * g));
  if (ACC) {
    const uint4 v = *p;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o[2 * q] += bf2f_lo(w[q]);
      o[2 * q + 1] += bf2f_hi(w[q]);
    }
  }
  *p = make_uint4(pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]), pack_bf2(o[4], o[5]),
                  pack_bf2(o[6], o[7]));
}

MOE_DEV float silu(float g) { return g / (1.0f + __expf(-g)); }
MOE_DEV float sigmoid(float g) { return 1.0f / (1.0f + __expf(-g)); }

// LDS tiles of 64 bf16 per row (128 bytes, no padding) whose 16-byte chunks are permuted per
// row: chunk c of row r sits at chunk c ^ (r & 7). Element offset of (row, chunk). An MFMA
// fragment read (16 rows, one chunk each, per 16 lanes) and a row store (8 chunks of a row per
// 8 lanes) then both spread over all banks. Measured with 16-byte reads in the fragment
// pattern: about 180 bytes per clock per CU, against 118 for rows padded to 144 bytes.
MOE_DEV int rowswz(int row, int chunk) { return row * 64 + ((chunk ^ (row & 7)) << 3); }

// K-major LDS tiles read as MFMA fragments. A tile of K rows x PITCH values (16-bit) is stored
// row by row as it sits in memory, with the 32-byte column groups of row k permuted by XOR
// with kmajor_swz(k) (a multiple of 16 elements, below 128): the four rows a 16-lane group
// reads at once, and the rows 8 further on, fall on different bank groups.
MOE_DEV int kmajor_swz(int k) { return 16 * ((k & 3) | ((k >> 1) & 4)); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
MOE_DEV s16x4 lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) s16x4* lds_ptr;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(p));
}

// MFMA fragment from a K-major LDS tile: lane l gets index base + l % 16 (a row or column of the
// product) at K rows kb + 8 (l / 16) .. + 8; base is a multiple of 16 and kb of 32. Within each
// group of 16 lanes, ds_read_b64_tr_b16 gives lane i element j of the 8 bytes that lane
// 4 j + i / 4 points at, taking element i % 4 of them (the layout was checked on the GPU with a
// one-hot matrix). Lane q of group g points at row kb + 8 g + q / 4, indices base + 4 (q % 4)
// .. + 4; so lane i receives rows kb + 8 g + 0..3 of index base + i, and the second read (4 rows
// on) the next four. The permutation of those rows does not depend on kb or on the 4-row step
// (kb is a multiple of 32, and q / 4 + 4 < 8), so both reads share one column and differ from
// other steps only by constant offsets.
template <int PITCH>
MOE_DEV uint4 kmajor_frag(const uint16_t* s, int base, int kb, int lane) {
  const int g = lane / 16, q = lane % 16, kr = 8 * g + q / 4;
  const int n = (base ^ kmajor_swz(kr)) + 4 * (q % 4);
  const uint16_t* p = s + (kb + kr) * PITCH + n;
  const s16x4 a = lds_read_tr16(p);
  const s16x4 b = lds_read_tr16(p + 4 * PITCH);
  uint4 v;
  v.x = (uint32_t)(uint16_t)a[0] | ((uint32_t)(uint16_t)a[1] << 16);
  v.y = (uint32_t)(uint16_t)a[2] | ((uint32_t)(uint16_t)a[3] << 16);
  v.z = (uint32_t)(uint16_t)b[0] | ((uint32_t)(uint16_t)b[1] << 16);
  v.w = (uint32_t)(uint16_t)b[2] | ((uint32_t)(uint16_t)b[3] << 16);
  return v;
}

// One 64-deep K step of a wave's MB x NB grid of 16 x 16 output blocks, as two 32-deep
// substeps, with fragments read from LDS: fa(ks, mb) returns the A fragment of row block mb and
// fb(ks, nb) the B fragment of column block nb for substep ks, issuing RA and RB LDS reads
// respectively. Both substeps walk the grid column by column. The reads go out ahead of the
// MFMAs that use them: all of substep 0's fragments first; then each B fragment's registers
// take its substep-1 successor once its column is issued, and during the last column each A
// fragment's registers take theirs. Every accumulator still sees substep 0 before substep 1.
// sched_group_barrier pins that order; left alone, the scheduler keeps fewer registers live by
// waiting for each fragment just before its MFMAs, which exposes the LDS latency eight times
// per substep.
template <int MB, int NB, int RA, int RB, class FA, class FB>
MOE_DEV void mma_k64(f32x4 (&acc)[MB][NB], FA fa, FB fb) {
  uint4 b[NB], a[MB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) b[nb] = fb(0, nb);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) a[mb] = fa(0, mb);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      acc[mb][nb] = mfma16(b[nb], a[mb], acc[mb][nb]);
      if (nb == NB - 1) a[mb] = fa(1, mb);
    }
    b[nb] = fb(1, nb);
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb][nb] = mfma16(b[nb], a[mb], acc[mb][nb]);
  // masks: 0x008 MFMA, 0x100 LDS read
  __builtin_amdgcn_sched_group_barrier(0x100, NB * RB + MB * RA, 0);
#pragma unroll
  for (int nb = 0; nb < NB - 1; ++nb) {
    __builtin_amdgcn_sched_group_barrier(0x008, MB, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, RB, 0);
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, RA, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, RB, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, MB * NB, 0);
}

// Workgroup id remapped so that each XCD gets one contiguous range of logical tiles. The
// hardware deals workgroup b to XCD b % 8; the logical id (b % 8) * R + b / 8 gives XCD x the
// range [x R, (x+1) R). `total` must be rounded up to a multiple of 8 by the launch.
MOE_DEV int xcd_contiguous(int b, int total8) {
  const int R = total8 / kXcds;
  return (b % kXcds) * R + b / kXcds;
}

}  // namespace moe
