// 256 x 256 MFMA tiles fed by direct global -> LDS loads (gfx950), shared by the grouped GEMMs
// (gemm.hip) and the weight gradients (wgrad.hip).
//
// In a register-staged K loop a step's loads are issued at the start of the step and written to
// LDS at its end, so they have one step to arrive, and a second step in flight would need 32
// more staging registers a lane does not have. Here each load writes LDS itself
// (buffer_load_dwordx4 with the LDS bit: lane l's 16 bytes land at byte 16 l of a 1 KB block
// whose base is M0), so no register holds a stage. Operand A moves through two stages and
// operand B through three, 32 KB each, 160 KB in all: a step's A loads have one step to arrive,
// its B loads two. B is the weight stream in the grouped GEMMs.
//
// The stages hold the register-staged layouts, so fragment reads and MFMAs are those of the
// register-staged kernels and so are the results, bit for bit:
//  * K-contiguous rows in rowswz's chunk-permuted rows. One load instruction covers 8 rows:
//    lane l fetches chunk (l % 8) ^ (l / 8) of row l / 8, each row one whole 128-byte line.
//  * K-major operands as 64 K rows of 256 values with kmajor_swz-permuted column groups, read
//    with the transposing LDS read. One instruction covers 2 K rows: lane l fetches the 8
//    values of row l / 32 that belong at position l % 32.
//
// The five stages are distinct LDS arrays and the K loop is unrolled by six (both stage
// cycles), so the compiler can tell which stage each load writes and each read reads, and does
// not wait for every load in flight before an LDS read. A wave's loads complete in issue order;
// a step issues the A loads of step kt + 1 before the B loads of step kt + 2, so at the top of
// step kt only the four B loads issued last may still be in flight. The step waits for the
// rest, then meets the other waves at a bare barrier: a workgroup fence there would wait for
// every load, since loads into LDS count as LDS writes. Loads past the last K chunk reload the
// last chunk into a free stage, so every step issues the same eight loads and the count holds.
//
// A trait D describes one product:
//   Args, Tile; kName; ntiles(a); decode(a, lt) -> Tile;
//   kAKmajor, kBKmajor: operand layouts (K-contiguous rows, or K-major);
//   brow(wn, nb): LDS row of B's column block nb for wave column wn (K-contiguous B);
//   kVoffStep: the K advance rides in the lane offset and the scalar offset stays zero, so a
//     buffer range limit (checked against the lane offset) zeroes the rows past the operand's
//     end;
//   kRoundOrder: tiles dealt round by round (tile r G + x G/8 + s to workgroup s of XCD x)
//     instead of one contiguous range per XCD;
//   src(a, t, wave, lane, DmaSrc&): the lane's sources; epilogue(a, t, acc).
// Wave tiles are 128 x 64 (waves 2 along M x 4 along N), accumulators as mfma16 leaves them.
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kDmaStage = 256 * 64;  // uint16 per stage: 256 rows of 64 K values, or 64 x 256
__shared__ __align__(1024) uint16_t dma_a0[kDmaStage];
__shared__ __align__(1024) uint16_t dma_a1[kDmaStage];
__shared__ __align__(1024) uint16_t dma_b0[kDmaStage];
__shared__ __align__(1024) uint16_t dma_b1[kDmaStage];
__shared__ __align__(1024) uint16_t dma_b2[kDmaStage];

template <int S>
MOE_DEV uint16_t* dma_stage_a() {
  if constexpr (S == 0) return dma_a0;
  else return dma_a1;
}
template <int S>
MOE_DEV uint16_t* dma_stage_b() {
  if constexpr (S == 0) return dma_b0;
  else if constexpr (S == 1) return dma_b1;
  else return dma_b2;
}

// Buffer resource over `bytes` bytes from base (raw: stride 0; gfx9 data format word): loads
// at or past the end return zeros. The default covers a whole tensor.
MOE_DEV __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t bytes = 0xffffffffu) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from rsrc's base + soff + voff bytes to LDS at lds + 16 * lane bytes (rsrc,
// soff and lds the same in every lane).
MOE_DEV void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff, uint16_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds,
                                           16, voff, soff, 0, 0);
}

// A 16-byte LDS read as one vector load. Read as a uint4 struct, the load is split into four
// 32-bit loads and put back together late, and the rebuilt load loses the alias scope that
// tells the stages apart: the compiler then waits for every load in flight before it.
MOE_DEV uint4 lds_read16(const uint16_t* p) {
  typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// kmajor_frag over a 256-wide stage, each transposing read through a restrict pointer of its
// own: the inlined intrinsic then carries an alias scope, and the compiler can tell it apart
// from the loads still writing other stages.
MOE_DEV s16x4 lds_read_tr16_scoped(const uint16_t* __restrict__ p) {
  typedef __attribute__((address_space(3))) s16x4* lds_ptr;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(p));
}
MOE_DEV uint4 kmajor_frag_dma(const uint16_t* s, int base, int kb, int lane) {
  const int g = lane / 16, q = lane % 16, kr = 8 * g + q / 4;
  const int n = (base ^ kmajor_swz(kr)) + 4 * (q % 4);
  const s16x4 a = lds_read_tr16_scoped(s + (kb + kr) * 256 + n);
  const s16x4 b = lds_read_tr16_scoped(s + (kb + kr + 4) * 256 + n);
  uint4 v;
  v.x = (uint32_t)(uint16_t)a[0] | ((uint32_t)(uint16_t)a[1] << 16);
  v.y = (uint32_t)(uint16_t)a[2] | ((uint32_t)(uint16_t)a[3] << 16);
  v.z = (uint32_t)(uint16_t)b[0] | ((uint32_t)(uint16_t)b[1] << 16);
  v.w = (uint32_t)(uint16_t)b[2] | ((uint32_t)(uint16_t)b[3] << 16);
  return v;
}

// gfx9 s_waitcnt immediates: vmcnt [3:0], expcnt [6:4], lgkmcnt [11:8]
constexpr int kWaitVm4Lgkm0 = 0x0074;  // vmcnt(4) lgkmcnt(0)
constexpr int kWaitVm0Lgkm0 = 0x0070;  // vmcnt(0) lgkmcnt(0)

// A lane's loads for one tile: the two operands' buffer resources, the byte offsets of the
// pieces its four A and four B load instructions fetch, and the bytes one K chunk advances each
// operand; K chunks run k0, k0 + 1, .., nk - 1, 0, .., k0 - 1.
struct DmaSrc {
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t ao[4], bo[4];
  uint32_t astep, bstep;
  int k0, nk;
};

// Row (of 256) that load j of a lane fetches in a K-contiguous tile, and the byte offset of its
// 16-byte piece within the 64-value K chunk.
MOE_DEV int dma_row(int wave, int j, int lane) { return 32 * wave + 8 * j + lane / 8; }
MOE_DEV uint32_t dma_piece(int lane) { return 16u * ((lane % 8) ^ (lane / 8)); }
// K row (of 64) that load j of a lane fetches in a K-major tile, and the byte offset of its
// 8 values within the row's 256.
MOE_DEV int dma_krow(int wave, int j, int lane) { return 8 * wave + 2 * j + lane / 32; }
MOE_DEV uint32_t dma_kpiece(int kr, int lane) {
  return 2u * (((lane % 32) * 8) ^ kmajor_swz(kr));
}

// K chunk kt of the tile (clamped to the last) into A stage S, or B stage S: the wave's 1 KB
// quarter of the stage, four load instructions.
template <class D, int S>
MOE_DEV void dma_issue_a(const DmaSrc& s, int kt, int wave) {
  int kk = min(kt, s.nk - 1) + s.k0;
  kk = kk >= s.nk ? kk - s.nk : kk;
  const uint32_t step = (uint32_t)kk * s.astep;
  uint16_t* st = dma_stage_a<S>() + wave * 2048;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (D::kVoffStep)
      dma16(s.ra, s.ao[j] + step, 0, st + j * 512);
    else
      dma16(s.ra, s.ao[j], step, st + j * 512);
  }
}
template <class D, int S>
MOE_DEV void dma_issue_b(const DmaSrc& s, int kt, int wave) {
  int kk = min(kt, s.nk - 1) + s.k0;
  kk = kk >= s.nk ? kk - s.nk : kk;
  const uint32_t step = (uint32_t)kk * s.bstep;
  uint16_t* st = dma_stage_b<S>() + wave * 2048;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (D::kVoffStep)
      dma16(s.rb, s.bo[j] + step, 0, st + j * 512);
    else
      dma16(s.rb, s.bo[j], step, st + j * 512);
  }
}

// K step kt on A stage SA and B stage SB: wait for them, refill the stages the previous step
// read (A of step kt + 1, B of step kt + 2), then the 64-deep MFMA step of a 128 x 64 wave
// tile.
template <class D, int SA, int SB>
MOE_DEV void dma_step(f32x4 (&acc)[8][4], const DmaSrc& s, int kt, int wave, int wm, int wn,
                      int lane) {
  __builtin_amdgcn_s_waitcnt(kWaitVm4Lgkm0);
  __builtin_amdgcn_s_barrier();
  dma_issue_a<D, SA ^ 1>(s, kt + 1, wave);
  dma_issue_b<D, (SB + 2) % 3>(s, kt + 2, wave);
  __builtin_amdgcn_sched_barrier(0);
  const uint16_t* sA = dma_stage_a<SA>();
  const uint16_t* sB = dma_stage_b<SB>();
  const int c0 = ((lane / 16) ^ (lane & 7)) << 3, c1 = ((4 + lane / 16) ^ (lane & 7)) << 3;
  const uint16_t* sAl = sA + (wm * 128 + lane % 16) * 64;
  const uint16_t* sBl = sB + (lane % 16) * 64;
  auto fa_rows = [&](int ks, int mb) { return lds_read16(sAl + mb * 16 * 64 + (ks ? c1 : c0)); };
  auto fa_kmaj = [&](int ks, int mb) {
    return kmajor_frag_dma(sA, wm * 128 + mb * 16, ks * 32, lane);
  };
  auto fb_rows = [&](int ks, int nb) {
    return lds_read16(sBl + D::brow(wn, nb) * 64 + (ks ? c1 : c0));
  };
  auto fb_kmaj = [&](int ks, int nb) {
    return kmajor_frag_dma(sB, wn * 64 + nb * 16, ks * 32, lane);
  };
  if constexpr (D::kAKmajor && D::kBKmajor)
    mma_k64<8, 4, 2, 2>(acc, fa_kmaj, fb_kmaj);
  else if constexpr (D::kBKmajor)
    mma_k64<8, 4, 1, 2>(acc, fa_rows, fb_kmaj);
  else
    mma_k64<8, 4, 1, 1>(acc, fa_rows, fb_rows);
}

template <class D>
__global__ void __launch_bounds__(512, 2) dma_kernel(const typename D::Args a) {
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wm = wave / 4, wn = wave % 4;
  const int ntiles = D::ntiles(a);
  const int R = (ntiles + kXcds - 1) / kXcds;
  const int G = gridDim.x, G8 = G / kXcds, xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  for (int it = 0;; ++it) {
    int lt;
    if constexpr (D::kRoundOrder) {
      lt = it * G + xcd * G8 + slot;
      if (lt >= ntiles) break;
    } else {
      const int sidx = slot + it * G8;  // XCD x takes tiles [x R, (x+1) R)
      if (sidx >= R) break;
      lt = xcd * R + sidx;
      if (lt >= ntiles) break;
    }
    const typename D::Tile t = D::decode(a, lt);
    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    DmaSrc s;
    D::src(a, t, wave, lane, s);
    if (s.nk > 0) {
      dma_issue_a<D, 0>(s, 0, wave);
      dma_issue_b<D, 0>(s, 0, wave);
      dma_issue_b<D, 1>(s, 1, wave);
      for (int kt = 0;; kt += 6) {
        dma_step<D, 0, 0>(acc, s, kt, wave, wm, wn, lane);
        if (kt + 1 >= s.nk) break;
        dma_step<D, 1, 1>(acc, s, kt + 1, wave, wm, wn, lane);
        if (kt + 2 >= s.nk) break;
        dma_step<D, 0, 2>(acc, s, kt + 2, wave, wm, wn, lane);
        if (kt + 3 >= s.nk) break;
        dma_step<D, 1, 0>(acc, s, kt + 3, wave, wm, wn, lane);
        if (kt + 4 >= s.nk) break;
        dma_step<D, 0, 1>(acc, s, kt + 4, wave, wm, wn, lane);
        if (kt + 5 >= s.nk) break;
        dma_step<D, 1, 2>(acc, s, kt + 5, wave, wm, wn, lane);
        if (kt + 6 >= s.nk) break;
      }
      // the trailing reloads have landed and no wave still reads a stage: the epilogue may use
      // LDS, and the next tile's first loads may go out once it is done
      __builtin_amdgcn_s_waitcnt(kWaitVm0Lgkm0);
      __builtin_amdgcn_s_barrier();
    }
    D::epilogue(a, t, acc);
  }
}

// Grid: one-shot grids cover every tile, persistent grids are the resident workgroup count
// (one per CU: the stages take all of its LDS); both multiples of 8.
template <class D>
hipError_t launch_dma(const typename D::Args& a, int max_tiles, bool persistent,
                      hipStream_t stream) {
  if (max_tiles <= 0) return hipSuccess;
  int grid = (max_tiles + kXcds - 1) / kXcds * kXcds;
  if (persistent) {
    static int resident = 0;  // per kernel; every device of one process is an MI355X
    if (resident == 0) {
      int dev = 0, cus = 0, per_cu = 0;
      hipError_t e = hipGetDevice(&dev);
      if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
      if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(&dma_kernel<D>), 512, 0);
      if (e != hipSuccess) return e;
      resident = (cus * (per_cu > 0 ? per_cu : 1)) / kXcds * kXcds;
    }
    if (resident > 0 && resident < grid) grid = resident;
  }
  {
    TraceScope trace(D::kName, stream);
    hipLaunchKernelGGL(dma_kernel<D>, dim3(grid), dim3(512), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace
}  // namespace moe
