// Expert-grouped GEMMs of the MoE layer on gfx950 MFMA (bf16 in, fp32 accumulate).
//
// The expert-grouped GEMMs are named in the MarkTechPost page on Mixture-of-Kittens (MoK),
// section "Three design decisions that matter". This file holds the four whose rows are
// token positions:
//   fwd  gate/up : [g|u][pos]   = Xp[pos]  . W1[e]^T      SwiGLU in the epilogue
//   fwd  down    : O[pos]       = A[pos]   . W2[e]^T
//   bwd  down dg : dA'[pos]     = dY[t]    . W2[e]        SwiGLU backward + router-weight grad
//   bwd  gate dg : dXp[pos]     = dH[pos]  . W1[e]
// The two weight gradients have their own kernel (wgrad.hip). One kernel template runs the
// four, in BF16 and (further down) in MXFP8. A workgroup owns a 128 x 128 output tile with 4
// waves; the full 256-row expert blocks of all four run on 256 x 256 tiles with 8 waves and
// direct global -> LDS loads (dma.h). Tiles of BK stream through double-buffered LDS, stored
// K-contiguous in rows of 64 values whose 16-byte chunks are permuted per row (rowswz), so every
// MFMA fragment is one 16-byte LDS read and neither those reads nor the row stores conflict on
// banks. In the 128 x 128 dgrads the weights, whose K axis is not contiguous in memory, sit in
// LDS as they are in memory and reach the MFMAs through gfx950's transposing LDS read.
//
// Determinism: every output element is produced by exactly one workgroup, which reduces K in a
// fixed order. There are no atomics and no split-K.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "dma.h"
#include "gemm_tiles.h"
#include "kernels.h"

namespace moe {


// ------------------------------------------------------------------------------------------
// Problem 3: backward down dgrad with the SwiGLU backward and the router-weight gradient fused
// into the epilogue. dA'[pos, i] = sum_n dY[t, n] W2[e][n, i] with t = row_src[pos] / k.
// Epilogue per (pos, i): partial dw += dA' * A (summed over the tile's columns in a fixed
// order: register, then lane groups, then waves), dA = w dA', and the SwiGLU derivative.
struct BwdDownDgrad {
  static constexpr const char* kName = "bwd_down_dgrad";
  using G = Geo<128, 128, 64, 1, 4>;
  static constexpr bool kBKMajor = true;  // W2[e] tiles are K-major (LoadKM)
  struct Args {
    const uint16_t* dy;      // [T, d]
    const int32_t* row_src;  // [T*k]
    const float* topk_w;     // [T*k] flat (row r)
    const uint16_t* w2;      // [E, d, I]
    const uint16_t* H;       // [T*k, 2I]
    const uint16_t* A;       // [T*k, I]
    uint16_t* dH;            // [T*k, 2I]
    float* dwpart;           // [T*k, I / BN]
    const int32_t* offsets;
    const int2* sched;
    int d, I, k;
  };
  struct Tile {
    MTile m;
    int n0;
  };
  static MOE_DEV int ntiles(const Args& a) { return a.sched[0].x * (a.I / G::BN); }
  static MOE_DEV Tile decode(const Args& a, int lt) {
    const int ntc = a.I / G::BN;
    const int2 mn = tile_mn<true>(lt, a.sched[0].x, ntc);
    Tile t;
    t.m = decode_mtile(a.sched, mn.x);
    t.n0 = mn.y * G::BN;
    return t;
  }
  static MOE_DEV int num_k(const Args& a, const Tile&) { return a.d / G::BK; }
  static MOE_DEV int k_first(const Tile&, int) { return 0; }
  static MOE_DEV bool m_active(const Tile& t, int m) { return m < t.m.mcount; }
  static MOE_DEV int brow(int wn, int nb) { return wn * G::WN + nb * 16; }
  struct Loader {
    LoadK<G::BM, G::BK, G::LDK, kThreads, false> la;
    LoadKM<G::BN, G::BK> lb;
    const uint16_t* wb;
    int ldw;
    MOE_DEV void init(const Args& a, const Tile& t) {
      const int32_t* rs = a.row_src;
      const int d = a.d, k = a.k, mc = t.m.mcount, row0 = t.m.row0;
      la.init(a.dy, [&](int m) { return (long long)(rs[row0 + min(m, mc - 1)] / k) * d; });
      wb = a.w2 + (size_t)t.m.e * a.d * a.I + t.n0;
      ldw = a.I;
    }
    MOE_DEV void load(int kt) {
      la.load(kt * G::BK);
      const uint16_t* w = wb;
      const int ld = ldw;
      lb.load(w + (size_t)(kt * G::BK) * ld, ld);
    }
    MOE_DEV void store(uint16_t* s) const {
      la.store(s);
      lb.store(s + G::BM * G::LDK);
    }
  };
  static MOE_DEV void epilogue(const Args& a, const Tile& t, f32x4 (&acc)[G::MB][G::NB],
                               uint16_t* smem) {
    const int lane = threadIdx.x % kWave, wn = (threadIdx.x / kWave) % G::WAVES_N;
    float* red = reinterpret_cast<float*>(smem);  // [WAVES_N][BM]; LDS is free after the K loop
    const int I = a.I;
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb) {
      const int m = mb * 16 + lane % 16;
      const bool live = m < t.m.mcount;
      float part = 0.f;
      if (live) {
        const size_t pos = t.m.row0 + m;
        const float w = a.topk_w[a.row_src[pos]];
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb) {
          const int i = t.n0 + wn * G::WN + nb * 16 + 4 * (lane / 16);
          const uint2 av = *reinterpret_cast<const uint2*>(a.A + pos * I + i);
          const uint2 gv = *reinterpret_cast<const uint2*>(a.H + pos * 2 * I + i);
          const uint2 uv = *reinterpret_cast<const uint2*>(a.H + pos * 2 * I + I + i);
          const float av4[4] = {bf2f_lo(av.x), bf2f_hi(av.x), bf2f_lo(av.y), bf2f_hi(av.y)};
          const float g4[4] = {bf2f_lo(gv.x), bf2f_hi(gv.x), bf2f_lo(gv.y), bf2f_hi(gv.y)};
          const float u4[4] = {bf2f_lo(uv.x), bf2f_hi(uv.x), bf2f_lo(uv.y), bf2f_hi(uv.y)};
          float dg[4], du[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float dap = acc[mb][nb][r];
            part = __builtin_fmaf(dap, av4[r], part);
            const float dA = w * dap;
            const float s = sigmoid(g4[r]);
            dg[r] = dA * u4[r] * s * (1.0f + g4[r] * (1.0f - s));
            du[r] = dA * (g4[r] * s);
          }
          uint2 o;
          o.x = pack_bf2(dg[0], dg[1]);
          o.y = pack_bf2(dg[2], dg[3]);
          *reinterpret_cast<uint2*>(a.dH + pos * 2 * I + i) = o;
          o.x = pack_bf2(du[0], du[1]);
          o.y = pack_bf2(du[2], du[3]);
          *reinterpret_cast<uint2*>(a.dH + pos * 2 * I + I + i) = o;
        }
      }
      // lanes l, l^16, l^32, l^48 share row m: butterfly in a fixed pattern
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      if (lane < 16) red[wn * G::BM + m] = part;
    }
    __syncthreads();
    if (threadIdx.x < G::BM && threadIdx.x < t.m.mcount) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < G::WAVES_N; ++w) s += red[w * G::BM + threadIdx.x];
      const size_t pos = t.m.row0 + threadIdx.x;
      a.dwpart[pos * (a.I / G::BN) + t.n0 / G::BN] = s;
    }
  }
};

// ------------------------------------------------------------------------------------------
// Problem 4: backward gate/up dgrad. dXp[pos] = dH[pos] . W1[e], stored bf16.
struct BwdGateDgrad {
  static constexpr const char* kName = "bwd_gate_dgrad";
  using G = Geo<128, 128, 64, 1, 4>;
  static constexpr bool kBKMajor = true;  // W1[e] tiles are K-major (LoadKM)
  struct Args {
    const uint16_t* dH;  // [T*k, 2I]
    const uint16_t* w1;  // [E, 2I, d]
    uint16_t* dXp;       // [T*k, d]
    const int32_t* offsets;
    const int2* sched;
    int d, I;
  };
  struct Tile {
    MTile m;
    int n0;
  };
  static MOE_DEV int ntiles(const Args& a) { return a.sched[0].x * (a.d / G::BN); }
  static MOE_DEV Tile decode(const Args& a, int lt) {
    const int ntc = a.d / G::BN;
    const int2 mn = tile_mn<true>(lt, a.sched[0].x, ntc);
    Tile t;
    t.m = decode_mtile(a.sched, mn.x);
    t.n0 = mn.y * G::BN;
    return t;
  }
  static MOE_DEV int num_k(const Args& a, const Tile&) { return 2 * a.I / G::BK; }
  static MOE_DEV int k_first(const Tile&, int) { return 0; }
  static MOE_DEV bool m_active(const Tile& t, int m) { return m < t.m.mcount; }
  static MOE_DEV int brow(int wn, int nb) { return wn * G::WN + nb * 16; }
  struct Loader {
    LoadK<G::BM, G::BK, G::LDK, kThreads, false> la;
    LoadKM<G::BN, G::BK> lb;
    const uint16_t* wb;
    int ldw;
    MOE_DEV void init(const Args& a, const Tile& t) {
      const int twoI = 2 * a.I, mc = t.m.mcount;
      // rows past the count repeat the last row, as in Problem 1's loader; the activations
      // stay first here (with the weights first the dgrads ran a quarter slower)
      la.init(a.dH + (size_t)t.m.row0 * twoI,
              [&](int m) { return (long long)min(m, mc - 1) * twoI; });
      wb = a.w1 + (size_t)t.m.e * 2 * a.I * a.d + t.n0;
      ldw = a.d;
    }
    MOE_DEV void load(int kt) {
      la.load(kt * G::BK);
      const uint16_t* w = wb;
      const int ld = ldw;
      lb.load(w + (size_t)(kt * G::BK) * ld, ld);
    }
    MOE_DEV void store(uint16_t* s) const {
      la.store(s);
      lb.store(s + G::BM * G::LDK);
    }
  };
  static MOE_DEV void epilogue(const Args& a, const Tile& t, f32x4 (&acc)[G::MB][G::NB],
                               uint16_t*) {
    const int lane = threadIdx.x % kWave, wn = (threadIdx.x / kWave) % G::WAVES_N;
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb) {
      const int m = mb * 16 + lane % 16;
      if (m >= t.m.mcount) continue;
      const size_t pos = t.m.row0 + m;
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb) {
        const int n = t.n0 + wn * G::WN + nb * 16 + 4 * (lane / 16);
        uint2 o;
        o.x = pack_bf2(acc[mb][nb][0], acc[mb][nb][1]);
        o.y = pack_bf2(acc[mb][nb][2], acc[mb][nb][3]);
        *reinterpret_cast<uint2*>(a.dXp + pos * a.d + n) = o;
      }
    }
  }
};

// Problems 4 and 3 on full 256-row blocks, where an expert's rows make them MFMA-bound: 256 x
// 256 tiles of eight 128 x 64 wave tiles. The weights (W1[e] d-contiguous, W2[e] I-contiguous)
// are K-major here, and a register transpose of a 256-wide tile does not fit beside 128
// accumulators; so a K step of weights (64 rows, 256 columns) sits in LDS as it is in memory,
// with kmajor_swz-permuted column groups, and its MFMA fragments come from gfx950's transposing
// LDS read. The kernel (dma_kernel, with the forward products) is further on.
constexpr int kDgT = 256;  // tile rows and columns

struct GateDgradBigArgs {
  const uint16_t* dH;  // [T*k, 2I]
  const uint16_t* w1;  // [E, 2I, d]
  uint16_t* dXp;       // [T*k, d]
  const int32_t* offsets;
  const int2* big;     // full 256-row blocks: count, then (expert, first row)
  int d, I;
};

struct DownDgradBigArgs {
  const uint16_t* dy;      // [T, d]
  const int32_t* row_src;  // [T*k]
  const float* topk_w;     // [T*k] flat (row r)
  const uint16_t* w2;      // [E, d, I]
  const uint16_t* H;       // [T*k, 2I]
  const uint16_t* A;       // [T*k, I]
  uint16_t* dH;            // [T*k, 2I]
  float* dwpart;           // [T*k, I / 128]
  const int32_t* offsets;
  const int2* big;         // full 256-row blocks: count, then (expert, first row)
  int d, I, k;
};


// ------------------------------------------------------------------------------------------
// MX modes. Both operands are K-contiguous codes with one E8M0 scale per 32 along K: E4M3, one
// a byte (MXFP8, F = 8), or E2M1, two a byte with element 2i in the low nibble (MXFP4, F = 4).
// One v_mfma_scale_f32_16x16x128_f8f6f4 covers 16 x 16 outputs and 128 K. Its operand layout on
// gfx950 (lane l, row or column l % 16, group g = l / 16): for E4M3, bytes 0..15 hold K
// [16 g, 16 g + 16) and bytes 16..31 hold K [64 + 16 g, 64 + 16 g + 16); for E2M1, bytes 0..15
// hold K [32 g, 32 g + 32) and the upper half of the operand is not read. The scale of K block
// b = [32 b, 32 b + 32) comes from byte 0 of lane (row + 16 b) in both. A K step moves 128
// bytes of every row: 128 K of E4M3 (one MFMA) or 256 K of E2M1 (two MFMAs, on the row's
// 16-byte chunks g and 4 + g). LDS holds each stage as [BM][128] A codes, [BN][128] B codes
// (chunk-permuted rows, mxswz), then the step's block scales, 4 (E4M3) or 8 (E2M1) bytes a row.

// GS: the K extent is a multiple of 512, so each row's scales load 16 bytes at a time (LoadK8).
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int F_ = 8, bool GS_ = true>
struct GeoMx {
  static constexpr int F = F_;                     // bits per code
  static constexpr bool GS = GS_;
  static_assert(F == 8 || F == 4, "E4M3 or E2M1 codes");
  static constexpr int BM = BM_, BN = BN_, BK = 1024 / F;  // K per step
  static constexpr int SCW = BK / 128;             // 32-bit scale words per row and step
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int MB = WM / 16, NB = WN / 16;
  static constexpr int LDK = 128;                  // bytes per LDS row (chunks permuted)
  static constexpr int SC_OFF = (BM + BN) * LDK;   // byte offset of the scale words
  static constexpr int STAGE = SC_OFF + (BM + BN) * 4 * SCW;
  static constexpr int kSmem = 2 * STAGE;
  static constexpr bool kMx = true;
  static constexpr int THREADS = WAVES_M * WAVES_N * kWave;
  static constexpr int kWavesPerEU = 2;
  static_assert(WAVES_M * WAVES_N == 4 || WAVES_M * WAVES_N == 8, "4 or 8 waves per workgroup");
};
// Full 256-row blocks on the direct-to-LDS kernel (dmx_kernel): eight waves of 128 x 64.
template <int F>
using GeoMxBig = GeoMx<256, 256, 2, 4, F>;

// Byte offset of 16-byte chunk `chunk` of row `row` in an fp8 code tile of 128-byte rows, with
// the chunks permuted per row as in rowswz (chunk c of row r at c ^ (r & 7)): fragment reads
// and row stores then spread over all banks, where rows padded to 144 bytes conflicted.
MOE_DEV int mxswz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

// ROWS rows of codes, K-contiguous: 8 vectors of 16 bytes per step. Thread t < ROWS also moves
// row t's SCW scale words (the step's block scales). With GS (rows of a multiple of 16 scale
// bytes: K a multiple of 512) they come 16 bytes at a time, one load per 16 / (4 SCW) steps;
// otherwise one 4- or 8-byte load per step, a cache line per lane each time. The two forms are
// separate instantiations: one scale path that merged words loaded on different branches made
// the compiler wait for every load right after issuing it. Every row is real (a tile's rows
// past its expert's count repeat the expert's last row; their outputs are never stored), so
// the code loads carry no per-row condition, as in LoadK.
template <int ROWS, int LDK, int SCW, bool GS>
struct LoadK8 {
  static constexpr int VPR = 8;
  static constexpr int NV = ROWS * VPR;
  static constexpr int PT = (NV + kThreads - 1) / kThreads;
  static constexpr int SPG = 4 / SCW;  // steps per 16 bytes of scales
  static_assert(SCW == 1 || SCW == 2, "4 or 8 scale bytes per step");
  const uint8_t* rp[PT];
  uint4 r[PT];
  const uint8_t* sp;
  uint4 s4;      // GS: the scale words of SPG consecutive steps; else this step's in s4.x (.y)
  int sg, sidx;  // GS: the group held in s4 and this step's place in it

  // The scale arrays start 16-byte aligned.
  template <class RowPtr, class ScalePtr>
  MOE_DEV void init(RowPtr rowptr, ScalePtr scaleptr) {
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const int v = threadIdx.x + kThreads * j;
      rp[j] = rowptr(min(v / VPR, ROWS - 1));
    }
    sp = threadIdx.x < ROWS ? scaleptr(threadIdx.x) : nullptr;
    sg = -1;
    sidx = 0;
    s4 = make_uint4(0x7f7f7f7fu, 0x7f7f7f7fu, 0x7f7f7f7fu, 0x7f7f7f7fu);
  }
  // The scale words are picked in store(), so no load result is waited for here.
  MOE_DEV void load(int kt) {
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const int v = threadIdx.x + kThreads * j;
      r[j] = *reinterpret_cast<const uint4*>(rp[j] + (size_t)kt * 128 + (v % VPR) * 16);
    }
    if (!sp) return;
    if constexpr (GS) {
      if (kt / SPG != sg) {
        sg = kt / SPG;
        s4 = *reinterpret_cast<const uint4*>(sp + (size_t)sg * 16);
      }
      sidx = kt % SPG;
    } else if constexpr (SCW == 1) {
      s4.x = *reinterpret_cast<const uint32_t*>(sp + (size_t)kt * 4);
    } else {
      const uint2 w = *reinterpret_cast<const uint2*>(sp + (size_t)kt * 8);
      s4.x = w.x;
      s4.y = w.y;
    }
  }
  MOE_DEV void store(uint8_t* rows, uint32_t* scales) const {
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const int v = threadIdx.x + kThreads * j;
      if (v < NV) *reinterpret_cast<uint4*>(rows + mxswz(v / VPR, v % VPR)) = r[j];
    }
    if (threadIdx.x >= ROWS) return;
    // masks rather than a selected vector element, which the compiler would index in scratch
    if constexpr (!GS) {
      if constexpr (SCW == 1)
        scales[threadIdx.x] = s4.x;
      else
        *reinterpret_cast<uint2*>(scales + 2 * threadIdx.x) = make_uint2(s4.x, s4.y);
    } else if constexpr (SCW == 1) {
      const uint32_t m0 = 0u - (sidx == 0), m1 = 0u - (sidx == 1), m2 = 0u - (sidx == 2),
                     m3 = 0u - (sidx == 3);
      scales[threadIdx.x] = (s4.x & m0) | (s4.y & m1) | (s4.z & m2) | (s4.w & m3);
    } else {
      const uint32_t m0 = 0u - (sidx == 0), m1 = ~m0;
      *reinterpret_cast<uint2*>(scales + 2 * threadIdx.x) =
          make_uint2((s4.x & m0) | (s4.z & m1), (s4.y & m0) | (s4.w & m1));
    }
  }
};

template <class G>
using LoadA8 = LoadK8<G::BM, G::LDK, G::SCW, G::GS>;
template <class G>
using LoadB8 = LoadK8<G::BN, G::LDK, G::SCW, G::GS>;

template <class G>
MOE_DEV void mx_store_stage(const LoadA8<G>& la, const LoadB8<G>& lb, uint8_t* stage) {
  la.store(stage, reinterpret_cast<uint32_t*>(stage + G::SC_OFF));
  lb.store(stage + G::BM * G::LDK,
           reinterpret_cast<uint32_t*>(stage + G::SC_OFF) + G::BM * G::SCW);
}

MOE_DEV i32x8 mx_frag(const uint8_t* tile, int row, int g) {
  const uint4 lo = *reinterpret_cast<const uint4*>(tile + mxswz(row, g));
  const uint4 hi = *reinterpret_cast<const uint4*>(tile + mxswz(row, 4 + g));
  i32x8 v;
  v[0] = static_cast<int>(lo.x);
  v[1] = static_cast<int>(lo.y);
  v[2] = static_cast<int>(lo.z);
  v[3] = static_cast<int>(lo.w);
  v[4] = static_cast<int>(hi.x);
  v[5] = static_cast<int>(hi.y);
  v[6] = static_cast<int>(hi.z);
  v[7] = static_cast<int>(hi.w);
  return v;
}

// Half H of an operand read by mx_frag (chunk g for H = 0, chunk 4 + g for H = 1) as the
// operand of an E2M1 MFMA, which reads the lower four registers only.
template <int H>
MOE_DEV i32x8 mx_half(const i32x8& v) {
  i32x8 h;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = v[4 * H + i];
    h[4 + i] = v[4 * H + i];
  }
  return h;
}

// The scale bytes a lane of group g passes for one row: byte g of the step's word 0 (E4M3, and
// the first 128 K of E2M1) and of word 1 (the second 128 K of E2M1).
template <int SCW>
MOE_DEV int2 mx_scales(const uint32_t* sc, int row, int g) {
  if constexpr (SCW == 1) {
    return make_int2(static_cast<int>((sc[row] >> (8 * g)) & 0xffu), 0);
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(sc + 2 * row);
    return make_int2(static_cast<int>((w.x >> (8 * g)) & 0xffu),
                     static_cast<int>((w.y >> (8 * g)) & 0xffu));
  }
}

// acc += the step's product of one row block and one column block
template <int F>
MOE_DEV f32x4 mx_mfma(const i32x8& b, const i32x8& a, f32x4 acc, int2 bs, int2 as) {
  if constexpr (F == 8) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, acc, 0, 0, 0, bs.x, 0, as.x);
  } else {
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(mx_half<0>(b), mx_half<0>(a), acc, 4,
                                                           4, 0, bs.x, 0, as.x);
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(mx_half<1>(b), mx_half<1>(a), acc, 4,
                                                            4, 0, bs.y, 0, as.y);
  }
}

template <class P>
MOE_DEV void run_tile_mx(const typename P::Args& a, const typename P::Tile& t, uint8_t* smem) {
  using G = typename P::G;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int wm = wave / G::WAVES_N, wn = wave % G::WAVES_N;
  const int r16 = lane % 16, g = lane / 16;
  f32x4 acc[G::MB][G::NB];
#pragma unroll
  for (int i = 0; i < G::MB; ++i)
#pragma unroll
    for (int j = 0; j < G::NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = P::num_k(a, t);
  if (nk > 0) {
    const int k0 = P::k_first(t, nk);  // K-chunks run k0, k0 + 1, .., nk - 1, 0, .., k0 - 1
    typename P::Loader ld;
    ld.init(a, t);
    ld.load(k0);
    mx_store_stage<G>(ld.la, ld.lb, smem);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      uint8_t* cur = smem + (kt & 1) * G::STAGE;
      if (kt + 1 < nk) ld.load(kt + 1 + k0 < nk ? kt + 1 + k0 : kt + 1 + k0 - nk);
      const uint8_t* sA = cur;
      const uint8_t* sB = cur + G::BM * G::LDK;
      const uint32_t* scA = reinterpret_cast<const uint32_t*>(cur + G::SC_OFF);
      const uint32_t* scB = scA + G::BM * G::SCW;
      i32x8 bf[G::NB];
      int2 bs[G::NB];
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb) {
        const int row = P::brow(wn, nb) + r16;
        bf[nb] = mx_frag(sB, row, g);
        bs[nb] = mx_scales<G::SCW>(scB, row, g);
      }
#pragma unroll
      for (int mb = 0; mb < G::MB; ++mb) {
        if (!P::m_active(t, wm * G::WM + mb * 16)) continue;
        const int row = wm * G::WM + mb * 16 + r16;
        const i32x8 af = mx_frag(sA, row, g);
        const int2 as = mx_scales<G::SCW>(scA, row, g);
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb)
          acc[mb][nb] = mx_mfma<G::F>(bf[nb], af, acc[mb][nb], bs[nb], as);
      }
      if (kt + 1 < nk) mx_store_stage<G>(ld.la, ld.lb, smem + ((kt + 1) & 1) * G::STAGE);
      __syncthreads();
    }
  }
  P::epilogue(a, t, acc, smem);
  __syncthreads();
}

// MX image of 8 values held by one lane, with the block scale shared by the four lanes l, l^16,
// l^32, l^48 (one row's 32 consecutive columns): the scale code for F-bit codes. Every lane must
// call it.
template <int F>
MOE_DEV uint32_t mx_block_code(const float (&v)[8]) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 16));
  amax = fmaxf(amax, __shfl_xor(amax, 32));
  return F == 8 ? mx_scale_code(amax) : mx4_scale_code(amax);
}
// The codes of four values times inv: four E4M3 bytes, or four E2M1 nibbles in the low 16 bits.
template <int F>
MOE_DEV uint32_t mx_pack4(const float* v, float inv) {
  if constexpr (F == 8)
    return e4m3x2(v[0] * inv, v[1] * inv) | (e4m3x2(v[2] * inv, v[3] * inv) << 16);
  else
    return e2m1x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
}
// Stores four codes of mx_pack4 at elements [c, c + 4) of a row of codes (c a multiple of 4).
template <int F>
MOE_DEV void mx_put4(uint8_t* row, int c, uint32_t codes) {
  if constexpr (F == 8)
    *reinterpret_cast<uint32_t*>(row + c) = codes;
  else
    *reinterpret_cast<uint16_t*>(row + c / 2) = static_cast<uint16_t>(codes);
}

// Problem 1 (MXFP8): forward gate/up with SwiGLU. A tile covers BN / 2 gate columns and the
// matching up columns. Wave (wm, wn) owns rows [WM wm, +WM) and gate columns [32 wn, +32) of the
// tile's with the matching up columns, so one row's 32 consecutive A columns sit in four lanes
// of one wave and A is quantised (along I, for the down GEMM) in registers. G is the 128-row
// tile (2 x 2 waves) or the 256-row one of dmx_kernel (2 x 4 waves).
template <class G_>
struct MxFwdGateUpT {
  static constexpr const char* kName = "fwd_gateup";
  using G = G_;
  static constexpr int kA = G::BN / 2;  // A columns per tile
  static_assert(G::WN == 64, "each wave holds 32 gate and 32 up columns");
  struct Args {
    const uint8_t* xp8;  // [T*k, d] codes (ring slot)
    const uint8_t* xps;  // [T*k, d/32]
    const uint8_t* w8;   // [E, 2I, d]
    const uint8_t* ws;   // [E, 2I, d/32]
    uint16_t* H;         // [T*k, 2I]
    uint16_t* A;         // [T*k, I]
    uint8_t* aq;         // [T*k, I]
    uint8_t* aqs;        // [T*k, I/32]
    const int32_t* offsets;
    const int2* sched;
    int d, I;
  };
  struct Tile {
    MTile m;
    int n0;
  };
  static MOE_DEV int ntiles(const Args& a) { return a.sched[0].x * (a.I / kA); }
  static MOE_DEV Tile decode(const Args& a, int lt) {
    const int ntc = a.I / kA;
    Tile t;
    if constexpr (G::BM > 128) {  // grouped order: row blocks of one expert share weight panels
      const int2 mn = tile_mn<true>(lt, a.sched[0].x, ntc);
      t.m = decode_mtile(a.sched, mn.x);
      t.n0 = mn.y * kA;
    } else {
      t.m = decode_mtile(a.sched, lt / ntc);
      t.n0 = (lt % ntc) * kA;
    }
    return t;
  }
  static MOE_DEV int num_k(const Args& a, const Tile&) { return a.d / G::BK; }
  static MOE_DEV int k_first(const Tile&, int) { return 0; }
  static MOE_DEV bool m_active(const Tile& t, int m) { return m < t.m.mcount; }
  static MOE_DEV int brow(int wn, int nb) {
    return nb < 2 ? wn * 32 + nb * 16 : kA + wn * 32 + (nb - 2) * 16;
  }
  struct Loader {
    LoadA8<G> la;
    LoadB8<G> lb;
    MOE_DEV void init(const Args& a, const Tile& t) {
      const int d = a.d, I = a.I, mc = t.m.mcount, row0 = t.m.row0, n0 = t.n0;
      const uint8_t* xp8 = a.xp8;
      const uint8_t* xps = a.xps;
      const size_t pb = (size_t)d * G::F / 8;  // bytes of codes per row
      la.init([&](int m) { return xp8 + (size_t)(row0 + min(m, mc - 1)) * pb; },
              [&](int m) { return xps + (size_t)(row0 + min(m, mc - 1)) * (d / 32); });
      const size_t wrow0 = (size_t)t.m.e * 2 * I;
      const uint8_t* w8 = a.w8;
      const uint8_t* ws = a.ws;
      auto wrow = [=](int n) { return wrow0 + (n < kA ? n0 + n : I + n0 + n - kA); };
      lb.init([&](int n) { return w8 + wrow(n) * pb; },
              [&](int n) { return ws + wrow(n) * (d / 32); });
    }
    MOE_DEV void load(int kt) {  // weights first: they are the HBM stream
      lb.load(kt);
      la.load(kt);
    }
  };
  static MOE_DEV void epilogue(const Args& a, const Tile& t, f32x4 (&acc)[G::MB][G::NB],
                               uint8_t*) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int wm = wave / G::WAVES_N, wn = wave % G::WAVES_N;
    const int I = a.I;
    const int c0 = t.n0 + wn * 32;  // first of this wave's 32 A columns: a 32-block
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb) {
      const int m = wm * G::WM + mb * 16 + lane % 16;
      const bool live = m < t.m.mcount;
      const size_t pos = t.m.row0 + m;
      float av[8];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int j = c0 + nb * 16 + 4 * (lane / 16);
        const f32x4 gv = acc[mb][nb], uv = acc[mb][nb + 2];
        uint2 hg, hu, aw;
        hg.x = pack_bf2(gv[0], gv[1]);
        hg.y = pack_bf2(gv[2], gv[3]);
        hu.x = pack_bf2(uv[0], uv[1]);
        hu.y = pack_bf2(uv[2], uv[3]);
        aw.x = pack_bf2(silu(gv[0]) * uv[0], silu(gv[1]) * uv[1]);
        aw.y = pack_bf2(silu(gv[2]) * uv[2], silu(gv[3]) * uv[3]);
        av[4 * nb + 0] = bf2f_lo(aw.x);
        av[4 * nb + 1] = bf2f_hi(aw.x);
        av[4 * nb + 2] = bf2f_lo(aw.y);
        av[4 * nb + 3] = bf2f_hi(aw.y);
        if (live) {
          *reinterpret_cast<uint2*>(a.H + pos * 2 * I + j) = hg;
          *reinterpret_cast<uint2*>(a.H + pos * 2 * I + I + j) = hu;
          *reinterpret_cast<uint2*>(a.A + pos * I + j) = aw;
        }
      }
      const uint32_t code = mx_block_code<G::F>(av);
      const float inv = mx_inv_scale(code);
      if (live) {
        uint8_t* q = a.aq + pos * (I * G::F / 8);
        mx_put4<G::F>(q, c0 + 4 * (lane / 16), mx_pack4<G::F>(av, inv));
        mx_put4<G::F>(q, c0 + 16 + 4 * (lane / 16), mx_pack4<G::F>(av + 4, inv));
        if (lane < 16) a.aqs[pos * (I / 32) + c0 / 32] = static_cast<uint8_t>(code);
      }
    }
  }
};

template <int F, bool GS>
using MxFwdGateUpS = MxFwdGateUpT<GeoMx<128, 128, 2, 2, F, GS>>;
template <int F>
using MxFwdGateUpBig = MxFwdGateUpT<GeoMxBig<F>>;

// Problem 2 (MXFP8): forward down. O[pos] = A[pos] . W2[e]^T, with A and W2 quantised along I.
template <class G_>
struct MxFwdDownT {
  static constexpr const char* kName = "fwd_down";
  using G = G_;
  struct Args {
    const uint8_t* aq;   // [T*k, I]
    const uint8_t* aqs;  // [T*k, I/32]
    const uint8_t* w8;   // [E, d, I]
    const uint8_t* ws;   // [E, d, I/32]
    uint16_t* O;         // [T*k, d]
    const int32_t* offsets;
    const int2* sched;
    int d, I;
  };
  struct Tile {
    MTile m;
    int n0;
  };
  static MOE_DEV int ntiles(const Args& a) { return a.sched[0].x * (a.d / G::BN); }
  static MOE_DEV Tile decode(const Args& a, int lt) {
    const int ntc = a.d / G::BN;
    const int2 mn = tile_mn<(G::BM > 128)>(lt, a.sched[0].x, ntc);
    Tile t;
    t.m = decode_mtile(a.sched, mn.x);
    t.n0 = mn.y * G::BN;
    return t;
  }
  static MOE_DEV int num_k(const Args& a, const Tile&) { return a.I / G::BK; }
  // The quantised W2's rows are I bytes apart: as in the BF16 down GEMM, each n-tile starts at
  // its own K-chunk so that concurrent tiles do not read one aliased column of rows.
  static MOE_DEV int k_first(const Tile& t, int nk) { return (t.n0 / G::BN) % nk; }
  static MOE_DEV bool m_active(const Tile& t, int m) { return m < t.m.mcount; }
  static MOE_DEV int brow(int wn, int nb) { return wn * G::WN + nb * 16; }
  struct Loader {
    LoadA8<G> la;
    LoadB8<G> lb;
    MOE_DEV void init(const Args& a, const Tile& t) {
      const int I = a.I, mc = t.m.mcount, row0 = t.m.row0;
      const uint8_t* aq = a.aq;
      const uint8_t* aqs = a.aqs;
      const size_t pb = (size_t)I * G::F / 8;  // bytes of codes per row
      la.init([&](int m) { return aq + (size_t)(row0 + min(m, mc - 1)) * pb; },
              [&](int m) { return aqs + (size_t)(row0 + min(m, mc - 1)) * (I / 32); });
      const size_t wrow0 = (size_t)t.m.e * a.d + t.n0;
      const uint8_t* w8 = a.w8;
      const uint8_t* ws = a.ws;
      lb.init([&](int n) { return w8 + (wrow0 + n) * pb; },
              [&](int n) { return ws + (wrow0 + n) * (I / 32); });
    }
    MOE_DEV void load(int kt) {  // weights first: they are the HBM stream
      lb.load(kt);
      la.load(kt);
    }
  };
  static MOE_DEV void epilogue(const Args& a, const Tile& t, f32x4 (&acc)[G::MB][G::NB],
                               uint8_t*) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int wm = wave / G::WAVES_N, wn = wave % G::WAVES_N;
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb) {
      const int m = wm * G::WM + mb * 16 + lane % 16;
      if (m >= t.m.mcount) continue;
      const size_t pos = t.m.row0 + m;
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb) {
        const int n = t.n0 + wn * G::WN + nb * 16 + 4 * (lane / 16);
        uint2 o;
        o.x = pack_bf2(acc[mb][nb][0], acc[mb][nb][1]);
        o.y = pack_bf2(acc[mb][nb][2], acc[mb][nb][3]);
        *reinterpret_cast<uint2*>(a.O + pos * a.d + n) = o;
      }
    }
  }
};
template <int F, bool GS>
using MxFwdDownS = MxFwdDownT<GeoMx<128, 128, 1, 4, F, GS>>;
template <int F>
using MxFwdDownBig = MxFwdDownT<GeoMxBig<F>>;

// Problem 3 (MXFP8): down dgrad, dA'[pos] = dY[t] . W2[e] with dY and W2 quantised along d
// (W2 stored transposed, [E, I, d]). The epilogue is the BF16 one (router-weight-gradient
// partials, SwiGLU backward, dH in bf16) plus dH quantised along 2I: the wave's 32 consecutive
// I columns make one 32-block of the gate half and one of the up half.
template <class G_>
struct MxBwdDownDgradT {
  static constexpr const char* kName = "bwd_down_dgrad";
  using G = G_;
  struct Args {
    const uint8_t* dyq;      // [T, d]
    const uint8_t* dys;      // [T, d/32]
    const int32_t* row_src;  // [T*k]
    const float* topk_w;     // [T*k]
    const uint8_t* w8;       // [E, I, d]
    const uint8_t* ws;       // [E, I, d/32]
    const uint16_t* H;       // [T*k, 2I]
    const uint16_t* A;       // [T*k, I]
    uint16_t* dH;            // [T*k, 2I]
    float* dwpart;           // [T*k, I / BN]
    uint8_t* dhq;            // [T*k, 2I]
    uint8_t* dhs;            // [T*k, 2I/32]
    const int32_t* offsets;
    const int2* sched;
    int d, I, k;
  };
  struct Tile {
    MTile m;
    int n0;
  };
  static MOE_DEV int ntiles(const Args& a) { return a.sched[0].x * (a.I / G::BN); }
  static MOE_DEV Tile decode(const Args& a, int lt) {
    const int ntc = a.I / G::BN;
    Tile t;
    t.m = decode_mtile(a.sched, lt / ntc);
    t.n0 = (lt % ntc) * G::BN;
    return t;
  }
  static MOE_DEV int num_k(const Args& a, const Tile&) { return a.d / G::BK; }
  static MOE_DEV int k_first(const Tile&, int) { return 0; }
  static MOE_DEV bool m_active(const Tile& t, int m) { return m < t.m.mcount; }
  static MOE_DEV int brow(int wn, int nb) { return wn * G::WN + nb * 16; }
  struct Loader {
    LoadA8<G> la;
    LoadB8<G> lb;
    MOE_DEV void init(const Args& a, const Tile& t) {
      const int d = a.d, k = a.k, mc = t.m.mcount, row0 = t.m.row0;
      const uint8_t* dyq = a.dyq;
      const uint8_t* dys = a.dys;
      const int32_t* rs = a.row_src;
      const size_t pb = (size_t)d * G::F / 8;  // bytes of codes per row
      la.init([&](int m) { return dyq + (size_t)(rs[row0 + min(m, mc - 1)] / k) * pb; },
              [&](int m) { return dys + (size_t)(rs[row0 + min(m, mc - 1)] / k) * (d / 32); });
      const size_t wrow0 = (size_t)t.m.e * a.I + t.n0;
      const uint8_t* w8 = a.w8;
      const uint8_t* ws = a.ws;
      lb.init([&](int n) { return w8 + (wrow0 + n) * pb; },
              [&](int n) { return ws + (wrow0 + n) * (d / 32); });
    }
    MOE_DEV void load(int kt) {  // weights first: they are the HBM stream
      lb.load(kt);
      la.load(kt);
    }
  };
  static MOE_DEV void epilogue(const Args& a, const Tile& t, f32x4 (&acc)[G::MB][G::NB],
                               uint8_t* smem) {
    const int lane = threadIdx.x % kWave, wn = (threadIdx.x / kWave) % G::WAVES_N;
    float* red = reinterpret_cast<float*>(smem);  // [WAVES_N][BM]; LDS is free after the K loop
    const int I = a.I;
    const int c0 = t.n0 + wn * G::WN;  // this wave's 32 I columns: one 32-block
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb) {
      const int m = mb * 16 + lane % 16;
      const bool live = m < t.m.mcount;
      const size_t pos = t.m.row0 + m;
      float part = 0.f;
      float dgv[8], duv[8];
      const float w = live ? a.topk_w[a.row_src[pos]] : 0.f;
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb) {
        const int i = c0 + nb * 16 + 4 * (lane / 16);
        uint2 av = make_uint2(0, 0), gv = make_uint2(0, 0), uv = make_uint2(0, 0);
        if (live) {
          av = *reinterpret_cast<const uint2*>(a.A + pos * I + i);
          gv = *reinterpret_cast<const uint2*>(a.H + pos * 2 * I + i);
          uv = *reinterpret_cast<const uint2*>(a.H + pos * 2 * I + I + i);
        }
        const float av4[4] = {bf2f_lo(av.x), bf2f_hi(av.x), bf2f_lo(av.y), bf2f_hi(av.y)};
        const float g4[4] = {bf2f_lo(gv.x), bf2f_hi(gv.x), bf2f_lo(gv.y), bf2f_hi(gv.y)};
        const float u4[4] = {bf2f_lo(uv.x), bf2f_hi(uv.x), bf2f_lo(uv.y), bf2f_hi(uv.y)};
        float dg[4], du[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float dap = acc[mb][nb][r];
          part = __builtin_fmaf(dap, av4[r], part);
          const float dA = w * dap;
          const float s = sigmoid(g4[r]);
          dg[r] = dA * u4[r] * s * (1.0f + g4[r] * (1.0f - s));
          du[r] = dA * (g4[r] * s);
        }
        uint2 og, ou;
        og.x = pack_bf2(dg[0], dg[1]);
        og.y = pack_bf2(dg[2], dg[3]);
        ou.x = pack_bf2(du[0], du[1]);
        ou.y = pack_bf2(du[2], du[3]);
        dgv[4 * nb + 0] = bf2f_lo(og.x);
        dgv[4 * nb + 1] = bf2f_hi(og.x);
        dgv[4 * nb + 2] = bf2f_lo(og.y);
        dgv[4 * nb + 3] = bf2f_hi(og.y);
        duv[4 * nb + 0] = bf2f_lo(ou.x);
        duv[4 * nb + 1] = bf2f_hi(ou.x);
        duv[4 * nb + 2] = bf2f_lo(ou.y);
        duv[4 * nb + 3] = bf2f_hi(ou.y);
        if (live) {
          *reinterpret_cast<uint2*>(a.dH + pos * 2 * I + i) = og;
          *reinterpret_cast<uint2*>(a.dH + pos * 2 * I + I + i) = ou;
        }
      }
      const uint32_t cg = mx_block_code<G::F>(dgv), cu = mx_block_code<G::F>(duv);
      const float ig = mx_inv_scale(cg), iu = mx_inv_scale(cu);
      if (live) {
        uint8_t* q = a.dhq + pos * (2 * I * G::F / 8);
        const int o = 4 * (lane / 16);
        mx_put4<G::F>(q, c0 + o, mx_pack4<G::F>(dgv, ig));
        mx_put4<G::F>(q, c0 + 16 + o, mx_pack4<G::F>(dgv + 4, ig));
        mx_put4<G::F>(q, I + c0 + o, mx_pack4<G::F>(duv, iu));
        mx_put4<G::F>(q, I + c0 + 16 + o, mx_pack4<G::F>(duv + 4, iu));
        if (lane < 16) {
          a.dhs[pos * (2 * I / 32) + c0 / 32] = static_cast<uint8_t>(cg);
          a.dhs[pos * (2 * I / 32) + (I + c0) / 32] = static_cast<uint8_t>(cu);
        }
      }
      // lanes l, l^16, l^32, l^48 share row m: butterfly in a fixed pattern
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      if (lane < 16) red[wn * G::BM + m] = part;
    }
    __syncthreads();
    if (threadIdx.x < G::BM && threadIdx.x < t.m.mcount) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < G::WAVES_N; ++w) s += red[w * G::BM + threadIdx.x];
      const size_t pos = t.m.row0 + threadIdx.x;
      a.dwpart[pos * (a.I / G::BN) + t.n0 / G::BN] = s;
    }
  }
};

template <int F, bool GS>
using MxBwdDownDgradS = MxBwdDownDgradT<GeoMx<128, 128, 1, 4, F, GS>>;

// Problem 4 (MXFP8): gate/up dgrad, dXp[pos] = dH[pos] . W1[e] with dH and W1 quantised along
// 2I (W1 stored transposed, [E, d, 2I]).
template <class G_>
struct MxBwdGateDgradT {
  static constexpr const char* kName = "bwd_gate_dgrad";
  using G = G_;
  struct Args {
    const uint8_t* dhq;  // [T*k, 2I]
    const uint8_t* dhs;  // [T*k, 2I/32]
    const uint8_t* w8;   // [E, d, 2I]
    const uint8_t* ws;   // [E, d, 2I/32]
    uint16_t* dXp;       // [T*k, d]
    const int32_t* offsets;
    const int2* sched;
    int d, I;
  };
  struct Tile {
    MTile m;
    int n0;
  };
  static MOE_DEV int ntiles(const Args& a) { return a.sched[0].x * (a.d / G::BN); }
  static MOE_DEV Tile decode(const Args& a, int lt) {
    const int ntc = a.d / G::BN;
    const int2 mn = tile_mn<(G::BM > 128)>(lt, a.sched[0].x, ntc);
    Tile t;
    t.m = decode_mtile(a.sched, mn.x);
    t.n0 = mn.y * G::BN;
    return t;
  }
  static MOE_DEV int num_k(const Args& a, const Tile&) { return 2 * a.I / G::BK; }
  static MOE_DEV int k_first(const Tile&, int) { return 0; }
  static MOE_DEV bool m_active(const Tile& t, int m) { return m < t.m.mcount; }
  static MOE_DEV int brow(int wn, int nb) { return wn * G::WN + nb * 16; }
  struct Loader {
    LoadA8<G> la;
    LoadB8<G> lb;
    MOE_DEV void init(const Args& a, const Tile& t) {
      const int twoI = 2 * a.I, mc = t.m.mcount, row0 = t.m.row0;
      const uint8_t* dhq = a.dhq;
      const uint8_t* dhs = a.dhs;
      const size_t pb = (size_t)twoI * G::F / 8;  // bytes of codes per row
      la.init([&](int m) { return dhq + (size_t)(row0 + min(m, mc - 1)) * pb; },
              [&](int m) { return dhs + (size_t)(row0 + min(m, mc - 1)) * (twoI / 32); });
      const size_t wrow0 = (size_t)t.m.e * a.d + t.n0;
      const uint8_t* w8 = a.w8;
      const uint8_t* ws = a.ws;
      lb.init([&](int n) { return w8 + (wrow0 + n) * pb; },
              [&](int n) { return ws + (wrow0 + n) * (twoI / 32); });
    }
    MOE_DEV void load(int kt) {  // weights first: they are the HBM stream
      lb.load(kt);
      la.load(kt);
    }
  };
  static MOE_DEV void epilogue(const Args& a, const Tile& t, f32x4 (&acc)[G::MB][G::NB],
                               uint8_t*) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int wm = wave / G::WAVES_N, wn = wave % G::WAVES_N;
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb) {
      const int m = wm * G::WM + mb * 16 + lane % 16;
      if (m >= t.m.mcount) continue;
      const size_t pos = t.m.row0 + m;
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb) {
        const int n = t.n0 + wn * G::WN + nb * 16 + 4 * (lane / 16);
        uint2 o;
        o.x = pack_bf2(acc[mb][nb][0], acc[mb][nb][1]);
        o.y = pack_bf2(acc[mb][nb][2], acc[mb][nb][3]);
        *reinterpret_cast<uint2*>(a.dXp + pos * a.d + n) = o;
      }
    }
  }
};
template <int F, bool GS>
using MxBwdGateDgradS = MxBwdGateDgradT<GeoMx<128, 128, 1, 4, F, GS>>;
template <int F>
using MxBwdGateDgradBig = MxBwdGateDgradT<GeoMxBig<F>>;

// MXFP8 weight gradients: dW[e][m][n] = sum over the expert's padded positions p of
// lq[m][poff[e] + p] rq[n][poff[e] + p], both operands quantised along the positions (mx.hip,
// quant_seg_kernel; codes past the count are zero). A 128 x 128 tile of one expert's dW per
// workgroup; its K loop walks the expert's 128-position chunks in order. An expert with no
// rows has no chunks: its tile is written as zeros (overwrite) or left as it is (accumulate).
// BF: dW is stored as bf16.
template <bool ACC, bool BF>
struct MxWgrad {
  static constexpr const char* kName = "bwd_wgrad_mx";
  using G = GeoMx<128, 128, 1, 4, 8, false>;  // a K step's scale words load one step at a time
  struct Args {
    const uint8_t* lq;
    const uint8_t* lqs;
    const uint8_t* rq;
    const uint8_t* rqs;
    void* dw;
    const int32_t* poff;
    int E, Mdim, Ndim, P;
  };
  struct Tile {
    int e, m0, n0;
  };
  // gg_kernel gives XCD x the tile range [x R, (x + 1) R), R = ntiles / 8. Expert by expert,
  // one XCD would hold one expert's tiles, and an expert with most of the rows would run on an
  // eighth of the GPU. So tile lt is the (lt % R)-th tile of slot lt / R in an order that deals
  // every expert's tiles round robin over the eight XCDs. The count is rounded up to a multiple
  // of 8; the surplus tiles have no expert (e = -1) and do nothing.
  static MOE_DEV int real_tiles(const Args& a) { return a.E * (a.Mdim / G::BM) * (a.Ndim / G::BN); }
  static MOE_DEV int ntiles(const Args& a) { return (real_tiles(a) + kXcds - 1) / kXcds * kXcds; }
  static MOE_DEV Tile decode(const Args& a, int lt) {
    const int R = ntiles(a) / kXcds;
    const int v = (lt % R) * kXcds + lt / R;
    if (v >= real_tiles(a)) return Tile{-1, 0, 0};
    const int nm = a.Mdim / G::BM, nn = a.Ndim / G::BN;
    const int2 mn = tile_mn<true>(v % (nm * nn), nm, nn);
    return Tile{v / (nm * nn), mn.x * G::BM, mn.y * G::BN};
  }
  static MOE_DEV int num_k(const Args& a, const Tile& t) {
    return t.e < 0 ? 0 : (a.poff[t.e + 1] - a.poff[t.e]) / G::BK;
  }
  static MOE_DEV int k_first(const Tile&, int) { return 0; }
  static MOE_DEV bool m_active(const Tile&, int) { return true; }
  static MOE_DEV int brow(int wn, int nb) { return wn * G::WN + nb * 16; }
  struct Loader {
    LoadA8<G> la;
    LoadB8<G> lb;
    MOE_DEV void init(const Args& a, const Tile& t) {
      const size_t P = a.P, p0 = a.poff[t.e];
      const uint8_t* lq = a.lq;
      const uint8_t* lqs = a.lqs;
      const uint8_t* rq = a.rq;
      const uint8_t* rqs = a.rqs;
      const int m0 = t.m0, n0 = t.n0;
      // the scale words are 4-byte aligned: P and p0 are multiples of 128
      la.init([&](int m) { return lq + (m0 + m) * P + p0; },
              [&](int m) { return lqs + (m0 + m) * (P / 32) + p0 / 32; });
      lb.init([&](int n) { return rq + (n0 + n) * P + p0; },
              [&](int n) { return rqs + (n0 + n) * (P / 32) + p0 / 32; });
    }
    MOE_DEV void load(int kt) {
      la.load(kt);
      lb.load(kt);
    }
  };
  static MOE_DEV void epilogue(const Args& a, const Tile& t, f32x4 (&acc)[G::MB][G::NB],
                               uint8_t*) {
    if (t.e < 0 || (ACC && a.poff[t.e + 1] == a.poff[t.e])) return;  // nothing to write / add
    const int lane = threadIdx.x % kWave, wn = (threadIdx.x / kWave) % G::WAVES_N;
    const size_t rstep = (size_t)16 * a.Ndim;
    if constexpr (BF) {
      // lane's row at the wave's first column; pairs of column blocks share 64-byte row pieces
      uint16_t* row = static_cast<uint16_t*>(a.dw) +
                      ((size_t)t.e * a.Mdim + t.m0 + lane % 16) * a.Ndim + t.n0 + wn * G::WN;
#pragma unroll
      for (int mb = 0; mb < G::MB; ++mb) {
#pragma unroll
        for (int nb = 0; nb < G::NB; nb += 2)
          store_dw8_bf16<ACC>(row + mb * rstep + nb * 16, acc[mb][nb], acc[mb][nb + 1], lane);
      }
    } else {
      // lane's first element; row block mb adds 16 rows, column block nb 16 columns
      float* out = static_cast<float*>(a.dw) +
                   ((size_t)t.e * a.Mdim + t.m0 + lane % 16) * a.Ndim + t.n0 + wn * G::WN +
                   4 * (lane / 16);
#pragma unroll
      for (int mb = 0; mb < G::MB; ++mb) {
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb)
          store_dw4<ACC>(out + mb * rstep + nb * 16, acc[mb][nb]);
      }
    }
  }
};

// ------------------------------------------------------------------------------------------
// The kernel: walks logical tiles. Each XCD owns one contiguous range of them (so the
// workgroups sharing an expert's activations share that XCD's L2), striding by the grid within
// the range. One-shot launches size the grid to cover every tile once; persistent launches
// use a resident grid that loops.


template <class P>
__global__ void __launch_bounds__(P::G::THREADS, P::G::kWavesPerEU) gg_kernel(const typename P::Args a) {
  extern __shared__ __align__(16) uint16_t smem[];
  const int ntiles = P::ntiles(a);
  const int R = (ntiles + kXcds - 1) / kXcds;
  const int b = blockIdx.x, step = gridDim.x / kXcds;
  for (int s = b / kXcds; s < R; s += step) {
    const int lt = (b % kXcds) * R + s;
    if (lt >= ntiles) break;
    const typename P::Tile t = P::decode(a, lt);
    if constexpr (P::G::kMx)
      run_tile_mx<P>(a, t, reinterpret_cast<uint8_t*>(smem));
    else
      run_tile<P>(a, t, smem);
  }
}

template <class P>
static size_t smem_bytes() {
  return P::G::kSmem;
}

// Grid: one-shot grids cover `max_tiles` (rounded up to a multiple of 8); persistent grids
// are the resident workgroup count, also a multiple of 8.
template <class P>
static hipError_t launch_named(const typename P::Args& a, int max_tiles, bool persistent,
                               const char* name, hipStream_t stream);
template <class P>
static hipError_t launch(const typename P::Args& a, int max_tiles, bool persistent,
                         hipStream_t stream) {
  return launch_named<P>(a, max_tiles, persistent, P::kName, stream);
}
template <class P>
static hipError_t launch_named(const typename P::Args& a, int max_tiles, bool persistent,
                               const char* name, hipStream_t stream) {
  if (max_tiles <= 0) return hipSuccess;
  const size_t sm = smem_bytes<P>();
  static bool attr_set = false;  // benign race: every caller sets the same value
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gg_kernel<P>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  int grid = (max_tiles + kXcds - 1) / kXcds * kXcds;
  if (persistent) {
    static int resident = 0;  // per kernel; every device of one process is an MI355X
    if (resident == 0) {
      int dev = 0, cus = 0, per_cu = 0;
      hipError_t e = hipGetDevice(&dev);
      if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
      if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(&gg_kernel<P>), P::G::THREADS, sm);
      if (e != hipSuccess) return e;
      resident = (cus * (per_cu > 0 ? per_cu : 1)) / kXcds * kXcds;
    }
    if (resident > 0 && resident < grid) grid = resident;
  }
  {
    TraceScope trace(name, stream);
    hipLaunchKernelGGL(gg_kernel<P>, dim3(grid), dim3(P::G::THREADS), sm, stream, a);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Full 256-row blocks of the four products on dma_kernel (dma.h): one trait per product.

// Problem 1's full blocks: rows of xp (pitch d) against W1[e]'s gate rows n0.. and up rows
// I + n0.. (pitch d), in the LDS row order of Problem 1's B tile.
struct DmaGateUp {
  using P = FwdGateUpBig;
  using Args = P::Args;
  using Tile = P::Tile;
  static constexpr const char* kName = "fwd_gateup_big";
  static constexpr bool kAKmajor = false, kBKmajor = false;
  static constexpr bool kVoffStep = false, kRoundOrder = false;
  static MOE_DEV int ntiles(const Args& a) { return P::ntiles(a); }
  static MOE_DEV Tile decode(const Args& a, int lt) { return P::decode(a, lt); }
  static MOE_DEV int brow(int wn, int nb) { return P::brow(wn, nb); }
  static MOE_DEV void src(const Args& a, const Tile& t, int wave, int lane, DmaSrc& s) {
    const int d = a.d, I = a.I;
    s.nk = d / 64;
    s.k0 = 0;
    s.ra = raw_rsrc(a.xp + (size_t)t.m.row0 * d);
    s.rb = raw_rsrc(a.w1 + (size_t)t.m.e * 2 * I * d);
    s.astep = s.bstep = 128;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = dma_row(wave, j, lane);
      const int wrow = row < 128 ? t.n0 + row : I + t.n0 + row - 128;
      // rows past the expert's count (none, on full blocks) would repeat its last row
      s.ao[j] = 2u * (uint32_t)min(row, t.m.mcount - 1) * d + dma_piece(lane);
      s.bo[j] = 2u * (uint32_t)wrow * d + dma_piece(lane);
    }
  }
  static MOE_DEV void epilogue(const Args& a, const Tile& t, f32x4 (&acc)[8][4]) {
    P::epilogue(a, t, acc, nullptr);
  }
};

// Problem 2's full blocks: rows of A (pitch I) against W2[e]'s rows n0.. (pitch I). W2's rows
// are 2I bytes apart, so each n-tile starts at its own K chunk, as in Problem 2.
struct DmaDown {
  using P = FwdDownBig;
  using Args = P::Args;
  using Tile = P::Tile;
  static constexpr const char* kName = "fwd_down_big";
  static constexpr bool kAKmajor = false, kBKmajor = false;
  static constexpr bool kVoffStep = false, kRoundOrder = false;
  static MOE_DEV int ntiles(const Args& a) { return P::ntiles(a); }
  static MOE_DEV Tile decode(const Args& a, int lt) { return P::decode(a, lt); }
  static MOE_DEV int brow(int wn, int nb) { return P::brow(wn, nb); }
  static MOE_DEV void src(const Args& a, const Tile& t, int wave, int lane, DmaSrc& s) {
    const int I = a.I;
    s.nk = I / 64;
    s.k0 = P::k_first(t, s.nk);
    s.ra = raw_rsrc(a.A + (size_t)t.m.row0 * I);
    s.rb = raw_rsrc(a.w2 + ((size_t)t.m.e * a.d + t.n0) * I);
    s.astep = s.bstep = 128;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = dma_row(wave, j, lane);
      s.ao[j] = 2u * (uint32_t)min(row, t.m.mcount - 1) * I + dma_piece(lane);
      s.bo[j] = 2u * (uint32_t)row * I + dma_piece(lane);
    }
  }
  static MOE_DEV void epilogue(const Args& a, const Tile& t, f32x4 (&acc)[8][4]) {
    P::epilogue(a, t, acc, nullptr);
  }
};

struct DgradTile {
  MTile m;
  int n0;
};

// Problem 4's full blocks: dXp = dH . W1[e]. dH rows (pitch 2I) are K-contiguous; W1[e]
// ([2I, d], d-contiguous) is K-major, 256 columns from n0.
struct DmaGateDgrad {
  using Args = GateDgradBigArgs;
  using Tile = DgradTile;
  static constexpr const char* kName = "bwd_gate_dgrad_big";
  static constexpr bool kAKmajor = false, kBKmajor = true;
  static constexpr bool kVoffStep = false, kRoundOrder = false;
  static MOE_DEV int ntiles(const Args& a) { return a.big[0].x * (a.d / 256); }
  static MOE_DEV Tile decode(const Args& a, int lt) {
    const int2 mn = tile_mn<true>(lt, a.big[0].x, a.d / 256);
    return Tile{decode_mtile(a.big, mn.x), mn.y * 256};
  }
  static MOE_DEV int brow(int, int) { return 0; }
  static MOE_DEV void src(const Args& a, const Tile& t, int wave, int lane, DmaSrc& s) {
    const int twoI = 2 * a.I, d = a.d;
    s.nk = twoI / 64;
    s.k0 = 0;
    s.ra = raw_rsrc(a.dH + (size_t)t.m.row0 * twoI);
    s.rb = raw_rsrc(a.w1 + (size_t)t.m.e * twoI * d + t.n0);
    s.astep = 128;
    s.bstep = 128u * (uint32_t)d;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = dma_row(wave, j, lane), kr = dma_krow(wave, j, lane);
      s.ao[j] = 2u * (uint32_t)min(row, t.m.mcount - 1) * twoI + dma_piece(lane);
      s.bo[j] = 2u * (uint32_t)kr * d + dma_kpiece(kr, lane);
    }
  }
  static MOE_DEV void epilogue(const Args& a, const Tile& t, f32x4 (&acc)[8][4]) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int wm = wave / 4, wn = wave % 4;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const size_t pos = t.m.row0 + wm * 128 + mb * 16 + lane % 16;
      uint16_t* orow = a.dXp + pos * a.d + t.n0 + wn * 64 + 4 * (lane / 16);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        uint2 o;
        o.x = pack_bf2(acc[mb][nb][0], acc[mb][nb][1]);
        o.y = pack_bf2(acc[mb][nb][2], acc[mb][nb][3]);
        *reinterpret_cast<uint2*>(orow + nb * 16) = o;
      }
    }
  }
};

// Problem 3's full blocks: dA' = dY[t] . W2[e] with dY rows (pitch d) gathered through row_src
// and W2[e] ([d, I], I-contiguous) K-major, 256 columns from n0. The epilogue is Problem 3's:
// per (pos, i) the SwiGLU backward into dH, and the router-weight partials
// dw = sum_i dA'[pos, i] A[pos, i] of each 128-column half, summed in a fixed order (a lane's
// columns, then its lane groups, then the two waves of the half).
struct DmaDownDgrad {
  using Args = DownDgradBigArgs;
  using Tile = DgradTile;
  static constexpr const char* kName = "bwd_down_dgrad_big";
  static constexpr bool kAKmajor = false, kBKmajor = true;
  static constexpr bool kVoffStep = false, kRoundOrder = false;
  static MOE_DEV int ntiles(const Args& a) { return a.big[0].x * (a.I / 256); }
  static MOE_DEV Tile decode(const Args& a, int lt) {
    const int2 mn = tile_mn<true>(lt, a.big[0].x, a.I / 256);
    return Tile{decode_mtile(a.big, mn.x), mn.y * 256};
  }
  static MOE_DEV int brow(int, int) { return 0; }
  static MOE_DEV void src(const Args& a, const Tile& t, int wave, int lane, DmaSrc& s) {
    const int d = a.d, I = a.I;
    s.nk = d / 64;
    s.k0 = 0;
    s.ra = raw_rsrc(a.dy);  // byte offsets into dY fit 32 bits: T d < 2^31 is an API limit
    s.rb = raw_rsrc(a.w2 + (size_t)t.m.e * d * I + t.n0);
    s.astep = 128;
    s.bstep = 128u * (uint32_t)I;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = dma_row(wave, j, lane), kr = dma_krow(wave, j, lane);
      const int tok = a.row_src[t.m.row0 + min(row, t.m.mcount - 1)] / a.k;
      s.ao[j] = 2u * (uint32_t)tok * d + dma_piece(lane);
      s.bo[j] = 2u * (uint32_t)kr * I + dma_kpiece(kr, lane);
    }
  }
  static MOE_DEV void epilogue(const Args& a, const Tile& t, f32x4 (&acc)[8][4]) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int wm = wave / 4, wn = wave % 4;
    const int I = a.I;
    float* red = reinterpret_cast<float*>(dma_a0);  // [4][256] row sums per wave column
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const int m = wm * 128 + mb * 16 + lane % 16;
      const size_t pos = t.m.row0 + m;
      const float w = a.topk_w[a.row_src[pos]];
      float part = 0.f;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int i = t.n0 + wn * 64 + nb * 16 + 4 * (lane / 16);
        const uint2 av = *reinterpret_cast<const uint2*>(a.A + pos * I + i);
        const uint2 gv = *reinterpret_cast<const uint2*>(a.H + pos * 2 * I + i);
        const uint2 uv = *reinterpret_cast<const uint2*>(a.H + pos * 2 * I + I + i);
        const float av4[4] = {bf2f_lo(av.x), bf2f_hi(av.x), bf2f_lo(av.y), bf2f_hi(av.y)};
        const float g4[4] = {bf2f_lo(gv.x), bf2f_hi(gv.x), bf2f_lo(gv.y), bf2f_hi(gv.y)};
        const float u4[4] = {bf2f_lo(uv.x), bf2f_hi(uv.x), bf2f_lo(uv.y), bf2f_hi(uv.y)};
        float dg[4], du[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float dap = acc[mb][nb][r];
          part = __builtin_fmaf(dap, av4[r], part);
          const float dA = w * dap;
          const float sg = sigmoid(g4[r]);
          dg[r] = dA * u4[r] * sg * (1.0f + g4[r] * (1.0f - sg));
          du[r] = dA * (g4[r] * sg);
        }
        uint2 o;
        o.x = pack_bf2(dg[0], dg[1]);
        o.y = pack_bf2(dg[2], dg[3]);
        *reinterpret_cast<uint2*>(a.dH + pos * 2 * I + i) = o;
        o.x = pack_bf2(du[0], du[1]);
        o.y = pack_bf2(du[2], du[3]);
        *reinterpret_cast<uint2*>(a.dH + pos * 2 * I + I + i) = o;
      }
      // lanes l, l^16, l^32, l^48 share row m: butterfly in a fixed pattern
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      if (lane < 16) red[wn * 256 + m] = part;
    }
    __syncthreads();
    if (threadIdx.x < 256) {
      const size_t pos = t.m.row0 + threadIdx.x;
      float* dst = a.dwpart + pos * (I / 128) + t.n0 / 128;
      dst[0] = red[0 * 256 + threadIdx.x] + red[1 * 256 + threadIdx.x];  // [n0, n0 + 128)
      dst[1] = red[2 * 256 + threadIdx.x] + red[3 * 256 + threadIdx.x];  // [n0 + 128, n0 + 256)
    }
    __syncthreads();  // red is the next tile's first token-row stage
  }
};


// ------------------------------------------------------------------------------------------
// MXFP8 products on full 256-row blocks: 256 x 256 tiles of eight 128 x 64 wave tiles fed by
// direct global -> LDS loads, as dma_kernel does for BF16. A 128-deep K step of fp8 codes is
// one 128-byte line per row, the bytes of a 64-deep bf16 step, so the code stages keep
// dma_kernel's row layout (mxswz is rowswz in bytes) and load mapping, and the fragments and
// scaled MFMAs are run_tile_mx's. Each stage also holds the step's scale word of every row (4
// bytes a row, 1 KB an operand), moved by one 4-byte load per lane: waves 0-3 load A's, waves
// 4-7 B's. Two stages of 66 KB fit: each step waits for its own loads, then refills the other
// stage for the next step, so loads have one step of MFMAs to arrive. The two stages are
// distinct LDS arrays and the loop is unrolled over both, so the compiler can tell the stage a
// load writes from the one the fragment reads read.
// E2M1 steps (256 K in the same 128 bytes a row) carry two scale words a row: word 0 of every A
// and B row, then word 1 of every row, each moved by one 4-byte load per lane.
constexpr int kDmxCodes = 256 * 128;   // bytes of one operand's codes
constexpr int kDmxWords = 2 * 256 * 4;  // one scale word of every A and B row
constexpr int kDmxStage = 2 * kDmxCodes + 2 * kDmxWords;  // A, B codes, then the scale words
__shared__ __align__(1024) uint8_t dmx_s0[kDmxStage];
__shared__ __align__(1024) uint8_t dmx_s1[kDmxStage];
template <int S>
MOE_DEV uint8_t* dmx_stage() {
  if constexpr (S == 0) return dmx_s0;
  else return dmx_s1;
}

// A lane's sources for one tile: code resources, the byte offsets of its four A pieces (rows
// may be gathered) and of its first B piece (its load j fetches B rows 8 j further on, bst bytes
// on, the same in every lane), and the resource and offset of the scale word it moves (its
// wave's operand, row 64 (wave % 4) + lane). K chunks run k0, k0 + 1, .., nk - 1, 0, .., k0 - 1.
struct DmxSrc {
  __amdgpu_buffer_rsrc_t ra, rb, rs;
  uint32_t ao[4], bo, so, bst;
  int k0, nk;
};

MOE_DEV void dmx16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint8_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, soff, 0, 0);
}
MOE_DEV void dmx4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint8_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4,
                                           voff, soff, 0, 0);
}

// K chunk kt of the tile (clamped to the last) into stage S: nine load instructions a wave (ten
// for E2M1 codes, F = 4).
template <int S, int F>
MOE_DEV void dmx_issue(const DmxSrc& s, int kt, int wave) {
  int kk = min(kt, s.nk - 1) + s.k0;
  kk = kk >= s.nk ? kk - s.nk : kk;
  uint8_t* st = dmx_stage<S>();
  const uint32_t step = (uint32_t)kk * 128;
#pragma unroll
  for (int j = 0; j < 4; ++j) dmx16(s.ra, s.ao[j], step, st + wave * 4096 + j * 1024);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    dmx16(s.rb, s.bo, step + j * s.bst, st + kDmxCodes + wave * 4096 + j * 1024);
  constexpr uint32_t SB = F == 8 ? 4 : 8;  // scale bytes a row per step
  dmx4(s.rs, s.so, (uint32_t)kk * SB, st + 2 * kDmxCodes + wave * 256);
  if constexpr (F == 4)
    dmx4(s.rs, s.so, (uint32_t)kk * SB + 4, st + 2 * kDmxCodes + kDmxWords + wave * 256);
}

// The scale bytes lane group g passes for LDS scale row q (A rows 0..255, B rows 256..511):
// byte g of word 0 and (E2M1) of word 1.
template <int F>
MOE_DEV int2 dmx_scales(const uint32_t* sc, int q, int g) {
  const int x = static_cast<int>((sc[q] >> (8 * g)) & 0xffu);
  if constexpr (F == 8) return make_int2(x, 0);
  else return make_int2(x, static_cast<int>((sc[512 + q] >> (8 * g)) & 0xffu));
}

template <class D, int S>
MOE_DEV void dmx_step(f32x4 (&acc)[8][4], const DmxSrc& s, int kt, int wave, int wm, int wn,
                      int lane) {
  constexpr int F = D::F;
  __builtin_amdgcn_s_waitcnt(kWaitVm0Lgkm0);
  __builtin_amdgcn_s_barrier();
  dmx_issue<S ^ 1, F>(s, kt + 1, wave);
  __builtin_amdgcn_sched_barrier(0);
  const uint8_t* st = dmx_stage<S>();
  const uint8_t* sA = st;
  const uint8_t* sB = st + kDmxCodes;
  const uint32_t* sc = reinterpret_cast<const uint32_t*>(st + 2 * kDmxCodes);
  // the lane's fragment addresses are recomputed in every step (a few adds) rather than held
  // across the loop, where the accumulators and fragments leave no register for them
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const int r16 = ln % 16, g = ln / 16;
  i32x8 bf[4];
  int2 bs[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int row = D::brow(wn, nb) + r16;
    bf[nb] = mx_frag(sB, row, g);
    bs[nb] = dmx_scales<F>(sc, 256 + row, g);
  }
  // row block mb + 1's A fragment is read while row block mb's MFMAs run
  const int row0 = wm * 128 + r16;
  i32x8 af = mx_frag(sA, row0, g);
  int2 as = dmx_scales<F>(sc, row0, g);
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    i32x8 an = af;
    int2 asn = as;
    if (mb + 1 < 8) {
      const int row = row0 + (mb + 1) * 16;
      an = mx_frag(sA, row, g);
      asn = dmx_scales<F>(sc, row, g);
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mx_mfma<F>(bf[nb], af, acc[mb][nb], bs[nb], as);
    af = an;
    as = asn;
  }
}

// The tile walk of dma_kernel (XCD x takes the contiguous tile range [x R, (x + 1) R)).
template <class D>
__global__ void __launch_bounds__(512, 2) dmx_kernel(const typename D::Args a) {
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wm = wave / 4, wn = wave % 4;
  const int ntiles = D::ntiles(a);
  const int R = (ntiles + kXcds - 1) / kXcds;
  const int G8 = gridDim.x / kXcds, xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  for (int it = 0;; ++it) {
    const int sidx = slot + it * G8;
    if (sidx >= R) break;
    const int lt = xcd * R + sidx;
    if (lt >= ntiles) break;
    const typename D::Tile t = D::decode(a, lt);
    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    DmxSrc s;
    D::src(a, t, wave, lane, s);
    if (s.nk > 0) {
      dmx_issue<0, D::F>(s, 0, wave);
      for (int kt = 0;; kt += 2) {
        dmx_step<D, 0>(acc, s, kt, wave, wm, wn, lane);
        if (kt + 1 >= s.nk) break;
        dmx_step<D, 1>(acc, s, kt + 1, wave, wm, wn, lane);
        if (kt + 2 >= s.nk) break;
      }
      // the trailing reload has landed and no wave still reads a stage
      __builtin_amdgcn_s_waitcnt(kWaitVm0Lgkm0);
      __builtin_amdgcn_s_barrier();
    }
    // The tile as the epilogue sees it, passed through an empty asm statement: the compiler
    // cannot compute the epilogue's addresses before the K loop and hold them across it, where
    // the accumulators and fragments already fill the register file.
    typename D::Tile te = t;  // wave-uniform fields
    te.m.e = __builtin_amdgcn_readfirstlane(te.m.e);
    te.m.row0 = __builtin_amdgcn_readfirstlane(te.m.row0);
    te.m.mcount = __builtin_amdgcn_readfirstlane(te.m.mcount);
    te.n0 = __builtin_amdgcn_readfirstlane(te.n0);
    asm volatile("" : "+s"(te.m.e), "+s"(te.m.row0), "+s"(te.m.mcount), "+s"(te.n0));
    D::epilogue(a, te, acc);
  }
}

template <class D>
hipError_t launch_dmx(const typename D::Args& a, int max_tiles, bool persistent,
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
            &per_cu, reinterpret_cast<const void*>(&dmx_kernel<D>), 512, 0);
      if (e != hipSuccess) return e;
      resident = (cus * (per_cu > 0 ? per_cu : 1)) / kXcds * kXcds;
    }
    if (resident > 0 && resident < grid) grid = resident;
  }
  {
    TraceScope trace(D::kName, stream);
    hipLaunchKernelGGL(dmx_kernel<D>, dim3(grid), dim3(512), 0, stream, a);
  }
  return hipGetLastError();
}

// Problem 1 (MX) on full 256-row blocks: 256 token rows (Xp codes, pitch d F / 8 bytes) against
// 128 gate rows and the 128 matching up rows of W1[e]'s codes (same pitch). Byte offsets fit 32
// bits: an expert's W1 codes are below 2^31 bytes (4 I d < 2^31 is an API limit).
template <int F_>
struct DmxGateUp {
  static constexpr int F = F_;
  using P = MxFwdGateUpBig<F>;
  using Args = typename P::Args;
  using Tile = typename P::Tile;
  static constexpr const char* kName = "fwd_gateup_big";
  static MOE_DEV int ntiles(const Args& a) { return P::ntiles(a); }
  static MOE_DEV Tile decode(const Args& a, int lt) { return P::decode(a, lt); }
  static MOE_DEV int brow(int wn, int nb) { return P::brow(wn, nb); }
  static MOE_DEV void src(const Args& a, const Tile& t, int wave, int lane, DmxSrc& s) {
    const int d = a.d, I = a.I, kA = P::kA;
    const int pb = d * F / 8;  // bytes of codes per row
    auto wrow = [&](int r) { return r < kA ? t.n0 + r : I + t.n0 + r - kA; };
    s.nk = d / P::G::BK;
    s.k0 = 0;
    s.ra = raw_rsrc(a.xp8 + (size_t)t.m.row0 * pb);
    s.rb = raw_rsrc(a.w8 + (size_t)t.m.e * 2 * I * pb);
    // load j's rows are 8 j further on, in the same half of the B tile (gate or up)
    const int row = dma_row(wave, 0, lane);
#pragma unroll
    for (int j = 0; j < 4; ++j) s.ao[j] = (uint32_t)(row + 8 * j) * pb + dma_piece(lane);
    s.bo = (uint32_t)wrow(row) * pb + dma_piece(lane);
    s.bst = 8u * (uint32_t)pb;
    const int r = 64 * (wave % 4) + lane;
    if (wave < 4) {
      s.rs = raw_rsrc(a.xps + (size_t)t.m.row0 * (d / 32));
      s.so = (uint32_t)r * (d / 32);
    } else {
      s.rs = raw_rsrc(a.ws + (size_t)t.m.e * 2 * I * (d / 32));
      s.so = (uint32_t)wrow(r) * (d / 32);
    }
  }
  static MOE_DEV void epilogue(const Args& a, const Tile& t, f32x4 (&acc)[8][4]) {
    P::epilogue(a, t, acc, nullptr);
  }
};

// Problem 2 (MX) on full 256-row blocks: A codes (pitch I F / 8 bytes) against W2[e]'s codes,
// rows n0.. (same pitch); each n-tile starts at its own K chunk, as in the 128-row kernel.
template <int F_>
struct DmxDown {
  static constexpr int F = F_;
  using P = MxFwdDownBig<F>;
  using Args = typename P::Args;
  using Tile = typename P::Tile;
  static constexpr const char* kName = "fwd_down_big";
  static MOE_DEV int ntiles(const Args& a) { return P::ntiles(a); }
  static MOE_DEV Tile decode(const Args& a, int lt) { return P::decode(a, lt); }
  static MOE_DEV int brow(int wn, int nb) { return P::brow(wn, nb); }
  static MOE_DEV void src(const Args& a, const Tile& t, int wave, int lane, DmxSrc& s) {
    const int I = a.I, pb = I * F / 8;
    s.nk = I / P::G::BK;
    s.k0 = P::k_first(t, s.nk);
    s.ra = raw_rsrc(a.aq + (size_t)t.m.row0 * pb);
    s.rb = raw_rsrc(a.w8 + ((size_t)t.m.e * a.d + t.n0) * pb);
    const int row = dma_row(wave, 0, lane);
#pragma unroll
    for (int j = 0; j < 4; ++j) s.ao[j] = (uint32_t)(row + 8 * j) * pb + dma_piece(lane);
    s.bo = (uint32_t)row * pb + dma_piece(lane);
    s.bst = 8u * (uint32_t)pb;
    const int r = 64 * (wave % 4) + lane;
    s.rs = wave < 4 ? raw_rsrc(a.aqs + (size_t)t.m.row0 * (I / 32))
                    : raw_rsrc(a.ws + ((size_t)t.m.e * a.d + t.n0) * (I / 32));
    s.so = (uint32_t)r * (I / 32);
  }
  static MOE_DEV void epilogue(const Args& a, const Tile& t, f32x4 (&acc)[8][4]) {
    P::epilogue(a, t, acc, nullptr);
  }
};

// Problem 4 (MX) on full 256-row blocks: dH codes (pitch 2I F / 8 bytes) against W1[e]'s
// transposed codes ([d, 2I], rows n0..).
template <int F_>
struct DmxGateDgrad {
  static constexpr int F = F_;
  using P = MxBwdGateDgradBig<F>;
  using Args = typename P::Args;
  using Tile = typename P::Tile;
  static constexpr const char* kName = "bwd_gate_dgrad_big";
  static MOE_DEV int ntiles(const Args& a) { return P::ntiles(a); }
  static MOE_DEV Tile decode(const Args& a, int lt) { return P::decode(a, lt); }
  static MOE_DEV int brow(int wn, int nb) { return P::brow(wn, nb); }
  static MOE_DEV void src(const Args& a, const Tile& t, int wave, int lane, DmxSrc& s) {
    const int twoI = 2 * a.I, pb = twoI * F / 8;
    s.nk = twoI / P::G::BK;
    s.k0 = 0;
    s.ra = raw_rsrc(a.dhq + (size_t)t.m.row0 * pb);
    s.rb = raw_rsrc(a.w8 + ((size_t)t.m.e * a.d + t.n0) * pb);
    const int row = dma_row(wave, 0, lane);
#pragma unroll
    for (int j = 0; j < 4; ++j) s.ao[j] = (uint32_t)(row + 8 * j) * pb + dma_piece(lane);
    s.bo = (uint32_t)row * pb + dma_piece(lane);
    s.bst = 8u * (uint32_t)pb;
    const int r = 64 * (wave % 4) + lane;
    s.rs = wave < 4 ? raw_rsrc(a.dhs + (size_t)t.m.row0 * (twoI / 32))
                    : raw_rsrc(a.ws + ((size_t)t.m.e * a.d + t.n0) * (twoI / 32));
    s.so = (uint32_t)r * (twoI / 32);
  }
  static MOE_DEV void epilogue(const Args& a, const Tile& t, f32x4 (&acc)[8][4]) {
    P::epilogue(a, t, acc, nullptr);
  }
};

// Problem 3 (MXFP8) on full 256-row blocks: the gathered dY codes (token rows, pitch d) against
// W2[e]'s transposed codes ([I, d], rows n0..). The epilogue is the 128-row kernel's per 32-block
// of I columns (a wave's 64 columns are two), and the router-weight partials of each 128-column
// half are the sums of its two waves' row sums, as in the BF16 256 x 256 kernel.
template <int F_>
struct DmxDownDgrad {
  static constexpr int F = F_;
  using Args = typename MxBwdDownDgradS<F, true>::Args;
  using Tile = DgradTile;
  static constexpr const char* kName = "bwd_down_dgrad_big";
  static MOE_DEV int ntiles(const Args& a) { return a.sched[0].x * (a.I / 256); }
  static MOE_DEV Tile decode(const Args& a, int lt) {
    const int2 mn = tile_mn<true>(lt, a.sched[0].x, a.I / 256);
    return Tile{decode_mtile(a.sched, mn.x), mn.y * 256};
  }
  static MOE_DEV int brow(int wn, int nb) { return wn * 64 + nb * 16; }
  // byte offsets into dY's codes fit 32 bits: T d < 2^31 is an API limit
  static MOE_DEV void src(const Args& a, const Tile& t, int wave, int lane, DmxSrc& s) {
    const int d = a.d, pb = d * F / 8;
    s.nk = d / (1024 / F);
    s.k0 = 0;
    s.ra = raw_rsrc(a.dyq);
    s.rb = raw_rsrc(a.w8 + ((size_t)t.m.e * a.I + t.n0) * pb);
    const int row = dma_row(wave, 0, lane);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      s.ao[j] = (uint32_t)(a.row_src[t.m.row0 + row + 8 * j] / a.k) * pb + dma_piece(lane);
    s.bo = (uint32_t)row * pb + dma_piece(lane);
    s.bst = 8u * (uint32_t)pb;
    const int r = 64 * (wave % 4) + lane;
    if (wave < 4) {
      s.rs = raw_rsrc(a.dys);
      s.so = (uint32_t)(a.row_src[t.m.row0 + r] / a.k) * (d / 32);
    } else {
      s.rs = raw_rsrc(a.ws + ((size_t)t.m.e * a.I + t.n0) * (d / 32));
      s.so = (uint32_t)r * (d / 32);
    }
  }
  static MOE_DEV void epilogue(const Args& a, const Tile& t, f32x4 (&acc)[8][4]) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int wm = wave / 4, wn = wave % 4;
    const int I = a.I;
    float* red = reinterpret_cast<float*>(dmx_s0);  // [4][256] row sums per wave column
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const int m = wm * 128 + mb * 16 + lane % 16;
      const size_t pos = t.m.row0 + m;
      const float w = a.topk_w[a.row_src[pos]];
      float part = 0.f;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {  // the wave's two 32-blocks of I columns
        const int c0 = t.n0 + wn * 64 + hb * 32;
        float dgv[8], duv[8];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int nb = 2 * hb + q;
          const int i = c0 + q * 16 + 4 * (lane / 16);
          const uint2 av = *reinterpret_cast<const uint2*>(a.A + pos * I + i);
          const uint2 gv = *reinterpret_cast<const uint2*>(a.H + pos * 2 * I + i);
          const uint2 uv = *reinterpret_cast<const uint2*>(a.H + pos * 2 * I + I + i);
          const float av4[4] = {bf2f_lo(av.x), bf2f_hi(av.x), bf2f_lo(av.y), bf2f_hi(av.y)};
          const float g4[4] = {bf2f_lo(gv.x), bf2f_hi(gv.x), bf2f_lo(gv.y), bf2f_hi(gv.y)};
          const float u4[4] = {bf2f_lo(uv.x), bf2f_hi(uv.x), bf2f_lo(uv.y), bf2f_hi(uv.y)};
          float dg[4], du[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float dap = acc[mb][nb][r];
            part = __builtin_fmaf(dap, av4[r], part);
            const float dA = w * dap;
            const float sg = sigmoid(g4[r]);
            dg[r] = dA * u4[r] * sg * (1.0f + g4[r] * (1.0f - sg));
            du[r] = dA * (g4[r] * sg);
          }
          uint2 og, ou;
          og.x = pack_bf2(dg[0], dg[1]);
          og.y = pack_bf2(dg[2], dg[3]);
          ou.x = pack_bf2(du[0], du[1]);
          ou.y = pack_bf2(du[2], du[3]);
          dgv[4 * q + 0] = bf2f_lo(og.x);
          dgv[4 * q + 1] = bf2f_hi(og.x);
          dgv[4 * q + 2] = bf2f_lo(og.y);
          dgv[4 * q + 3] = bf2f_hi(og.y);
          duv[4 * q + 0] = bf2f_lo(ou.x);
          duv[4 * q + 1] = bf2f_hi(ou.x);
          duv[4 * q + 2] = bf2f_lo(ou.y);
          duv[4 * q + 3] = bf2f_hi(ou.y);
          *reinterpret_cast<uint2*>(a.dH + pos * 2 * I + i) = og;
          *reinterpret_cast<uint2*>(a.dH + pos * 2 * I + I + i) = ou;
        }
        const uint32_t cg = mx_block_code<F>(dgv), cu = mx_block_code<F>(duv);
        const float ig = mx_inv_scale(cg), iu = mx_inv_scale(cu);
        uint8_t* qp = a.dhq + pos * (2 * I * F / 8);
        const int o = 4 * (lane / 16);
        mx_put4<F>(qp, c0 + o, mx_pack4<F>(dgv, ig));
        mx_put4<F>(qp, c0 + 16 + o, mx_pack4<F>(dgv + 4, ig));
        mx_put4<F>(qp, I + c0 + o, mx_pack4<F>(duv, iu));
        mx_put4<F>(qp, I + c0 + 16 + o, mx_pack4<F>(duv + 4, iu));
        if (lane < 16) {
          a.dhs[pos * (2 * I / 32) + c0 / 32] = static_cast<uint8_t>(cg);
          a.dhs[pos * (2 * I / 32) + (I + c0) / 32] = static_cast<uint8_t>(cu);
        }
      }
      // lanes l, l^16, l^32, l^48 share row m: butterfly in a fixed pattern
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      if (lane < 16) red[wn * 256 + m] = part;
    }
    __syncthreads();
    if (threadIdx.x < 256) {
      const size_t pos = t.m.row0 + threadIdx.x;
      float* dst = a.dwpart + pos * (I / 128) + t.n0 / 128;
      dst[0] = red[0 * 256 + threadIdx.x] + red[1 * 256 + threadIdx.x];  // [n0, n0 + 128)
      dst[1] = red[2 * 256 + threadIdx.x] + red[3 * 256 + threadIdx.x];  // [n0 + 128, n0 + 256)
    }
    __syncthreads();  // red is the next tile's first stage
  }
};

// ------------------------------------------------------------------------------------------
// Schedule tables, built on the device from the offsets so the host never learns the counts.
// Entry 0 of each holds its count; entry i >= 1 is (expert, first row within the expert).
//  * full: every 128-row block of every expert;
//  * big:  every full 256-row block (the experts' first 256 * floor(c / 256) rows);
//  * rem:  the 128-row blocks of what the big blocks leave of each expert (at most two).
// Problems with a 256-row kernel run big + rem; the others run full.

MOE_DEV int block_scan_1024(int v, int* scan) {  // inclusive scan of one value per thread
  const int e = threadIdx.x;
  scan[e] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int u = e >= off ? scan[e - off] : 0;
    __syncthreads();
    scan[e] += u;
    __syncthreads();
  }
  const int r = scan[e];
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(1024) sched_build_kernel(const int32_t* offsets, int E,
                                                           int2* full, int2* big, int2* rem) {
  __shared__ int scan[1024];
  const int e = threadIdx.x;
  const int p0 = e < E ? offsets[e] : 0;
  const int c = e < E ? offsets[e + 1] - p0 : 0;
  const int nfull = (c + kSchedBM - 1) / kSchedBM;
  const int nbig = c / kSchedBigBM;
  const int nrem = (c - nbig * kSchedBigBM + kSchedBM - 1) / kSchedBM;
  const int efull = block_scan_1024(nfull, scan);
  const int ebig = block_scan_1024(nbig, scan);
  const int erem = block_scan_1024(nrem, scan);
  for (int i = 0; i < nfull; ++i)
    full[1 + efull - nfull + i] =
        mtile_entry(e, p0 + i * kSchedBM, min(kSchedBM, c - i * kSchedBM));
  for (int i = 0; i < nbig; ++i)
    big[1 + ebig - nbig + i] = mtile_entry(e, p0 + i * kSchedBigBM, kSchedBigBM);
  for (int i = 0; i < nrem; ++i) {
    const int r = nbig * kSchedBigBM + i * kSchedBM;
    rem[1 + erem - nrem + i] = mtile_entry(e, p0 + r, min(kSchedBM, c - r));
  }
  if (e == 1023) {
    full[0] = make_int2(efull, 0);
    big[0] = make_int2(ebig, 0);
    rem[0] = make_int2(erem, 0);
  }
}

int sched_max_mtiles(int Tk, int E) { return (Tk + E * (kSchedBM - 1)) / kSchedBM; }
int sched_max_big(int Tk) { return Tk / kSchedBigBM; }
int sched_max_rem(int Tk, int E) { return std::min(2 * E, sched_max_mtiles(Tk, E)); }
size_t sched_entries(int Tk, int E) {
  return 3 + (size_t)sched_max_mtiles(Tk, E) + sched_max_big(Tk) + sched_max_rem(Tk, E);
}
namespace {
struct SchedTables {
  int2 *full, *big, *rem;
};
SchedTables sched_tables(const int2* sched, int Tk, int E) {
  int2* f = const_cast<int2*>(sched);
  int2* b = f + 1 + sched_max_mtiles(Tk, E);
  return {f, b, b + 1 + sched_max_big(Tk)};
}
}  // namespace

hipError_t launch_sched_build(const int32_t* offsets, int E, int Tk, int2* sched, hipStream_t s) {
  const SchedTables t = sched_tables(sched, Tk, E);
  {
    TraceScope trace("sched_build", s);
    hipLaunchKernelGGL(sched_build_kernel, dim3(1), dim3(1024), 0, s, offsets, E, t.full, t.big,
                       t.rem);
  }
  return hipGetLastError();
}

// The forward GEMMs run the 256-row blocks with the big-tile kernel, then the remainders.
hipError_t launch_fwd_gateup(const GemmFwdGateUpArgs& x, bool persistent, hipStream_t s) {
  const SchedTables st = sched_tables(x.sched, x.Tk, x.E);
  FwdGateUpBig::Args ab{x.xp, x.w1, x.H, x.A, x.offsets, st.big, x.d, x.I};
  hipError_t e = launch_dma<DmaGateUp>(ab, sched_max_big(x.Tk) * (x.I / 128), persistent, s);
  if (e != hipSuccess) return e;
  FwdGateUp::Args a{x.xp, x.w1, x.H, x.A, x.offsets, st.rem, x.d, x.I};
  return launch<FwdGateUp>(a, sched_max_rem(x.Tk, x.E) * (x.I / 64), persistent, s);
}

hipError_t launch_fwd_down(const GemmFwdDownArgs& x, bool persistent, hipStream_t s) {
  const SchedTables st = sched_tables(x.sched, x.Tk, x.E);
  FwdDownBig::Args ab{x.A, x.w2, x.O, x.offsets, st.big, x.d, x.I};
  hipError_t e = launch_dma<DmaDown>(ab, sched_max_big(x.Tk) * (x.d / 256), persistent, s);
  if (e != hipSuccess) return e;
  FwdDown::Args a{x.A, x.w2, x.O, x.offsets, st.rem, x.d, x.I};
  return launch<FwdDown>(a, sched_max_rem(x.Tk, x.E) * (x.d / 128), persistent, s);
}

// With I a multiple of 256 the down dgrad runs the 256-row blocks with dma_kernel<DmaDownDgrad>,
// then the remainders; otherwise every 128-row block with the 128 x 128 kernel.
hipError_t launch_bwd_down_dgrad(const GemmBwdDownDgradArgs& x, bool persistent, hipStream_t s) {
  const SchedTables st = sched_tables(x.sched, x.Tk, x.E);
  const bool big = x.I % kDgT == 0;
  const int max_big = big ? sched_max_big(x.Tk) * (x.I / kDgT) : 0;
  if (max_big > 0) {
    DownDgradBigArgs ab{x.dy, x.row_src, x.topk_w, x.w2, x.H, x.A, x.dH, x.dwpart,
                        x.offsets, st.big, x.d, x.I, x.k};
    const hipError_t e = launch_dma<DmaDownDgrad>(ab, max_big, true, s);
    if (e != hipSuccess) return e;
  }
  BwdDownDgrad::Args a{x.dy, x.row_src, x.topk_w, x.w2, x.H, x.A, x.dH, x.dwpart,
                       x.offsets, big ? st.rem : st.full, x.d, x.I, x.k};
  const int max_small = big ? sched_max_rem(x.Tk, x.E) : sched_max_mtiles(x.Tk, x.E);
  return launch<BwdDownDgrad>(a, max_small * (x.I / 128), persistent, s);
}

// The gate dgrad runs the 256-row blocks with dma_kernel<DmaGateDgrad>, then the remainders.
hipError_t launch_bwd_gate_dgrad(const GemmBwdGateDgradArgs& x, bool persistent, hipStream_t s) {
  const SchedTables st = sched_tables(x.sched, x.Tk, x.E);
  const int max_big = sched_max_big(x.Tk) * (x.d / kDgT);
  if (max_big > 0) {
    GateDgradBigArgs ab{x.dH, x.w1, x.dXp, x.offsets, st.big, x.d, x.I};
    const hipError_t e = launch_dma<DmaGateDgrad>(ab, max_big, true, s);
    if (e != hipSuccess) return e;
  }
  BwdGateDgrad::Args a{x.dH, x.w1, x.dXp, x.offsets, st.rem, x.d, x.I};
  return launch<BwdGateDgrad>(a, sched_max_rem(x.Tk, x.E) * (x.d / 128), persistent, s);
}

// The 128-row MX kernels, instantiated for both scale-load forms (GeoMx::GS) and picked by the
// GEMM's K extent, and the 256-row ones, each for both code widths.
template <class T>
struct Tag {
  using type = T;
};
// f(Tag<P<F, K % 512 == 0>>) for the code width fbits
template <template <int, bool> class P, class Fn>
hipError_t with_mx(int fbits, int K, Fn&& f) {
  const bool gs = K % 512 == 0;
  if (fbits == 4) return gs ? f(Tag<P<4, true>>{}) : f(Tag<P<4, false>>{});
  return gs ? f(Tag<P<8, true>>{}) : f(Tag<P<8, false>>{});
}
// f(Tag<D<F>>) for the code width fbits
template <template <int> class D, class Fn>
hipError_t with_big(int fbits, Fn&& f) {
  return fbits == 4 ? f(Tag<D<4>>{}) : f(Tag<D<8>>{});
}

// The MX GEMMs run the 256-row blocks with dmx_kernel, then the remainders on the 128-row
// kernels.
hipError_t launch_fwd_gateup_mx(const GemmMxGateUpArgs& x, bool persistent, hipStream_t s) {
  const SchedTables st = sched_tables(x.sched, x.Tk, x.E);
  hipError_t e = with_big<DmxGateUp>(x.fbits, [&](auto tag) {
    using D = typename decltype(tag)::type;
    typename D::Args ab{x.xp8, x.xps, x.w8, x.ws, x.H, x.A, x.aq, x.aqs, x.offsets, st.big,
                        x.d, x.I};
    return launch_dmx<D>(ab, sched_max_big(x.Tk) * (x.I / D::P::kA), true, s);
  });
  if (e != hipSuccess) return e;
  return with_mx<MxFwdGateUpS>(x.fbits, x.d, [&](auto tag) {
    using P = typename decltype(tag)::type;
    typename P::Args a{x.xp8, x.xps, x.w8, x.ws, x.H, x.A, x.aq, x.aqs, x.offsets, st.rem,
                       x.d, x.I};
    return launch<P>(a, sched_max_rem(x.Tk, x.E) * (x.I / P::kA), persistent, s);
  });
}

hipError_t launch_fwd_down_mx(const GemmMxDownArgs& x, bool persistent, hipStream_t s) {
  const SchedTables st = sched_tables(x.sched, x.Tk, x.E);
  hipError_t e = with_big<DmxDown>(x.fbits, [&](auto tag) {
    using D = typename decltype(tag)::type;
    typename D::Args ab{x.aq, x.aqs, x.w8, x.ws, x.O, x.offsets, st.big, x.d, x.I};
    return launch_dmx<D>(ab, sched_max_big(x.Tk) * (x.d / 256), true, s);
  });
  if (e != hipSuccess) return e;
  return with_mx<MxFwdDownS>(x.fbits, x.I, [&](auto tag) {
    using P = typename decltype(tag)::type;
    typename P::Args a{x.aq, x.aqs, x.w8, x.ws, x.O, x.offsets, st.rem, x.d, x.I};
    return launch<P>(a, sched_max_rem(x.Tk, x.E) * (x.d / 128), persistent, s);
  });
}

// With I a multiple of 256 (always so in MXFP4) the MX down dgrad runs the 256-row blocks with
// dmx_kernel, then the remainders; otherwise every 128-row block on the 128-row kernel.
hipError_t launch_bwd_down_dgrad_mx(const GemmMxDownDgradArgs& x, bool persistent, hipStream_t s) {
  const SchedTables st = sched_tables(x.sched, x.Tk, x.E);
  const bool big = x.I % 256 == 0;
  const int max_big = big ? sched_max_big(x.Tk) * (x.I / 256) : 0;
  if (max_big > 0) {
    const hipError_t e = with_big<DmxDownDgrad>(x.fbits, [&](auto tag) {
      using D = typename decltype(tag)::type;
      typename D::Args ab{x.dyq,    x.dys, x.row_src, x.topk_w, x.w8, x.ws,
                          x.H,      x.A,   x.dH,      x.dwpart, x.dhq, x.dhs,
                          x.offsets, st.big, x.d,     x.I,      x.k};
      return launch_dmx<D>(ab, max_big, true, s);
    });
    if (e != hipSuccess) return e;
  }
  const int mt = big ? sched_max_rem(x.Tk, x.E) : sched_max_mtiles(x.Tk, x.E);
  return with_mx<MxBwdDownDgradS>(x.fbits, x.d, [&](auto tag) {
    using P = typename decltype(tag)::type;
    typename P::Args a{x.dyq, x.dys, x.row_src, x.topk_w, x.w8,  x.ws, x.H,
                       x.A,   x.dH,  x.dwpart,  x.dhq,    x.dhs, x.offsets,
                       big ? st.rem : st.full, x.d, x.I, x.k};
    return launch<P>(a, mt * (x.I / 128), persistent, s);
  });
}

hipError_t launch_bwd_gate_dgrad_mx(const GemmMxGateDgradArgs& x, bool persistent, hipStream_t s) {
  const SchedTables st = sched_tables(x.sched, x.Tk, x.E);
  hipError_t e = with_big<DmxGateDgrad>(x.fbits, [&](auto tag) {
    using D = typename decltype(tag)::type;
    typename D::Args ab{x.dhq, x.dhs, x.w8, x.ws, x.dXp, x.offsets, st.big, x.d, x.I};
    return launch_dmx<D>(ab, sched_max_big(x.Tk) * (x.d / 256), true, s);
  });
  if (e != hipSuccess) return e;
  return with_mx<MxBwdGateDgradS>(x.fbits, 2 * x.I, [&](auto tag) {
    using P = typename decltype(tag)::type;
    typename P::Args a{x.dhq, x.dhs, x.w8, x.ws, x.dXp, x.offsets, st.rem, x.d, x.I};
    return launch<P>(a, sched_max_rem(x.Tk, x.E) * (x.d / 128), persistent, s);
  });
}

template <bool ACC, bool BF>
hipError_t launch_mx_wgrad_as(const GemmMxWgradArgs& x, int max_tiles, bool persistent,
                              hipStream_t s) {
  typename MxWgrad<ACC, BF>::Args a{x.lq, x.lqs, x.rq, x.rqs, x.dw, x.poff, x.E, x.Mdim, x.Ndim,
                                    x.P};
  return launch_named<MxWgrad<ACC, BF>>(a, max_tiles, persistent, x.name, s);
}

hipError_t launch_mx_wgrad(const GemmMxWgradArgs& x, bool persistent, hipStream_t s) {
  const int max_tiles = (x.E * (x.Mdim / 128) * (x.Ndim / 128) + kXcds - 1) / kXcds * kXcds;
  if (x.bf16_dw)
    return x.accumulate ? launch_mx_wgrad_as<true, true>(x, max_tiles, persistent, s)
                        : launch_mx_wgrad_as<false, true>(x, max_tiles, persistent, s);
  return x.accumulate ? launch_mx_wgrad_as<true, false>(x, max_tiles, persistent, s)
                      : launch_mx_wgrad_as<false, false>(x, max_tiles, persistent, s);
}

}  // namespace moe
