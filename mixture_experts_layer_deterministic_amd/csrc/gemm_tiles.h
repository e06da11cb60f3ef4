// Tile code of the BF16 grouped GEMMs whose rows are token positions: the register-staged
// loaders, the tile geometry, the row-block schedule decode, Problems 1 and 2 (the forward
// gate/up with its SwiGLU epilogue, and the forward down projection) and the K loop of a
// 128 x 128 (or 256 x 256) tile. gemm.hip launches them as grouped GEMMs; the single-launch
// forward (fused.hip) runs the same tiles inside one persistent kernel.
//
// The expert-grouped GEMMs are named in the MarkTechPost page on Mixture-of-Kittens (MoK),
// section "Three design decisions that matter".
#pragma once

#include <type_traits>

#include "common.h"

namespace moe {

constexpr int kThreads = 256;

// ------------------------------------------------------------------------------------------
// Tile loaders (global -> registers -> LDS)

// ROWS x BK tile whose rows are K-contiguous in memory. Rows are element offsets from one base
// pointer (32 bits each, so a thread holds one register per row rather than a pointer);
// rowoff(r) < 0 marks a row that loads zeros. With MAYBE_NULL false every row is real, and the
// loads carry no per-row condition (no branches around them). Every loader here passes real
// rows (a tile's rows past its expert's count repeat the last row). The null form stays: the
// same loaders written without it allocate registers differently and spill 32-56 bytes a lane.
template <int ROWS, int BK, int LDK, int THREADS = kThreads, bool MAYBE_NULL = true>
struct LoadK {
  static constexpr int VPR = BK / 8;
  static constexpr int NV = ROWS * VPR;
  static constexpr int PT = (NV + THREADS - 1) / THREADS;
  static constexpr uint32_t kNull = 0xffffffffu;
  static_assert(BK == 64 && LDK == 64, "rows of 64 values in the chunk-permuted LDS layout");
  const uint16_t* base;
  uint32_t off[PT];
  uint4 r[PT];

  template <class RowOff>
  MOE_DEV void init(const uint16_t* b, RowOff rowoff) {
    base = b;
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const int v = threadIdx.x + THREADS * j;
      const long long o = v < NV ? rowoff(v / VPR) : -1;
      off[j] = o < 0 ? kNull : static_cast<uint32_t>(o + (v % VPR) * 8);
    }
  }
  MOE_DEV void load(int k0) {
#pragma unroll
    for (int j = 0; j < PT; ++j)
      r[j] = !MAYBE_NULL || off[j] != kNull ? *reinterpret_cast<const uint4*>(base + off[j] + k0)
                                            : make_uint4(0, 0, 0, 0);
  }
  MOE_DEV void store(uint16_t* s) const {
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const int v = threadIdx.x + THREADS * j;
      if (v < NV) *reinterpret_cast<uint4*>(s + rowswz(v / VPR, v % VPR)) = r[j];
    }
  }
};

// BK x MN tile stored MN-contiguous in memory (K is the slow axis), copied into LDS as it sits
// in memory: K row k of the stage holds the tile's MN values, with its 32-byte column groups
// permuted by kmajor_swz(k). The MFMA fragments come from gfx950's transposing LDS read
// (kmajor_frag), so no value is transposed in registers. Each thread moves BK * MN / 8 /
// kThreads 16-byte pieces; MN / 8 consecutive threads cover one K row. The pieces are the
// dgrads' weight stream, read once, so they are read non-temporally (gate dgrad at the
// DeepSeek-V3 shape 3.06-3.11 -> 2.81-2.98 ms).
template <int MN, int BK>
struct LoadKM {
  static constexpr int CPR = MN / 8;
  static constexpr int NV = BK * CPR;
  static constexpr int PT = NV / kThreads;
  static_assert(NV % kThreads == 0 && MN <= 128, "whole pieces per thread, swizzle in a row");
  uint4 r[PT];

  // w: the tile's first column in its first K row of this step; ld: the row pitch
  MOE_DEV void load(const uint16_t* w, int ld) {
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const int v = threadIdx.x + kThreads * j;
      r[j] = nt_load16(w + (uint32_t)((v / CPR) * ld + (v % CPR) * 8));
    }
  }
  MOE_DEV void store(uint16_t* s) const {
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const int v = threadIdx.x + kThreads * j, k = v / CPR;
      *reinterpret_cast<uint4*>(s + k * MN + (((v % CPR) * 8) ^ kmajor_swz(k))) = r[j];
    }
  }
};

// Whether problem P keeps its B operand K-major in LDS (P::kBKMajor, LoadKM) rather than in
// rowswz rows; false where P does not say.
template <class P, class = void>
struct BKMajor {
  static constexpr bool value = false;
};
template <class P>
struct BKMajor<P, std::void_t<decltype(P::kBKMajor)>> {
  static constexpr bool value = P::kBKMajor;
};

// ------------------------------------------------------------------------------------------
// Tile geometry shared by all problems

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_>
struct Geo {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int MB = WM / 16, NB = WN / 16;
  static constexpr int LDK = BK;                 // LDS row pitch (chunk-permuted rows, rowswz)
  static constexpr int STAGE = (BM + BN) * LDK;  // uint16 elements per LDS stage
  static constexpr int kSmem = 2 * STAGE * 2;    // bytes, two stages
  static constexpr bool kMx = false;
  static constexpr int THREADS = WAVES_M * WAVES_N * kWave;
  static constexpr int kWavesPerEU = 2;  // at most 256 registers per lane
  // 256-row tiles only ever cover full 256-row blocks of one expert: every row is real
  static constexpr bool kFull = BM == 256;
  static_assert(WAVES_M * WAVES_N == 4 || WAVES_M * WAVES_N == 8, "4 or 8 waves per workgroup");
  static_assert(BK % 32 == 0 && WM % 16 == 0 && WN % 16 == 0, "tile shape");
};
using GeoSmall = Geo<128, 128, 64, 1, 4>;
// Tiles of 256 full rows of one expert, for experts whose row count makes the GEMM MFMA-bound.
// There the kernel's rate follows the flops per byte its tile loads (mostly L2 hits): 64 flop/B
// for 128 x 128 tiles, 128 for 256 x 256. Eight waves of 128 x 64 (128 accumulators each) make
// the 256 x 256 tile, one workgroup per CU; K steps of 64 keep each row load a whole 128-byte
// line (steps of 32 fetched half lines and ran 16% slower).
using GeoBig = Geo<256, 256, 64, 2, 4>;

// Row segment of one expert for dynamic-M problems. A tile table entry holds the expert and
// the segment's row count (x = e | mcount << 16) and its first row position (y), so a tile
// finds its rows with one read.
struct MTile {
  int e, row0, mcount;
};
MOE_DEV int2 mtile_entry(int e, int row0, int mcount) {
  return make_int2(e | (mcount << 16), row0);
}
MOE_DEV MTile decode_mtile(const int2* sched, int mt) {
  const int2 ent = sched[1 + mt];
  MTile t;
  t.e = ent.x & 0xffff;
  t.mcount = ent.x >> 16;
  t.row0 = ent.y;
  return t;
}

// Linear tile index -> (m-tile, n-tile). Ungrouped, n runs fastest: the workgroups an XCD runs
// at once share one m-tile's activations in its L2. Grouped, kGroupM consecutive m-tiles take
// each n-tile in turn, so the workgroups in flight on an XCD share a few activation panels and
// a few weight panels: an expert with many row blocks re-reads each weight panel once per block,
// and grouped blocks fetch it from L2 rather than from beyond it.
constexpr int kGroupM = 4;
template <bool kGrouped>
MOE_DEV int2 tile_mn(int lt, int nm, int ntc) {
  if constexpr (!kGrouped) {
    return make_int2(lt / ntc, lt % ntc);
  } else {
    const int group = lt / (kGroupM * ntc);
    const int m_first = group * kGroupM;
    const int gm = min(kGroupM, nm - m_first);
    const int r = lt - m_first * ntc;
    return make_int2(m_first + r % gm, r / gm);
  }
}

// ------------------------------------------------------------------------------------------
// Problem 1: forward gate/up GEMM with the SwiGLU epilogue.
// B rows 0..BN/2-1 of the LDS tile are gate rows n0.. of W1[e], rows BN/2.. the matching up
// rows I+n0..; wave w owns gate columns [w*WN/2, (w+1)*WN/2) and the same up columns, so each
// lane holds g and u for the same (row, column) and can finish SwiGLU in registers.
template <class G_>
struct FwdGateUpT {
  static constexpr const char* kName = G_::BM == 256 ? "fwd_gateup_big" : "fwd_gateup";
  using G = G_;
  struct Args {
    const uint16_t* xp;    // [T*k, d]
    const uint16_t* w1;    // [E, 2I, d]
    uint16_t* H;           // [T*k, 2I]
    uint16_t* A;           // [T*k, I]
    const int32_t* offsets;
    const int2* sched;
    int d, I;
  };
  struct Tile {
    MTile m;
    int n0;  // first gate column
  };
  static MOE_DEV int ntiles(const Args& a) { return a.sched[0].x * (a.I / (G::BN / 2)); }
  static MOE_DEV Tile decode(const Args& a, int lt) {
    const int nt_count = a.I / (G::BN / 2);
    const int2 mn = tile_mn<(G::BM > 128)>(lt, a.sched[0].x, nt_count);
    Tile t;
    t.m = decode_mtile(a.sched, mn.x);
    t.n0 = mn.y * (G::BN / 2);
    return t;
  }
  static MOE_DEV int num_k(const Args& a, const Tile&) { return a.d / G::BK; }
  static MOE_DEV int k_first(const Tile&, int) { return 0; }
  static MOE_DEV bool m_active(const Tile& t, int m) { return m < t.m.mcount; }
  static MOE_DEV int brow(int wn, int nb) {  // LDS B row of n-block nb for wave wn
    constexpr int H2 = G::BN / 2, WH = G::WN / 2;
    return nb < G::NB / 2 ? wn * WH + nb * 16 : H2 + wn * WH + (nb - G::NB / 2) * 16;
  }
  struct Loader {
    LoadK<G::BM, G::BK, G::LDK, G::THREADS, false> la;
    LoadK<G::BN, G::BK, G::LDK, G::THREADS, false> lb;
    // Rows past the expert's count repeat its last row (their outputs are never stored), so no
    // load is conditional. Zero rows behind per-row branches made the compiler wait on half the
    // activation loads before issuing the weight loads of each K step (fwd_gateup at the
    // DeepSeek-V3 shape 3.0 -> 2.87 ms with this and the weights-first order).
    MOE_DEV void init(const Args& a, const Tile& t) {
      const int d = a.d, mc = t.m.mcount;
      la.init(a.xp + (size_t)t.m.row0 * d, [&](int m) { return (long long)min(m, mc - 1) * d; });
      const int n0 = t.n0, I = a.I;
      lb.init(a.w1 + (size_t)t.m.e * 2 * I * d, [&](int n) {
        const int row = n < G::BN / 2 ? n0 + n : I + n0 + n - G::BN / 2;
        return (long long)row * d;
      });
    }
    MOE_DEV void load(int kt) {  // weights first: they are the HBM stream
      lb.load(kt * G::BK);
      la.load(kt * G::BK);
    }
    MOE_DEV void store(uint16_t* s) const {
      la.store(s);
      lb.store(s + G::BM * G::LDK);
    }
  };
  static MOE_DEV void epilogue(const Args& a, const Tile& t, f32x4 (&acc)[G::MB][G::NB],
                               uint16_t*) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int wn = wave % G::WAVES_N, wm = wave / G::WAVES_N;
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb) {
      const int m = wm * G::WM + mb * 16 + lane % 16;
      if (m >= t.m.mcount) continue;
      const size_t pos = t.m.row0 + m;
#pragma unroll
      for (int nb = 0; nb < G::NB / 2; ++nb) {
        const int j = t.n0 + wn * (G::WN / 2) + nb * 16 + 4 * (lane / 16);
        const f32x4 g = acc[mb][nb], u = acc[mb][nb + G::NB / 2];
        uint2 hg, hu, av;
        hg.x = pack_bf2(g[0], g[1]);
        hg.y = pack_bf2(g[2], g[3]);
        hu.x = pack_bf2(u[0], u[1]);
        hu.y = pack_bf2(u[2], u[3]);
        av.x = pack_bf2(silu(g[0]) * u[0], silu(g[1]) * u[1]);
        av.y = pack_bf2(silu(g[2]) * u[2], silu(g[3]) * u[3]);
        *reinterpret_cast<uint2*>(a.H + pos * 2 * a.I + j) = hg;
        *reinterpret_cast<uint2*>(a.H + pos * 2 * a.I + a.I + j) = hu;
        *reinterpret_cast<uint2*>(a.A + pos * a.I + j) = av;
      }
    }
  }
};

using FwdGateUp = FwdGateUpT<GeoSmall>;
using FwdGateUpBig = FwdGateUpT<GeoBig>;

// ------------------------------------------------------------------------------------------
// Problem 2: forward down GEMM. O[pos] = A[pos] . W2[e]^T, stored bf16.
template <class G_>
struct FwdDownT {
  static constexpr const char* kName = G_::BM == 256 ? "fwd_down_big" : "fwd_down";
  using G = G_;
  struct Args {
    const uint16_t* A;   // [T*k, I]
    const uint16_t* w2;  // [E, d, I]
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
  // W2's rows are 2I bytes apart (4 KB at I = 2048): tiles that start K together read the same
  // column of 128 rows, which alias in HBM. Each n-tile starts at its own K-chunk and wraps.
  static MOE_DEV int k_first(const Tile& t, int nk) { return (t.n0 / G::BN) % nk; }
  static MOE_DEV bool m_active(const Tile& t, int m) { return m < t.m.mcount; }
  static MOE_DEV int brow(int wn, int nb) { return wn * G::WN + nb * 16; }
  struct Loader {
    LoadK<G::BM, G::BK, G::LDK, G::THREADS, false> la;
    LoadK<G::BN, G::BK, G::LDK, G::THREADS, false> lb;
    // rows past the count repeat the last row, as in Problem 1's loader
    MOE_DEV void init(const Args& a, const Tile& t) {
      const int I = a.I, mc = t.m.mcount;
      la.init(a.A + (size_t)t.m.row0 * I, [&](int m) { return (long long)min(m, mc - 1) * I; });
      lb.init(a.w2 + ((size_t)t.m.e * a.d + t.n0) * I, [&](int n) { return (long long)n * I; });
    }
    MOE_DEV void load(int kt) {  // weights first: they are the HBM stream
      lb.load(kt * G::BK);
      la.load(kt * G::BK);
    }
    MOE_DEV void store(uint16_t* s) const {
      la.store(s);
      lb.store(s + G::BM * G::LDK);
    }
  };
  static MOE_DEV void epilogue(const Args& a, const Tile& t, f32x4 (&acc)[G::MB][G::NB],
                               uint16_t*) {
    const int lane = threadIdx.x % kWave, wn = (threadIdx.x / kWave) % G::WAVES_N;
    const int wm = (threadIdx.x / kWave) / G::WAVES_N;
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

using FwdDown = FwdDownT<GeoSmall>;
using FwdDownBig = FwdDownT<GeoBig>;

// ------------------------------------------------------------------------------------------
// The K loop of one tile: double-buffered LDS stages, fragments read ahead of the MFMAs, then
// the problem's epilogue.
template <class P>
MOE_DEV void run_tile(const typename P::Args& a, const typename P::Tile& t, uint16_t* smem) {
  using G = typename P::G;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int wm = wave / G::WAVES_N, wn = wave % G::WAVES_N;
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
    ld.store(smem);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      uint16_t* cur = smem + (kt & 1) * G::STAGE;
      if (kt + 1 < nk) ld.load(kt + 1 + k0 < nk ? kt + 1 + k0 : kt + 1 + k0 - nk);
      // fragment rows are 16-row blocks, so rowswz's permutation is the lane's own: chunk
      // (4 ks + lane / 16) ^ (lane & 7) of row (block + lane % 16)
      const uint16_t* sA = cur + (wm * G::WM + lane % 16) * G::LDK;
      const uint16_t* sB = cur + G::BM * G::LDK + (lane % 16) * G::LDK;
      const int c0 = ((lane / 16) ^ (lane & 7)) << 3, c1 = ((4 + lane / 16) ^ (lane & 7)) << 3;
      if constexpr (G::kFull && G::BK == 64) {
        mma_k64<G::MB, G::NB, 1, 1>(
            acc,
            [&](int ks, int mb) {
              return *reinterpret_cast<const uint4*>(sA + mb * 16 * G::LDK + (ks ? c1 : c0));
            },
            [&](int ks, int nb) {
              return *reinterpret_cast<const uint4*>(sB + P::brow(wn, nb) * G::LDK +
                                                     (ks ? c1 : c0));
            });
      } else
#pragma unroll
      for (int ks = 0; ks < G::BK / 32; ++ks) {
        const int co = ks ? c1 : c0;
        // All fragments of the step are read before the first MFMA, so the LDS latency is paid
        // once per step rather than once per 16-row block.
        uint4 bf[G::NB], af[G::MB];
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb) {
          if constexpr (BKMajor<P>::value)
            bf[nb] = kmajor_frag<G::BN>(cur + G::BM * G::LDK, P::brow(wn, nb), 32 * ks, lane);
          else
            bf[nb] = *reinterpret_cast<const uint4*>(sB + P::brow(wn, nb) * G::LDK + co);
        }
#pragma unroll
        for (int mb = 0; mb < G::MB; ++mb)
          af[mb] = *reinterpret_cast<const uint4*>(sA + mb * 16 * G::LDK + co);
#pragma unroll
        for (int mb = 0; mb < G::MB; ++mb) {
          if (!P::m_active(t, wm * G::WM + mb * 16)) continue;
#pragma unroll
          for (int nb = 0; nb < G::NB; ++nb) acc[mb][nb] = mfma16(bf[nb], af[mb], acc[mb][nb]);
        }
      }
      if (kt + 1 < nk) ld.store(smem + ((kt + 1) & 1) * G::STAGE);
      __syncthreads();
    }
  }
  P::epilogue(a, t, acc, smem);
  __syncthreads();
}

}  // namespace moe
