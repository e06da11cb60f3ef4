// Expert weight gradients on gfx950 MFMA: dW[e] = sum over the positions p of expert e, in
// ascending order, of L[p]^T (x) R[p], accumulated in fp32.
//   gate/up : L = dH  [T*k, 2I], R = Xp [T*k, d]  -> dW1 [E, 2I, d]
//   down    : L = dYw [T*k, d],  R = A  [T*k, I]  -> dW2 [E, d, I]   (dYw = bf16(w * dY[t]))
// The expert-grouped GEMMs are named in the MarkTechPost page on Mixture-of-Kittens (MoK),
// section "Three design decisions that matter"; their wgrad is a plain sum over the tokens an
// expert received.
//
// Both operands are position-major in memory (K is the slow axis), and the output is the big
// tensor: with tens of positions per expert the kernel is bound by writing dW. It is a
// persistent grid that walks a device-built task table. Each task is one 256-row stripe of
// one expert's dW and a run of consecutive 128-column tiles; the stripe's L rows are loaded
// once per task and shared by all its tiles, which halves the R traffic of 128-row stripes.
// Inside a task the pipeline runs on across tile boundaries. The table orders experts by
// decreasing row count (ties to the lower index), so the longest tasks start first. Each task
// holds roughly the same number of K-steps: an expert with few rows gets long runs of tiles, a
// heavy expert runs of one tile.
//
// The waves are specialised. On gfx950 a wave's vector-memory counter covers its loads and
// stores in issue order, so a wave that stores a 64 KB dW tile and then waits for its next
// operand load also waits for those stores to land. Here eight consumer waves (one 64 x 64 block
// of the 256 x 128 tile each) run the MFMAs and store dW, and never load; four producer waves
// only load the operands into LDS. The two sides meet at a barrier that waits for LDS traffic
// only, so stores of many tiles stay in flight.
//
// Experts with many rows (at least kWgradBigRows) make the product MFMA-bound rather than
// write-bound. They go to a second kernel with 256 x 256 output tiles and 64-position K steps,
// twice the flops per loaded byte of the 256 x 128 tiles (see DmaWgrad).
//
// Determinism: every dW element belongs to exactly one task, whose workgroup reduces K in
// ascending position order. No atomics, no split-K.
#include <type_traits>

#include "common.h"
#include "dma.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int BM = kWgradBM, BN = kWgradBN, BK = 32;
constexpr int kWgradBigRows = 512;  // experts with at least this many rows: DmaWgrad
constexpr int kEmptyRun = 4;        // tiles per task of an expert with no rows (zero fill)
constexpr int KRES = 128;           // positions of L kept resident in LDS for a whole task
constexpr int LDL = KRES + 8;       // row pitch of the L buffer [BM][LDL]
constexpr int LDR = BK + 8;         // row pitch of an R stage [BN][LDR]
constexpr int kConsumerWaves = (BM / 64) * (BN / 64);  // one 64 x 64 block of dW each
constexpr int kConsumers = kWave * kConsumerWaves;      // MFMA and dW stores
constexpr int kProducers = 4;                           // the next waves: operand loads
constexpr int kThreads = kConsumers + kWave * kProducers;
constexpr int kWavesPerSimd = (kThreads / kWave + 3) / 4;
constexpr int R_STAGE = BN * LDR;   // uint16 elements per R stage

struct Args {
  const uint16_t* L;  // [T*k, Mdim]
  const uint16_t* R;  // [T*k, Ndim] bf16, or null when R is MX: codes R8, scales R8s
  const uint8_t* R8;  // [T*k, Ndim * F / 8]: E4M3 (F = 8) or packed E2M1 (F = 4) codes
  const uint8_t* R8s; // [T*k, Ndim/32]
  void* dw;           // [E, Mdim, Ndim], fp32 or (BF kernels) bf16
  const int32_t* offsets;
  const int4* table;  // (expert, first row, first n-tile, n-tile count)
  const int32_t* count;
  int Mdim, Ndim, accumulate;
};

// One producer wave moves a whole chunk of 32 positions x 64 NH columns of an operand: blocks
// of 4 positions x 8 columns, NH per lane (block b = lane + 64 h covers positions [4 (b % 8),
// +4) and columns [8 (b / 8), +8)). Rows are read as 16-byte vectors and transposed in
// registers, so LDS holds [MN][K] and each MFMA fragment is one 16-byte LDS read.
template <int NH>
struct Mover {
  const uint16_t* base;  // operand base, already offset to the task's first column
  const uint8_t* base8;  // MX operand: codes and per-32 scales (MX loads only)
  const uint8_t* sc8;
  int ld;                // row pitch of the operand (elements)
  uint4 r[NH][4];

  // RF = 8: the operand is MXFP8 (E4M3 codes with one scale per 32 along the row); RF = 4:
  // MXFP4 (E2M1 codes, two a byte). The load keeps the raw codes (x, and y for E4M3) and the
  // scale code (z) of each 8-column piece; `store` expands them to their exact bf16 values, so
  // the conversion waits for data only when the chunk is written. RF = 0: bf16.
  template <int RF = 0>
  MOE_DEV void load(int pbase, int p1, int col0, int lane) {
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int b = lane + kWave * h, kq = b % 8, mb = b / 8;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int p = pbase + kq * 4 + rr;
        if constexpr (RF == 0) {
          r[h][rr] = p < p1 ? *reinterpret_cast<const uint4*>(base + (size_t)p * ld + col0 + mb * 8)
                            : make_uint4(0, 0, 0, 0);
        } else {
          uint4 v = make_uint4(0, 0, 0, 0);
          if (p < p1) {
            const int c = col0 + mb * 8;
            if constexpr (RF == 8) {
              const uint2 q = *reinterpret_cast<const uint2*>(base8 + (size_t)p * ld + c);
              v.x = q.x;
              v.y = q.y;
            } else {
              v.x = *reinterpret_cast<const uint32_t*>(base8 + (size_t)p * (ld / 2) + c / 2);
            }
            v.z = sc8[(size_t)p * (ld / 32) + c / 32];
          }
          r[h][rr] = v;
        }
      }
    }
  }
  static MOE_DEV uint4 expand_fp8(const uint4 raw) {
    const float s = mx_scale(raw.z);
    float f[4], g[4];
    e4m3x4_to_f32(raw.x, f);
    e4m3x4_to_f32(raw.y, g);
    uint4 v;
    v.x = pack_bf2(f[0] * s, f[1] * s);
    v.y = pack_bf2(f[2] * s, f[3] * s);
    v.z = pack_bf2(g[0] * s, g[1] * s);
    v.w = pack_bf2(g[2] * s, g[3] * s);
    return v;
  }
  static MOE_DEV uint4 expand_fp4(const uint4 raw) {
    const float s = mx_scale(raw.z);
    const float2 f0 = e2m1x2_to_f32<0>(raw.x), f1 = e2m1x2_to_f32<1>(raw.x),
                 f2 = e2m1x2_to_f32<2>(raw.x), f3 = e2m1x2_to_f32<3>(raw.x);
    uint4 v;
    v.x = pack_bf2(f0.x * s, f0.y * s);
    v.y = pack_bf2(f1.x * s, f1.y * s);
    v.z = pack_bf2(f2.x * s, f2.y * s);
    v.w = pack_bf2(f3.x * s, f3.y * s);
    return v;
  }
  template <int RF>
  static MOE_DEV uint4 expand(const uint4 raw) {
    if constexpr (RF == 8) return expand_fp8(raw);
    else if constexpr (RF == 4) return expand_fp4(raw);
    else return raw;
  }
  // Writes the transposed blocks into an LDS buffer [MN][ldk] at K column kcol.
  template <int RF = 0>
  MOE_DEV void store(uint16_t* s, int ldk, int kcol, int lane) const {
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int b = lane + kWave * h, kq = b % 8, mb = b / 8;
      uint4 e[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) e[rr] = expand<RF>(r[h][rr]);
      const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&e[0]);
      const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&e[1]);
      const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&e[2]);
      const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&e[3]);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int q = c >> 1;
        uint2 v;
        if (c & 1) {
          v.x = (w0[q] >> 16) | (w1[q] & 0xffff0000u);
          v.y = (w2[q] >> 16) | (w3[q] & 0xffff0000u);
        } else {
          v.x = (w0[q] & 0xffffu) | (w1[q] << 16);
          v.y = (w2[q] & 0xffffu) | (w3[q] << 16);
        }
        *reinterpret_cast<uint2*>(s + (mb * 8 + c) * ldk + kcol + kq * 4) = v;
      }
    }
  }
};

constexpr int WMR = 64;        // dW rows per consumer wave (BM / 64 x BN / 64 waves)
constexpr int MBW = WMR / 16;  // 16-row MFMA blocks per consumer wave

// dW element type: fp32, or bf16 in the BF kernels
template <bool BF>
using DwT = std::conditional_t<BF, uint16_t, float>;

// out: the element offset of the task's first dW row (column 0)
template <bool ACC, bool BF>
MOE_DEV void store_tile(const Args& a, size_t out, int n0, const f32x4 (&acc)[MBW][4]) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int wm = wave / (BN / 64), wn = wave % (BN / 64);
  DwT<BF>* base = static_cast<DwT<BF>*>(a.dw) + out;
#pragma unroll
  for (int mb = 0; mb < MBW; ++mb) {
    const int m = wm * WMR + mb * 16 + lane % 16;
    if constexpr (BF) {
      uint16_t* row = base + (size_t)m * a.Ndim + n0 + wn * 64;
#pragma unroll
      for (int nb = 0; nb < 4; nb += 2)
        store_dw8_bf16<ACC>(row + nb * 16, acc[mb][nb], acc[mb][nb + 1], lane);
    } else {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int n = n0 + wn * 64 + nb * 16 + 4 * (lane / 16);
        store_dw4<ACC>(base + (size_t)m * a.Ndim + n, acc[mb][nb]);
      }
    }
  }
}

// Workgroup barrier that waits for this wave's LDS operations only; global stores stay in
// flight across it.
MOE_DEV void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// L lives in LDS as [BM][LDL]. When the expert has at most KRES positions (nk <= KRES / BK
// K-chunks), all of its chunks are loaded once per task at columns 32 kt, and only R streams
// through the two R stages. Otherwise L streams too, chunk c into columns 32 (c & 1).
//
// Chunk c of a task (tile c / nk, K-chunk c % nk) belongs to producer wave c % kProducers. That
// wave issues its global loads at iteration c - kProducers and writes it to LDS at iteration
// c - 1, so every load has kProducers - 1 iterations to arrive. Producers and consumers run
// separate loops with the same number of barriers per task (1 + nt * nk); the role is a
// wave-uniform scalar, so each wave branches over the other role's code.
// GATE only separates the two instances (dW1 and dW2) for profilers. RF: R is bf16 (0), MXFP8
// (8) or MXFP4 (4). BF: dW is stored as bf16.
template <bool ACC, bool GATE, int RF, bool BF>
__global__ void __launch_bounds__(kThreads, kWavesPerSimd) wgrad_kernel(const Args a,
                                                           const int4* __restrict__ table,
                                                           const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ count) {
  __shared__ __align__(16) uint16_t lbuf[BM * LDL];
  __shared__ __align__(16) uint16_t rbuf[2 * R_STAGE];
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const bool producer = wave >= kConsumers / kWave;
  const int pq = wave - kConsumers / kWave;  // producer index 0..kProducers-1
  const int wm = wave / (BN / 64), wn = wave % (BN / 64);  // consumer waves only
  const int ntasks = *count;
  const int G = gridDim.x, G8 = G / kXcds, xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;

  // Round r gives XCD x the contiguous task range [r G + x G/8, r G + (x+1) G/8), so tasks of
  // one expert (adjacent in the table) share that XCD's L2. Producers and consumers walk the
  // same tasks in separate loops, which keeps their register live ranges apart.
  // A task's tiles are its stripe's n-tiles [tfirst, tfirst + nt), taken rotated by rot: the
  // stripes of one expert run at the same time on one XCD, and without the rotation they would
  // all write the same columns of rows a stripe apart, which alias in HBM. The rotation is a
  // bijection of the stripe's tiles and changes no value.
  const int ntn = a.Ndim / BN;
  struct TaskInfo {
    int e, m0, nt, tfirst, rot, p0, p1, nk, total;
    bool resident;
    MOE_DEV int col(int j, int ntn) const {
      const int q = tfirst + j + rot;
      return (q < ntn ? q : q - ntn) * BN;
    }
  };
  auto task_at = [&](int ti) {
    const int4 task = table[ti];
    TaskInfo t;
    t.e = task.x;
    t.m0 = task.y;
    t.nt = task.w;
    t.tfirst = task.z;
    t.rot = (5 * (task.y / BM) + 3 * task.x) % ntn;
    t.p0 = offsets[t.e];
    t.p1 = offsets[t.e + 1];
    t.nk = (t.p1 - t.p0 + BK - 1) / BK;
    t.resident = t.nk <= KRES / BK;
    t.total = t.nt * t.nk;
    return t;
  };

  if (producer) {
    for (int round = 0;; ++round) {
      const int ti = round * G + xcd * G8 + slot;
      if (ti >= ntasks) break;
      const TaskInfo t = task_at(ti);
      if (t.nk == 0) continue;
      const int p0 = t.p0, p1 = t.p1, nk = t.nk, total = t.total;
      const bool resident = t.resident;
      Mover<BM / 64> ml;
      Mover<BN / 64> mr;
      ml.base = a.L + t.m0;
      ml.ld = a.Mdim;
      mr.base = a.R;
      mr.base8 = a.R8;
      mr.sc8 = a.R8s;
      mr.ld = a.Ndim;
      if (resident) {
        for (int kt = pq; kt < nk; kt += kProducers) {
          ml.load(p0 + kt * BK, p1, 0, lane);
          ml.store(lbuf, LDL, kt * BK, lane);
        }
      }
      // chunk pq: loads now; chunk 0 is written before the first barrier
      if (pq < total) {
        const int pb = p0 + (pq % nk) * BK;
        mr.load<RF>(pb, p1, t.col(pq / nk, ntn), lane);
        if (!resident) ml.load(pb, p1, 0, lane);
        if (pq == 0) {
          mr.store<RF>(rbuf, LDR, 0, lane);
          if (!resident) ml.store(lbuf, LDL, 0, lane);
        }
      }
      lds_barrier();
      for (int it = 0; it < total; ++it) {
        const int c = it + 1;
        if (c < total && c % kProducers == pq) {  // its loads were issued kProducers - 1 ago
          mr.store<RF>(rbuf + (c & 1) * R_STAGE, LDR, 0, lane);
          if (!resident) ml.store(lbuf, LDL, (c & 1) * BK, lane);
        }
        const int cn = it + kProducers;
        if (it % kProducers == pq && cn < total) {
          const int pb = p0 + (cn % nk) * BK;
          mr.load<RF>(pb, p1, t.col(cn / nk, ntn), lane);
          if (!resident) ml.load(pb, p1, 0, lane);
        }
        lds_barrier();
      }
    }
  } else {
    const int koff = (lane / 16) * 8;
    for (int round = 0;; ++round) {
      const int ti = round * G + xcd * G8 + slot;
      if (ti >= ntasks) break;
      const TaskInfo t = task_at(ti);
      const int nk = t.nk, total = t.total;
      const bool resident = t.resident;
      const size_t out = ((size_t)t.e * a.Mdim + t.m0) * a.Ndim;
      f32x4 acc[MBW][4];
#pragma unroll
      for (int i = 0; i < MBW; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][q] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (nk == 0) {  // an expert with no rows: its dW block is zero
        if (!ACC)
          for (int j = 0; j < t.nt; ++j) store_tile<false, BF>(a, out, t.col(j, ntn), acc);
        continue;
      }
      lds_barrier();
      int j = 0, kt = 0;
      for (int it = 0; it < total; ++it) {
        const uint16_t* rs = rbuf + (it & 1) * R_STAGE;
        const int lcol = (resident ? kt : (it & 1)) * BK + koff;
        uint4 bf[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          bf[nb] = *reinterpret_cast<const uint4*>(rs + (wn * 64 + nb * 16 + lane % 16) * LDR + koff);
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) {
          const uint4 af =
              *reinterpret_cast<const uint4*>(lbuf + (wm * WMR + mb * 16 + lane % 16) * LDL + lcol);
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma16(bf[nb], af, acc[mb][nb]);
        }
        if (kt == nk - 1) {
          store_tile<ACC, BF>(a, out, t.col(j, ntn), acc);
#pragma unroll
          for (int i = 0; i < MBW; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[i][q] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if (++kt == nk) {
          kt = 0;
          ++j;
        }
        lds_barrier();
      }
    }
  }
}

// Task table for one weight gradient, built by one workgroup from the device offsets. Thread
// e handles expert e: its K-steps nk = max(ceil(c_e / BK), 1), its run length
// nt = min(ceil(kWgradTaskSteps / nk), ntn) tiles, and its tasks
// mstripes * ceil(ntn / nt). An expert with no rows only writes zeros; its runs are kEmptyRun
// tiles, so the zero fill spreads over the grid. Experts are laid out by decreasing row count
// (ties to the lower index), each expert's tasks stripe-major. count[0] receives the number of
// tasks.
// Experts with c_e >= big_rows get no tasks here: big[0].x receives their number and
// big[1 + i] = (expert, rows) their list in the same order (they hold the first ranks).
__global__ void __launch_bounds__(1024) wgrad_sched_kernel(const int32_t* __restrict__ offsets,
                                                           int E, int mstripes, int ntn,
                                                           int big_rows, int4* __restrict__ big,
                                                           int4* __restrict__ table,
                                                           int32_t* __restrict__ count) {
  __shared__ int cnt[1024];
  __shared__ int scan[1024];
  const int e = threadIdx.x;
  const int c = e < E ? offsets[e + 1] - offsets[e] : -1;
  const bool isbig = e < E && c >= big_rows;
  const int nbig = __syncthreads_count(isbig);
  cnt[e] = c;
  __syncthreads();
  int rank = e;
  int ntask = 0, nt = 1, nchunks = 0;
  if (e < E) {
    rank = 0;
    for (int j = 0; j < E; ++j) {
      const int cj = cnt[j];
      rank += (cj > c) || (cj == c && j < e);
    }
    if (!isbig) {
      const int nk = max((c + BK - 1) / BK, 1);
      nt = min(c == 0 ? kEmptyRun : (kWgradTaskSteps + nk - 1) / nk, ntn);
      nchunks = (ntn + nt - 1) / nt;
      ntask = mstripes * nchunks;
    }
  }
  scan[rank] = ntask;  // ranks of the E experts are a permutation of 0..E-1
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = rank >= off ? scan[rank - off] : 0;
    __syncthreads();
    scan[rank] += v;
    __syncthreads();
  }
  const int start = scan[rank] - ntask;
  for (int s = 0; s < mstripes && nchunks > 0; ++s)
    for (int ch = 0; ch < nchunks; ++ch)
      table[start + s * nchunks + ch] = make_int4(e, s * BM, ch * nt, min(nt, ntn - ch * nt));
  if (isbig) big[1 + rank] = make_int4(e, c, 0, 0);
  if (e == 0) big[0] = make_int4(nbig, 0, 0, 0);
  if (rank == 1023) count[0] = scan[1023];
}

// ------------------------------------------------------------------------------------------
// Experts with many rows. With thousands of positions per expert the product is MFMA-bound,
// and the kernel's rate follows the flops per byte its tiles load into LDS: 256 x 256 output
// tiles with 64-position K steps carry 128 flop/B, against 85 for the 256 x 128 stripes with
// 32-position steps above. They run on dma_kernel (dma.h): eight waves of 128 x 64 outputs, one
// workgroup per CU, operands loaded straight into LDS (L through two stages, R through three).
//
// Both operands are position-major, so a K step of either is 64 rows of 256 contiguous values,
// and both sit in LDS as they are in memory, with the 32-byte column groups of row k permuted
// by XOR with kmajor_swz(k); the MFMA fragments (8 consecutive positions of one row or column
// per lane) come from gfx950's transposing LDS read, so neither operand is transposed in
// registers. Each operand's buffer range ends at the expert's last position, so the rows of
// the last K step past it load as zeros.
struct WgBigArgs {
  const uint16_t* L;       // [T*k, Mdim]
  const uint16_t* R;       // [T*k, Ndim]
  void* dw;                // [E, Mdim, Ndim], fp32 or (BF) bf16
  const int4* big;         // count, then the listed experts (x = expert)
  const int32_t* offsets;
  int Mdim, Ndim;
};
struct WgBigTile {
  int e, m0, n0, p0, p1;
};

// Tiles of the listed experts, expert by expert in list order (decreasing rows); inside an
// expert, groups of four 256-row blocks take each 256-column block in turn. Round r gives XCD x
// the tiles [r G + x G/8, r G + (x+1) G/8): neighbouring tiles share operand panels in its L2.
// GATE only separates the two instances (dW1 and dW2) for profilers; BF stores dW as bf16.
template <bool ACC, bool GATE, bool BF>
struct DmaWgrad {
  using Args = WgBigArgs;
  using Tile = WgBigTile;
  static constexpr const char* kName = GATE ? "bwd_gate_wgrad_big" : "bwd_down_wgrad_big";
  static constexpr bool kAKmajor = true, kBKmajor = true;
  static constexpr bool kVoffStep = true, kRoundOrder = true;
  static MOE_DEV int ntiles(const Args& a) { return a.big[0].x * (a.Mdim / 256) * (a.Ndim / 256); }
  static MOE_DEV Tile decode(const Args& a, int ti) {
    const int ntm = a.Mdim / 256, ntn = a.Ndim / 256, tpe = ntm * ntn;
    Tile t;
    t.e = a.big[1 + ti / tpe].x;
    const int lt = ti % tpe;
    const int group = lt / (4 * ntn), mfirst = group * 4, gm = min(4, ntm - mfirst);
    const int rr = lt - mfirst * ntn;
    t.m0 = (mfirst + rr % gm) * 256;
    t.n0 = (rr / gm) * 256;
    t.p0 = a.offsets[t.e];
    t.p1 = a.offsets[t.e + 1];
    return t;
  }
  static MOE_DEV int brow(int, int) { return 0; }
  // byte offsets fit 32 bits: an expert has at most T positions, and T d, T 2I < 2^31 are API
  // limits
  static MOE_DEV void src(const Args& a, const Tile& t, int wave, int lane, DmaSrc& s) {
    const int rows = t.p1 - t.p0;
    s.nk = (rows + 63) / 64;
    s.k0 = 0;
    s.ra = raw_rsrc(a.L + (size_t)t.p0 * a.Mdim + t.m0, 2u * (uint32_t)rows * (uint32_t)a.Mdim);
    s.rb = raw_rsrc(a.R + (size_t)t.p0 * a.Ndim + t.n0, 2u * (uint32_t)rows * (uint32_t)a.Ndim);
    s.astep = 128u * (uint32_t)a.Mdim;
    s.bstep = 128u * (uint32_t)a.Ndim;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kr = dma_krow(wave, j, lane);
      s.ao[j] = 2u * (uint32_t)kr * (uint32_t)a.Mdim + dma_kpiece(kr, lane);
      s.bo[j] = 2u * (uint32_t)kr * (uint32_t)a.Ndim + dma_kpiece(kr, lane);
    }
  }
  static MOE_DEV void epilogue(const Args& a, const Tile& t, f32x4 (&acc)[8][4]) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int wm = wave / 4, wn = wave % 4;
    DwT<BF>* out =
        static_cast<DwT<BF>*>(a.dw) + ((size_t)t.e * a.Mdim + t.m0) * a.Ndim + t.n0;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const int m = wm * 128 + mb * 16 + lane % 16;
      if constexpr (BF) {
#pragma unroll
        for (int nb = 0; nb < 4; nb += 2)
          store_dw8_bf16<ACC>(out + (size_t)m * a.Ndim + wn * 64 + nb * 16, acc[mb][nb],
                              acc[mb][nb + 1], lane);
      } else {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int n = wn * 64 + nb * 16 + 4 * (lane / 16);
          store_dw4<ACC>(out + (size_t)m * a.Ndim + n, acc[mb][nb]);
        }
      }
    }
  }
};

// The exact bf16 image (codes times their scale, as Mover::expand makes it) of the rows of the
// listed big experts of an MX operand (F = 8: E4M3 codes; F = 4: E2M1 codes, two a byte), at
// the same row positions. One thread per 8-column piece, grid-stride over each expert's rows in
// turn.
template <int F>
__global__ void __launch_bounds__(256) expand_big_rows_kernel(const uint8_t* __restrict__ r8,
                                                              const uint8_t* __restrict__ r8s,
                                                              uint16_t* __restrict__ out,
                                                              const int4* __restrict__ big,
                                                              const int32_t* __restrict__ offsets,
                                                              int Ndim) {
  const int per_row = Ndim / 8;
  const int nbig = big[0].x;
  for (int i = 0; i < nbig; ++i) {
    const int e = big[1 + i].x;
    const int p0 = offsets[e];
    const long long n = (long long)(offsets[e + 1] - p0) * per_row;
    for (long long c = (long long)blockIdx.x * blockDim.x + threadIdx.x; c < n;
         c += (long long)gridDim.x * blockDim.x) {
      const size_t p = (size_t)p0 + (size_t)(c / per_row);
      const int col = (int)(c % per_row) * 8;
      uint4 raw = make_uint4(0, 0, r8s[p * (Ndim / 32) + col / 32], 0);
      if constexpr (F == 8) {
        const uint2 q = *reinterpret_cast<const uint2*>(r8 + p * Ndim + col);
        raw.x = q.x;
        raw.y = q.y;
      } else {
        raw.x = *reinterpret_cast<const uint32_t*>(r8 + p * (Ndim / 2) + col / 2);
      }
      *reinterpret_cast<uint4*>(out + p * Ndim + col) = Mover<1>::expand<F>(raw);
    }
  }
}

int resident_grid() {
  static int grid = 0;  // every device of one process is an MI355X
  if (grid == 0) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(&wgrad_kernel<false, false, 0, false>),
            kThreads, 0) != hipSuccess)
      return 0;
    grid = (cus * (per_cu > 0 ? per_cu : 1)) / kXcds * kXcds;
  }
  return grid;
}

}  // namespace

// Entries: the list of big experts (1 + E), then the task table of the others.
size_t wgrad_table_entries(int Tk, int E, int Mdim, int Ndim) {
  const long long mstripes = Mdim / BM, ntn = Ndim / BN;
  const long long per_stripe = ntn * ((long long)Tk + (long long)E * BK) / (BK * kWgradTaskSteps) + E +
                               (long long)E * ((ntn + kEmptyRun - 1) / kEmptyRun);
  const long long cap = (long long)E * ntn;
  return (size_t)(1 + E + mstripes * (per_stripe < cap ? per_stripe : cap));
}

hipError_t launch_wgrad(const WgradArgs& x, hipStream_t s) {
  // the big-expert kernel takes bf16 operands whose dW dimensions are multiples of its tile; an
  // MX R needs the scratch for its bf16 image
  const bool big_ok = (!x.R8 || x.Rx) && x.Mdim % 256 == 0 && x.Ndim % 256 == 0;
  const int big_rows = big_ok ? kWgradBigRows : 0x7fffffff;
  int4* big = x.table;
  int4* table = x.table + 1 + x.E;
  {
    TraceScope trace(x.name_sched, s);
    hipLaunchKernelGGL(wgrad_sched_kernel, dim3(1), dim3(1024), 0, s, x.offsets, x.E, x.Mdim / BM,
                       x.Ndim / BN, big_rows, big, table, x.count);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int grid = resident_grid();
  if (grid <= 0) return hipErrorInvalidValue;
  Args a{x.L, x.R, x.R8, x.R8s, x.dw, x.offsets, table, x.count, x.Mdim, x.Ndim, x.accumulate};
  {
    TraceScope trace(x.name, s);
    using K = void (*)(const Args, const int4*, const int32_t*, const int32_t*);
    // [accumulate][gate][R: bf16, E4M3, E2M1][bf16 dW]; an MX R comes with the gate wgrad only
    static const K kernels[2][2][3][2] = {
        {{{wgrad_kernel<false, false, 0, false>, wgrad_kernel<false, false, 0, true>},
          {nullptr, nullptr},
          {nullptr, nullptr}},
         {{wgrad_kernel<false, true, 0, false>, wgrad_kernel<false, true, 0, true>},
          {wgrad_kernel<false, true, 8, false>, wgrad_kernel<false, true, 8, true>},
          {wgrad_kernel<false, true, 4, false>, wgrad_kernel<false, true, 4, true>}}},
        {{{wgrad_kernel<true, false, 0, false>, wgrad_kernel<true, false, 0, true>},
          {nullptr, nullptr},
          {nullptr, nullptr}},
         {{wgrad_kernel<true, true, 0, false>, wgrad_kernel<true, true, 0, true>},
          {wgrad_kernel<true, true, 8, false>, wgrad_kernel<true, true, 8, true>},
          {wgrad_kernel<true, true, 4, false>, wgrad_kernel<true, true, 4, true>}}}};
    if (x.R8 && x.rbits != 8 && x.rbits != 4) return hipErrorInvalidValue;
    const int rf = x.R8 ? (x.rbits == 8 ? 1 : 2) : 0;
    const K kern = kernels[x.accumulate ? 1 : 0][x.gate ? 1 : 0][rf][x.bf16_dw ? 1 : 0];
    if (!kern) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), 0, s, a, table, x.offsets, x.count);
  }
  err = hipGetLastError();
  if (err != hipSuccess || !big_ok) return err;
  if (x.R8) {
    TraceScope trace("bwd_gate_wgrad_expand", s);
    if (x.rbits == 4)
      hipLaunchKernelGGL(expand_big_rows_kernel<4>, dim3(1024), dim3(256), 0, s, x.R8, x.R8s,
                         x.Rx, big, x.offsets, x.Ndim);
    else
      hipLaunchKernelGGL(expand_big_rows_kernel<8>, dim3(1024), dim3(256), 0, s, x.R8, x.R8s,
                         x.Rx, big, x.offsets, x.Ndim);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // the big experts' tile count is known on the device only: a resident grid walks it
  const WgBigArgs ab{x.L, x.R8 ? x.Rx : x.R, x.dw, big, x.offsets, x.Mdim, x.Ndim};
  constexpr int kAnyTiles = 1 << 30;
  if (x.bf16_dw) {
    if (x.accumulate)
      return x.gate ? launch_dma<DmaWgrad<true, true, true>>(ab, kAnyTiles, true, s)
                    : launch_dma<DmaWgrad<true, false, true>>(ab, kAnyTiles, true, s);
    return x.gate ? launch_dma<DmaWgrad<false, true, true>>(ab, kAnyTiles, true, s)
                  : launch_dma<DmaWgrad<false, false, true>>(ab, kAnyTiles, true, s);
  }
  if (x.accumulate)
    return x.gate ? launch_dma<DmaWgrad<true, true, false>>(ab, kAnyTiles, true, s)
                  : launch_dma<DmaWgrad<true, false, false>>(ab, kAnyTiles, true, s);
  return x.gate ? launch_dma<DmaWgrad<false, true, false>>(ab, kAnyTiles, true, s)
                : launch_dma<DmaWgrad<false, false, false>>(ab, kAnyTiles, true, s);
}

}  // namespace moe
