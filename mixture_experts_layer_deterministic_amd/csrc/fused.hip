// The layer's forward in one launch: router, permutation into the ring slot, both grouped
// GEMMs and the combine, as phases of one persistent kernel separated by grid-wide barriers.
//
// The pages describe one persistent kernel that fuses every step of the MoE layer (MarkTechPost,
// "Cursor Open-Sources Mixture-of-Kittens (MoK)": introduction and the closing paragraph of
// "Three design decisions that matter"; toknow.ai summary). Their design schedules that kernel
// with Blackwell hardware that CDNA has no equivalent of; here the grid is launched
// cooperatively (every workgroup resident at once) and the phases meet at barriers on a counter
// in device memory. Where a layer is small its separate launches cost more than its work, and
// one launch removes the gaps between them.
//
// Each phase runs the same device code as the separate kernels (router.h, permute.h,
// gemm_tiles.h, combine.h) over virtual block indices, so every value equals theirs. The one
// difference is the tiling of the grouped GEMMs: all row blocks take the 128 x 128 tile here,
// where moe_forward gives full 256-row blocks the 256 x 256 kernel (dma.h); the down
// projection then starts its K loop at another chunk for those rows, so outputs of experts with
// 256 rows or more agree to rounding rather than bit for bit.
#include <algorithm>

#include "combine.h"
#include "common.h"
#include "gemm_tiles.h"
#include "kernels.h"
#include "moe.h"
#include "permute.h"
#include "router.h"

namespace moe {

namespace {

constexpr int kFusedThreads = 256;
constexpr int kRouterWaves = kFusedThreads / kWave;  // experts per router block
constexpr unsigned kBarrierSpins = 1u << 21;         // about two seconds of waiting

// Barrier state, one per GPU, zero when the code object loads; every completed barrier leaves
// the counters at zero again. The workgroups arrive in kBarrierGroups groups (workgroup b in
// group b % kBarrierGroups), each on a counter of its own, and the last of each group arrives
// on the top counter: no counter takes more than n / kBarrierGroups arrivals, so the atomics,
// which one memory channel serialises per address, spread over kBarrierGroups + 1 addresses.
// Every field sits in its own 256-byte line, and the generation that the waiting workgroups
// poll in yet another, so the polls do not queue behind the arrivals.
constexpr int kBarrierGroups = 8;
struct alignas(256) BarrierWord {
  unsigned v;
};
struct GridBarrier {
  BarrierWord group[kBarrierGroups];
  BarrierWord top;
  BarrierWord gen;
};
static __device__ GridBarrier fused_barrier;
static_assert(kXcds % kBarrierGroups == 0, "the grid is a multiple of kXcds workgroups");

// All `n` workgroups of the grid meet here (n a multiple of kBarrierGroups). Each arrival is
// an acquire-release atomic: thread 0 of a workgroup releases its workgroup's writes (they
// leave the XCD's L2 for memory), and the last arrival of a group acquires the group's writes
// before it releases them again on the top counter. The last arrival there starts the next
// generation; the others poll the generation with relaxed loads and leave with one acquire
// fence (an acquire on every poll would invalidate the L2 each time, under the feet of the
// workgroups still working). So every write before the barrier is visible to every read after
// it, across the XCDs' L2 caches. A workgroup that waits longer than kBarrierSpins polls gives
// up, marks *status and goes on, so the kernel always ends.
MOE_DEV void grid_sync(GridBarrier* b, unsigned n, int32_t* status) {
  __syncthreads();
  if (threadIdx.x == 0) {
    // gen cannot move before this workgroup arrives, and this thread saw its last change
    const unsigned g = __hip_atomic_load(&b->gen.v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    BarrierWord* grp = &b->group[blockIdx.x % kBarrierGroups];
    bool done = false;
    if (__hip_atomic_fetch_add(&grp->v, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) + 1 ==
        n / kBarrierGroups) {
      __hip_atomic_store(&grp->v, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__hip_atomic_fetch_add(&b->top.v, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) + 1 ==
          (unsigned)kBarrierGroups) {
        __hip_atomic_store(&b->top.v, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&b->gen.v, g + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        done = true;
      }
    }
    if (!done) {
      unsigned spins = 0;
      while (__hip_atomic_load(&b->gen.v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == g) {
        __builtin_amdgcn_s_sleep(2);
        if (++spins == kBarrierSpins) {
          atomicOr(status, MOE_DEVICE_BARRIER_TIMEOUT);
          break;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
  }
  __syncthreads();
}

// Exclusive scan over the experts, run by one workgroup of kFusedThreads threads: thread i
// owns the four consecutive experts 4i .. 4i + 3 (E <= 1024) and passes their values v; excl
// receives their exclusive prefixes and *total the sum. sh: 256 ints of LDS.
MOE_DEV void scan4(const int (&v)[4], int (&excl)[4], int* total, int* sh) {
  const int tid = threadIdx.x;
  int local[4];
  int s = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    local[q] = s;
    s += v[q];
  }
  sh[tid] = s;
  __syncthreads();
  for (int off = 1; off < kFusedThreads; off <<= 1) {
    const int u = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += u;
    __syncthreads();
  }
  const int before = sh[tid] - s;
#pragma unroll
  for (int q = 0; q < 4; ++q) excl[q] = before + local[q];
  *total = sh[kFusedThreads - 1];
  __syncthreads();
}

// The i-th GEMM tile of workgroup b, dealt as the separate grouped-GEMM kernels deal them: XCD
// x = b % 8 takes the contiguous tile range [x R, (x + 1) R), R = ceil(nt / 8), so workgroups
// sharing an expert's activation rows share that XCD's L2. -1 when b has no i-th tile.
MOE_DEV int xcd_tile(int b, int G, int nt, int i) {
  const int R = (nt + kXcds - 1) / kXcds;
  const int s = b / kXcds + i * (G / kXcds);
  if (s >= R) return -1;
  const int lt = (b % kXcds) * R + s;
  return lt < nt ? lt : -1;
}

}  // namespace

__global__ void __launch_bounds__(kFusedThreads, 2) fused_forward_kernel(const FusedFwdParams p) {
  extern __shared__ __align__(16) uint16_t smem[];
  int* ish = reinterpret_cast<int*>(smem);
  GridBarrier* bar = &fused_barrier;
  const unsigned nwg = gridDim.x;
  const int G = gridDim.x, b0 = blockIdx.x, tid = threadIdx.x;
  const int T = p.T, d = p.d, E = p.E, k = p.k, I = p.I, Tk = T * k;

  // 0. the device status word starts clear (the scan below adds the bad-index bit)
  if (b0 == 0 && tid == 0) p.status[0] = 0;
  // 1. the router weight widened to fp32 (exact)
  {
    const long long n4 = (long long)E * d / 4;
    for (long long i = (long long)b0 * kFusedThreads + tid; i < n4; i += (long long)G * kFusedThreads)
      widen_router_item(p.wr, p.w32, i * 4);
  }
  grid_sync(bar, nwg, p.status);
  // 2. logits: blocks of 64 tokens x 4 experts
  {
    const int nbx = (T + kWave - 1) / kWave, nby = (E + kRouterWaves - 1) / kRouterWaves;
    for (int vb = b0; vb < nbx * nby; vb += G) {
      router_logits_block<kRouterWaves>(vb % nbx, vb / nbx, p.x, p.w32, p.logits, T, d, E, smem);
      __syncthreads();  // the next block's first stage reuses the LDS
    }
  }
  grid_sync(bar, nwg, p.status);
  // 3. top-k: one wave per token
  {
    const int wave = tid / kWave;
    for (int t = b0 * kRouterWaves + wave; t < T; t += G * kRouterWaves)
      router_topk_token(t, p.logits, E, k, p.topk_idx, p.topk_w);
  }
  grid_sync(bar, nwg, p.status);
  // 4. per-block expert histograms and in-block ranks
  for (int vb = b0; vb < p.nb; vb += G) {
    perm_hist_block(vb, p.topk_idx, Tk, E, p.blk_cnt, p.rank, p.blk_flag, ish, ish + kPermRows);
    __syncthreads();
  }
  grid_sync(bar, nwg, p.status);
  // 5. one workgroup: expert totals, offsets and per-block bases (the scan of permute.hip);
  // then the 128-row block table of every expert (moe_forward's sched_build, full table)
  if (b0 == 0) {
    int tot[4], excl[4], total;
    int flag = 0;
    for (int b = tid; b < p.nb; b += kFusedThreads) flag |= p.blk_flag[b];
    flag = __syncthreads_or(flag);
    constexpr int U = 16;  // block counts loaded together before their running sum
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * tid + q;
      int run = 0;
      if (e < E)
        for (int bs = 0; bs < p.nb; bs += U) {
          int c[U];
#pragma unroll
          for (int u = 0; u < U; ++u) c[u] = bs + u < p.nb ? p.blk_cnt[(size_t)(bs + u) * E + e] : 0;
#pragma unroll
          for (int u = 0; u < U; ++u) {
            if (bs + u < p.nb) p.blk_cnt[(size_t)(bs + u) * E + e] = run;
            run += c[u];
          }
        }
      tot[q] = e < E ? run : 0;
    }
    scan4(tot, excl, &total, ish);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * tid + q;
      if (e >= E) continue;
      p.counts[e] = tot[q];
      p.offsets[e] = excl[q];
      for (int bs = 0; bs < p.nb; bs += U) {
        int c[U];
#pragma unroll
        for (int u = 0; u < U; ++u) c[u] = bs + u < p.nb ? p.blk_cnt[(size_t)(bs + u) * E + e] : 0;
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (bs + u < p.nb) p.blk_cnt[(size_t)(bs + u) * E + e] = c[u] + excl[q];
      }
    }
    if (tid == 0) {
      p.offsets[E] = total;
      if (flag) atomicOr(p.status, MOE_DEVICE_BAD_EXPERT_INDEX);
    }
    int nfull[4], first[4], ntot;
#pragma unroll
    for (int q = 0; q < 4; ++q) nfull[q] = (tot[q] + kSchedBM - 1) / kSchedBM;
    scan4(nfull, first, &ntot, ish);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      for (int i = 0; i < nfull[q]; ++i)
        p.sched[1 + first[q] + i] = mtile_entry(4 * tid + q, excl[q] + i * kSchedBM,
                                                min(kSchedBM, tot[q] - i * kSchedBM));
    if (tid == 0) p.sched[0] = make_int2(ntot, 0);
  }
  grid_sync(bar, nwg, p.status);
  // 6. placement of every row and the copy of its token into the ring slot
  for (int vb = b0; vb * p.tpb < T; vb += G) {
    perm_place_block<0>(vb, p.topk_idx, p.rank, p.blk_cnt, T, E, k, p.row_src, p.tk_row, p.x,
                            p.xp, nullptr, nullptr, d, p.tpb, ish);
    __syncthreads();
  }
  grid_sync(bar, nwg, p.status);
  // 7. gate/up GEMM with the SwiGLU epilogue
  {
    const FwdGateUp::Args a{p.xp, p.w1, p.H, p.A, p.offsets, p.sched, d, I};
    const int nt = FwdGateUp::ntiles(a);
    for (int i = 0, lt; (lt = xcd_tile(b0, G, nt, i)) >= 0; ++i)
      run_tile<FwdGateUp>(a, FwdGateUp::decode(a, lt), smem);
  }
  grid_sync(bar, nwg, p.status);
  // 8. down GEMM
  {
    const FwdDown::Args a{p.A, p.w2, p.O, p.offsets, p.sched, d, I};
    const int nt = FwdDown::ntiles(a);
    for (int i = 0, lt; (lt = xcd_tile(b0, G, nt, i)) >= 0; ++i)
      run_tile<FwdDown>(a, FwdDown::decode(a, lt), smem);
  }
  grid_sync(bar, nwg, p.status);
  // 9. combine
  {
    const int n = T * (d / 8);
    const bool wt = (d / 8) % kWave == 0;
    for (int i = b0 * kFusedThreads + tid; i < n; i += G * kFusedThreads) {
      if (wt)
        combine_slice<true>(i, p.O, p.tk_row, p.topk_w, k, d, p.y);
      else
        combine_slice<false>(i, p.O, p.tk_row, p.topk_w, k, d, p.y);
    }
  }
}

// The grid: the resident workgroups (two per CU), but no more than the largest phase needs, a
// multiple of 8.
hipError_t launch_fused_forward(const FusedFwdParams& p, hipStream_t s) {
  static int resident = 0;  // every device of one process is an MI355X
  constexpr size_t smem = GeoSmall::kSmem;
  if (resident == 0) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&fused_forward_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    int dev = 0, cus = 0, per_cu = 0;
    if (e == hipSuccess) e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(&fused_forward_kernel), kFusedThreads, smem);
    if (e != hipSuccess) return e;
    resident = cus * (per_cu > 0 ? per_cu : 1) / kXcds * kXcds;
  }
  const long long Tk = (long long)p.T * p.k;
  const long long mt = sched_max_mtiles((int)Tk, p.E);
  long long need = std::max({mt * (p.I / 64), mt * (p.d / 128),
                             (long long)((p.T + kWave - 1) / kWave) * ((p.E + 3) / 4),
                             (long long)p.nb, (long long)p.T * (p.d / 8) / kFusedThreads + 1});
  int grid = (int)std::min<long long>(resident, (need + kXcds - 1) / kXcds * kXcds);
  if (grid < kXcds) grid = kXcds;
  FusedFwdParams copy = p;
  void* args[] = {&copy};
  TraceScope trace("fused_forward", s);
  hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&fused_forward_kernel),
                                            dim3(grid), dim3(kFusedThreads), args, smem, s);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace moe
