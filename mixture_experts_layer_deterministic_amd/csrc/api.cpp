// C ABI of the MoE layer: argument checks, buffer layout and launch sequences.
// Every call checks its arguments on the host, then enqueues its kernels on the caller's
// stream. It never allocates, synchronises or prints.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>

#include "moe.h"
#include "kernels.h"

namespace {

using namespace moe;
static_assert(MOE_STATIC_SCRATCH_BYTES == kStaticPermScratchBytes, "one size in both places");

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  bool mx;
  int fb;  // MX code bits: 8 (MXFP8) or 4 (MXFP4); 0 in BF16 mode
  // workspace
  size_t status, sched, blk_cnt, blk_flag, rank, O, dH, dXp, dyw, dwpart, dl_pos, wg_count,
      wg_table1, wg_table2, wr32, total;
  // workspace, MX modes only: dY, A and dH quantised along their GEMM's K (codes, scales)
  size_t dyq, dys, aq, aqs, dhq, dhs;
  // workspace, MXFP8 weight gradients only: padded segment offsets [E + 1], and the two
  // operands of one weight gradient quantised along the positions, [rows][P] with scales
  size_t poff, lq, lqs, rq, rqs;
  int P;
  // saved
  size_t H, A, saved_total;
  // ring slot: bf16 Xp, or MX Xp codes at 0 and scales at slot_sc
  size_t slot, slot_sc;
  // quantised weights (MX): W1 and W2 along their forward K, and transposed along their
  // dgrad K: W1f [E,2I,d], W2f [E,d,I], W2b [E,I,d], W1b [E,d,2I], each with per-32 scales
  size_t w1f, w1fs, w2f, w2fs, w2b, w2bs, w1b, w1bs, wq_total;
  int nb, nIt, max_mtiles;
};

bool cfg_ok(const moe_cfg* c) {
  if (!c) return false;
  if (c->T < 1 || c->d < 256 || c->d % 256 != 0 || c->I < 128 || c->I % 128 != 0) return false;
  if (c->E < 1 || c->E > 1024 || c->k < 1 || c->k > c->E || c->k > kMaxTopK) return false;
  const long long T = c->T, d = c->d, I = c->I, Tk = T * c->k;
  if (Tk >= (1LL << 31) || T * c->E >= (1LL << 31)) return false;
  // The kernels address rows with 32-bit offsets. Element offsets into X and dY, and byte
  // offsets into one expert's rows of Xp, dXp, dYw, H, A and dH: a caller's routing may send
  // every row to one expert (a token may even repeat an expert), so an expert has up to T*k
  // rows. Byte offsets into one expert's weights: W1[e] is 2I x d bf16.
  if (T * d >= (1LL << 31)) return false;
  if (Tk * d >= (1LL << 31) || Tk * 2 * I >= (1LL << 31)) return false;
  if (4 * I * d >= (1LL << 31)) return false;
  return true;
}

// The kernels are built for gfx950 only. The current device's architecture is read once per
// device and kept.
int check_device() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> arch_seen[kMaxDev];  // 0 unknown, 1 gfx950, 2 another device
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return MOE_ERR_HIP;
  }
  if (dev < kMaxDev) {
    const int v = arch_seen[dev].load(std::memory_order_relaxed);
    if (v) return v == 1 ? MOE_OK : MOE_ERR_UNSUPPORTED;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return MOE_ERR_HIP;
  }
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
                  (prop.gcnArchName[6] == 0 || prop.gcnArchName[6] == ':');
  if (dev < kMaxDev) arch_seen[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? MOE_OK : MOE_ERR_UNSUPPORTED;
}

Layout layout(const moe_cfg* c) {
  Layout L{};
  const size_t Tk = (size_t)c->T * c->k, d = c->d, I = c->I, E = c->E;
  L.nb = (int)((Tk + kPermRows - 1) / kPermRows);
  L.nIt = c->I / kDgradBN;
  L.max_mtiles = sched_max_mtiles((int)Tk, c->E);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  L.status = take(16);
  L.sched = take(sizeof(int2) * sched_entries((int)Tk, (int)E));
  L.blk_cnt = take(sizeof(int32_t) * (size_t)L.nb * E);
  L.blk_flag = take(sizeof(int32_t) * (size_t)L.nb);
  L.rank = take(sizeof(int32_t) * Tk);
  L.O = take(2 * Tk * d);
  L.dH = take(2 * Tk * 2 * I);
  L.dXp = take(2 * Tk * d);
  L.dyw = take(2 * Tk * d);
  L.wg_count = take(2 * sizeof(int32_t));
  L.wg_table1 = take(16 * wgrad_table_entries((int)Tk, c->E, 2 * c->I, c->d));
  L.wg_table2 = take(16 * wgrad_table_entries((int)Tk, c->E, c->d, c->I));
  L.dwpart = take(sizeof(float) * Tk * L.nIt);
  L.dl_pos = take(sizeof(float) * Tk);
  L.wr32 = take(sizeof(float) * E * d);
  L.mx = c->precision == MOE_PREC_MXFP8 || c->precision == MOE_PREC_MXFP4;
  L.fb = c->precision == MOE_PREC_MXFP8 ? 8 : c->precision == MOE_PREC_MXFP4 ? 4 : 0;
  const size_t T = c->T, mxs = L.mx ? 1 : 0;
  // bytes of n codes
  auto cb = [&](size_t n) { return n * L.fb / 8; };
  L.dyq = take(mxs * cb(T * d));
  L.dys = take(mxs * T * d / 32);
  L.aq = take(mxs * cb(Tk * I));
  L.aqs = take(mxs * Tk * I / 32);
  L.dhq = take(mxs * cb(Tk * 2 * I));
  L.dhs = take(mxs * Tk * 2 * I / 32);
  const size_t mxw = L.mx && (c->flags & MOE_FLAG_MXFP8_WGRAD) ? 1 : 0;
  L.P = mxw ? seg_capacity((int)Tk, c->E) : 0;
  const size_t P = L.P, lrows = std::max(2 * I, d), rrows = std::max(d, I);
  L.poff = take(mxw * sizeof(int32_t) * (E + 1));
  L.lq = take(lrows * P);
  L.lqs = take(lrows * P / 32);
  L.rq = take(rrows * P);
  L.rqs = take(rrows * P / 32);
  L.total = o;
  o = 0;
  L.H = take(2 * Tk * 2 * I);
  L.A = take(2 * Tk * I);
  L.saved_total = o;
  if (L.mx) {
    o = 0;
    take(cb(Tk * d));
    L.slot_sc = o;
    take(Tk * d / 32);
    L.slot = o;
    o = 0;
    L.w1f = take(cb(E * 2 * I * d));
    L.w1fs = take(E * 2 * I * d / 32);
    L.w2f = take(cb(E * d * I));
    L.w2fs = take(E * d * I / 32);
    L.w2b = take(cb(E * I * d));
    L.w2bs = take(E * I * d / 32);
    L.w1b = take(cb(E * d * 2 * I));
    L.w1bs = take(E * d * 2 * I / 32);
    L.wq_total = o;
  } else {
    L.slot = 2 * Tk * d;
  }
  return L;
}

bool aligned16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) % 16) == 0; }
bool aligned4(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) % 4) == 0; }

template <class T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}
template <class T>
const T* at(const void* base, size_t off) {
  return reinterpret_cast<const T*>(static_cast<const char*>(base) + off);
}

// First error wins; later launches are skipped once one fails.
struct Launches {
  hipError_t err = hipSuccess;
  void operator()(hipError_t e) {
    if (err == hipSuccess) err = e;
  }
  int status() const { return err == hipSuccess ? MOE_OK : MOE_ERR_HIP; }
};

int check_mode(const moe_cfg* c) {
  if (!cfg_ok(c)) return MOE_ERR_INVALID_ARG;
  if (c->precision != MOE_PREC_BF16 && c->precision != MOE_PREC_MXFP8 &&
      c->precision != MOE_PREC_MXFP4)
    return MOE_ERR_UNSUPPORTED;
  if (c->precision == MOE_PREC_MXFP4 && c->I % 256 != 0) return MOE_ERR_INVALID_ARG;
  if (c->flags & ~(MOE_FLAG_PERSISTENT | MOE_FLAG_MXFP8_WGRAD | MOE_FLAG_BF16_DW))
    return MOE_ERR_INVALID_ARG;
  if ((c->flags & MOE_FLAG_MXFP8_WGRAD) && c->precision != MOE_PREC_MXFP8)
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

int check_ring(const Layout& L, const void* ring, size_t ring_bytes, int32_t slot) {
  if (!aligned16(ring)) return MOE_ERR_INVALID_ARG;
  if (slot < 0 || (size_t)(slot + 1) * L.slot > ring_bytes) return MOE_ERR_RING_TOO_SMALL;
  return MOE_OK;
}

// The quantised weights of the MX modes, or an error code when they are missing.
int check_wq(const Layout& Y, const void* wq, size_t wq_bytes) {
  if (!Y.mx) return MOE_OK;
  if (!aligned16(wq)) return MOE_ERR_INVALID_ARG;
  if (wq_bytes < Y.wq_total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return MOE_OK;
}

// Launch tracing (moe_trace_begin / moe_trace_end).
std::atomic<void* const*> g_trace_events{nullptr};
std::mutex g_trace_mu;
const char** g_trace_names = nullptr;
int g_trace_cap = 0;
int g_trace_count = 0;

}  // namespace

namespace moe {
void trace_pre(const char* name, hipStream_t s) {
  if (!g_trace_events.load(std::memory_order_acquire)) return;
  std::lock_guard<std::mutex> lk(g_trace_mu);
  void* const* ev = g_trace_events.load(std::memory_order_relaxed);
  const int i = g_trace_count;
  if (ev && 2 * i + 1 < g_trace_cap) {
    (void)hipEventRecord(static_cast<hipEvent_t>(ev[2 * i]), s);
    if (g_trace_names) g_trace_names[i] = name;
  }
}
void trace_post(hipStream_t s) {
  if (!g_trace_events.load(std::memory_order_acquire)) return;
  std::lock_guard<std::mutex> lk(g_trace_mu);
  void* const* ev = g_trace_events.load(std::memory_order_relaxed);
  const int i = g_trace_count++;
  if (ev && 2 * i + 1 < g_trace_cap) (void)hipEventRecord(static_cast<hipEvent_t>(ev[2 * i + 1]), s);
}
}  // namespace moe

extern "C" {

int moe_trace_begin(void* const* events, int capacity, const char** names) {
  if (!events || capacity < 2) return MOE_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(g_trace_mu);
  g_trace_names = names;
  g_trace_cap = capacity;
  g_trace_count = 0;
  g_trace_events.store(events, std::memory_order_release);
  return MOE_OK;
}

int moe_trace_end(void) {
  std::lock_guard<std::mutex> lk(g_trace_mu);
  g_trace_events.store(nullptr, std::memory_order_release);
  const int n = g_trace_count;
  g_trace_count = 0;
  g_trace_cap = 0;
  g_trace_names = nullptr;
  return n;
}

int moe_query(const moe_cfg* cfg, moe_sizes* out) {
  if (!out) return MOE_ERR_INVALID_ARG;
  if (const int st = check_mode(cfg)) return st;
  const Layout L = layout(cfg);
  out->ring_slot = L.slot;
  out->saved = L.saved_total;
  out->saved_H = L.H;
  out->saved_A = L.A;
  out->workspace = L.total;
  out->ws_O = L.O;
  out->ws_dH = L.dH;
  out->ws_dXp = L.dXp;
  out->wq = L.mx ? L.wq_total : 0;
  return MOE_OK;
}

int moe_quantize_weights(const moe_cfg* cfg, const void* w1, const void* w2, void* wq,
                         size_t wq_bytes, moe_stream_t stream) {
  int st = check_mode(cfg);
  if (st) return st;
  const Layout Y = layout(cfg);
  if (!Y.mx) return MOE_ERR_INVALID_ARG;
  if (!aligned16(w1) || !aligned16(w2) || !aligned16(wq)) return MOE_ERR_INVALID_ARG;
  if (wq_bytes < Y.wq_total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if ((st = check_device())) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int E = cfg->E, d = cfg->d, I = cfg->I;
  const uint16_t* a1 = static_cast<const uint16_t*>(w1);
  const uint16_t* a2 = static_cast<const uint16_t*>(w2);
  Launches L;
  L(launch_quant_weight(a1, E, 2 * I, d, at<uint8_t>(wq, Y.w1f), at<uint8_t>(wq, Y.w1fs),
                        at<uint8_t>(wq, Y.w1b), at<uint8_t>(wq, Y.w1bs), Y.fb, "quant_w1", s));
  if (!L.err)
    L(launch_quant_weight(a2, E, d, I, at<uint8_t>(wq, Y.w2f), at<uint8_t>(wq, Y.w2fs),
                          at<uint8_t>(wq, Y.w2b), at<uint8_t>(wq, Y.w2bs), Y.fb, "quant_w2", s));
  return L.status();
}

int moe_route(const moe_cfg* cfg, const void* x, const void* w_router, float* logits,
              int32_t* topk_idx, float* topk_w, void* workspace, size_t ws_bytes,
              moe_stream_t stream) {
  int st = check_mode(cfg);
  if (st) return st;
  if (!aligned16(x) || !aligned16(w_router) || !aligned4(logits) || !aligned4(topk_idx) ||
      !aligned4(topk_w) || !aligned16(workspace))
    return MOE_ERR_INVALID_ARG;
  const Layout Y = layout(cfg);
  if (ws_bytes < Y.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if ((st = check_device())) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Launches L;
  L(launch_router_logits(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_router),
                         at<float>(workspace, Y.wr32), logits, cfg->T, cfg->d, cfg->E, s));
  if (L.err == hipSuccess)
    L(launch_router_topk(logits, cfg->T, cfg->E, cfg->k, topk_idx, topk_w, s));
  return L.status();
}

int moe_permute(const moe_cfg* cfg, const int32_t* topk_idx, const void* x, void* ring,
                size_t ring_bytes, int32_t slot, int32_t* counts, int32_t* offsets,
                int32_t* row_src, int32_t* tk_row, void* workspace, size_t ws_bytes,
                moe_stream_t stream) {
  int st = check_mode(cfg);
  if (st) return st;
  const Layout Y = layout(cfg);
  if (!aligned4(topk_idx) || !aligned16(x) || !aligned4(counts) || !aligned4(offsets) ||
      !aligned4(row_src) || !aligned4(tk_row) || !aligned16(workspace))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ring(Y, ring, ring_bytes, slot))) return st;
  if (ws_bytes < Y.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if ((st = check_device())) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int Tk = cfg->T * cfg->k;
  int32_t* blk = at<int32_t>(workspace, Y.blk_cnt);
  int32_t* flag = at<int32_t>(workspace, Y.blk_flag);
  int32_t* rank = at<int32_t>(workspace, Y.rank);
  uint8_t* slot_base = at<uint8_t>(ring, (size_t)slot * Y.slot);
  uint16_t* xp = Y.mx ? nullptr : reinterpret_cast<uint16_t*>(slot_base);
  uint8_t* xp8 = Y.mx ? slot_base : nullptr;
  uint8_t* xps = Y.mx ? slot_base + Y.slot_sc : nullptr;
  Launches L;
  L(launch_perm_hist(topk_idx, Tk, cfg->E, blk, rank, flag, s));
  if (!L.err)
    L(launch_perm_scan(blk, Y.nb, cfg->E, flag, counts, offsets, at<int32_t>(workspace, Y.status),
                       s));
  if (!L.err)
    L(launch_perm_place(topk_idx, rank, blk, Tk, cfg->E, cfg->k, row_src, tk_row,
                        static_cast<const uint16_t*>(x), xp, xp8, xps, cfg->d, Y.fb, s));
  return L.status();
}

int moe_permute_static(const moe_cfg* cfg, const int32_t* topk_idx, const void* x, void* ring,
                       size_t ring_bytes, int32_t slot, int32_t* counts, int32_t* offsets,
                       int32_t* row_src, int32_t* tk_row, int32_t* device_status,
                       moe_stream_t stream) {
  int st = check_mode(cfg);
  if (st) return st;
  const Layout Y = layout(cfg);
  if (!aligned4(topk_idx) || !aligned16(x) || !aligned4(counts) || !aligned4(offsets) ||
      !aligned4(row_src) || !aligned4(tk_row) || !aligned4(device_status))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ring(Y, ring, ring_bytes, slot))) return st;
  // the permutation's scratch, packed from offset 0 of the fixed array
  const size_t Tk = (size_t)cfg->T * cfg->k;
  const size_t o_flag = align_up(sizeof(int32_t) * (size_t)Y.nb * cfg->E);
  const size_t o_rank = o_flag + align_up(sizeof(int32_t) * (size_t)Y.nb);
  if (o_rank + sizeof(int32_t) * Tk > MOE_STATIC_SCRATCH_BYTES)
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  if ((st = check_device())) return st;
  void* base = nullptr;
  if (static_perm_scratch(&base) != hipSuccess) {
    (void)hipGetLastError();
    return MOE_ERR_HIP;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* slot_base = at<uint8_t>(ring, (size_t)slot * Y.slot);
  uint16_t* xp = Y.mx ? nullptr : reinterpret_cast<uint16_t*>(slot_base);
  uint8_t* xp8 = Y.mx ? slot_base : nullptr;
  uint8_t* xps = Y.mx ? slot_base + Y.slot_sc : nullptr;
  int32_t* blk = at<int32_t>(base, 0);
  int32_t* flag = at<int32_t>(base, o_flag);
  int32_t* rank = at<int32_t>(base, o_rank);
  // every scratch word is written before it is read: nothing needs clearing
  Launches L;
  L(launch_perm_hist(topk_idx, (int)Tk, cfg->E, blk, rank, flag, s));
  if (!L.err)
    L(launch_perm_scan(blk, Y.nb, cfg->E, flag, counts, offsets, device_status, s));
  if (!L.err)
    L(launch_perm_place(topk_idx, rank, blk, (int)Tk, cfg->E, cfg->k, row_src, tk_row,
                        static_cast<const uint16_t*>(x), xp, xp8, xps, cfg->d, Y.fb, s));
  return L.status();
}

int moe_forward(const moe_cfg* cfg, const void* ring, size_t ring_bytes, int32_t slot,
                const int32_t* offsets, const int32_t* tk_row, const float* topk_w,
                const void* w1, const void* w2, const void* wq, size_t wq_bytes, void* y,
                void* saved, size_t saved_bytes, void* workspace, size_t ws_bytes,
                moe_stream_t stream) {
  int st = check_mode(cfg);
  if (st) return st;
  const Layout Y = layout(cfg);
  if (!aligned4(offsets) || !aligned4(tk_row) || !aligned4(topk_w) || !aligned16(w1) ||
      !aligned16(w2) || !aligned16(y) || !aligned16(saved) || !aligned16(workspace))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ring(Y, ring, ring_bytes, slot))) return st;
  if ((st = check_wq(Y, wq, wq_bytes))) return st;
  if (saved_bytes < Y.saved_total || ws_bytes < Y.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if ((st = check_device())) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool pers = cfg->flags & MOE_FLAG_PERSISTENT;
  const int Tk = cfg->T * cfg->k, d = cfg->d, I = cfg->I, E = cfg->E;
  const uint8_t* slot_base = at<uint8_t>(ring, (size_t)slot * Y.slot);
  int2* sched = at<int2>(workspace, Y.sched);
  uint16_t* H = at<uint16_t>(saved, Y.H);
  uint16_t* A = at<uint16_t>(saved, Y.A);
  uint16_t* O = at<uint16_t>(workspace, Y.O);
  Launches L;
  L(launch_sched_build(offsets, E, Tk, sched, s));
  if (Y.mx) {
    uint8_t* aq = at<uint8_t>(workspace, Y.aq);
    uint8_t* aqs = at<uint8_t>(workspace, Y.aqs);
    if (!L.err)
      L(launch_fwd_gateup_mx({slot_base, slot_base + Y.slot_sc, at<uint8_t>(wq, Y.w1f),
                              at<uint8_t>(wq, Y.w1fs), H, A, aq, aqs, offsets, sched, d, I, Tk, E,
                              Y.fb},
                             pers, s));
    if (!L.err)
      L(launch_fwd_down_mx({aq, aqs, at<uint8_t>(wq, Y.w2f), at<uint8_t>(wq, Y.w2fs), O, offsets,
                            sched, d, I, Tk, E, Y.fb},
                           pers, s));
  } else {
    const uint16_t* xp = reinterpret_cast<const uint16_t*>(slot_base);
    if (!L.err)
      L(launch_fwd_gateup({xp, static_cast<const uint16_t*>(w1), H, A, offsets, sched, d, I, Tk, E},
                          pers, s));
    if (!L.err)
      L(launch_fwd_down({A, static_cast<const uint16_t*>(w2), O, offsets, sched, d, I, Tk, E}, pers,
                        s));
  }
  if (!L.err)
    L(launch_combine(O, tk_row, topk_w, cfg->T, cfg->k, d, static_cast<uint16_t*>(y), s));
  return L.status();
}

int moe_forward_fused(const moe_cfg* cfg, const void* x, const void* w_router, float* logits,
                      int32_t* topk_idx, float* topk_w, void* ring, size_t ring_bytes,
                      int32_t slot, int32_t* counts, int32_t* offsets, int32_t* row_src,
                      int32_t* tk_row, const void* w1, const void* w2, void* y, void* saved,
                      size_t saved_bytes, void* workspace, size_t ws_bytes, moe_stream_t stream) {
  int st = check_mode(cfg);
  if (st) return st;
  if (cfg->precision != MOE_PREC_BF16) return MOE_ERR_UNSUPPORTED;
  const Layout Y = layout(cfg);
  if (!aligned16(x) || !aligned16(w_router) || !aligned4(logits) || !aligned4(topk_idx) ||
      !aligned4(topk_w) || !aligned4(counts) || !aligned4(offsets) || !aligned4(row_src) ||
      !aligned4(tk_row) || !aligned16(w1) || !aligned16(w2) || !aligned16(y) ||
      !aligned16(saved) || !aligned16(workspace))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ring(Y, ring, ring_bytes, slot))) return st;
  if (saved_bytes < Y.saved_total || ws_bytes < Y.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if ((st = check_device())) return st;
  const int Tk = cfg->T * cfg->k;
  FusedFwdParams p{};
  p.x = static_cast<const uint16_t*>(x);
  p.wr = static_cast<const uint16_t*>(w_router);
  p.w32 = at<float>(workspace, Y.wr32);
  p.logits = logits;
  p.topk_idx = topk_idx;
  p.topk_w = topk_w;
  p.blk_cnt = at<int32_t>(workspace, Y.blk_cnt);
  p.rank = at<int32_t>(workspace, Y.rank);
  p.blk_flag = at<int32_t>(workspace, Y.blk_flag);
  p.counts = counts;
  p.offsets = offsets;
  p.status = at<int32_t>(workspace, Y.status);
  p.row_src = row_src;
  p.tk_row = tk_row;
  p.xp = at<uint16_t>(ring, (size_t)slot * Y.slot);
  p.sched = at<int2>(workspace, Y.sched);  // the 128-row block table opens the region
  p.w1 = static_cast<const uint16_t*>(w1);
  p.w2 = static_cast<const uint16_t*>(w2);
  p.H = at<uint16_t>(saved, Y.H);
  p.A = at<uint16_t>(saved, Y.A);
  p.O = at<uint16_t>(workspace, Y.O);
  p.y = static_cast<uint16_t*>(y);
  p.T = cfg->T;
  p.d = cfg->d;
  p.E = cfg->E;
  p.k = cfg->k;
  p.I = cfg->I;
  p.nb = Y.nb;
  // tokens per placement block, as moe_permute's launch chooses them
  int tpb = 1024 / (cfg->d / 8);
  if (tpb < 1) tpb = 1;
  if (tpb > 256 / cfg->k) tpb = 256 / cfg->k;
  p.tpb = tpb;
  (void)Tk;
  Launches L;
  L(launch_fused_forward(p, static_cast<hipStream_t>(stream)));
  return L.status();
}

int moe_backward(const moe_cfg* cfg, const void* ring, size_t ring_bytes, int32_t slot,
                 const int32_t* offsets, const int32_t* row_src, const int32_t* tk_row,
                 const int32_t* topk_idx, const float* topk_w, const void* w_router,
                 const void* w1, const void* w2, const void* wq, size_t wq_bytes,
                 const void* saved, size_t saved_bytes, const void* dy, void* dx, void* dw1,
                 void* dw2, float* dwr, float* d_topk_w, int32_t accumulate, void* workspace,
                 size_t ws_bytes, moe_stream_t stream) {
  int st = check_mode(cfg);
  if (st) return st;
  const Layout Y = layout(cfg);
  const bool routed = w_router != nullptr;
  if (!aligned4(offsets) || !aligned4(row_src) || !aligned4(tk_row) || !aligned4(topk_idx) ||
      !aligned4(topk_w) || !aligned16(w1) || !aligned16(w2) || !aligned16(saved) ||
      !aligned16(dy) || !aligned16(dx) || !aligned16(dw1) || !aligned16(dw2) ||
      !aligned4(d_topk_w) || !aligned16(workspace))
    return MOE_ERR_INVALID_ARG;
  if (routed && (!aligned16(w_router) || !aligned16(dwr))) return MOE_ERR_INVALID_ARG;
  if ((st = check_ring(Y, ring, ring_bytes, slot))) return st;
  if ((st = check_wq(Y, wq, wq_bytes))) return st;
  if (saved_bytes < Y.saved_total || ws_bytes < Y.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if ((st = check_device())) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool pers = cfg->flags & MOE_FLAG_PERSISTENT;
  const int bdw = (cfg->flags & MOE_FLAG_BF16_DW) ? 1 : 0;  // dW stored as bf16
  const int Tk = cfg->T * cfg->k, d = cfg->d, I = cfg->I, E = cfg->E, k = cfg->k;
  const uint8_t* slot_base = at<uint8_t>(ring, (size_t)slot * Y.slot);
  const uint16_t* xp = Y.mx ? nullptr : reinterpret_cast<const uint16_t*>(slot_base);
  const uint8_t* xp8 = Y.mx ? slot_base : nullptr;
  const uint8_t* xps = Y.mx ? slot_base + Y.slot_sc : nullptr;
  const uint16_t* H = at<uint16_t>(saved, Y.H);
  const uint16_t* A = at<uint16_t>(saved, Y.A);
  int2* sched = at<int2>(workspace, Y.sched);
  uint16_t* dH = at<uint16_t>(workspace, Y.dH);
  uint16_t* dXp = at<uint16_t>(workspace, Y.dXp);
  float* dwpart = at<float>(workspace, Y.dwpart);
  float* dl_pos = at<float>(workspace, Y.dl_pos);
  uint16_t* dyw = at<uint16_t>(workspace, Y.dyw);
  int32_t* wg_count = at<int32_t>(workspace, Y.wg_count);
  const uint16_t* dyp = static_cast<const uint16_t*>(dy);
  const uint16_t* w1p = static_cast<const uint16_t*>(w1);
  const uint16_t* w2p = static_cast<const uint16_t*>(w2);
  Launches L;
  L(launch_sched_build(offsets, E, Tk, sched, s));
  if (Y.mx) {
    uint8_t* dyq = at<uint8_t>(workspace, Y.dyq);
    uint8_t* dys = at<uint8_t>(workspace, Y.dys);
    uint8_t* dhq = at<uint8_t>(workspace, Y.dhq);
    uint8_t* dhs = at<uint8_t>(workspace, Y.dhs);
    if (!L.err) L(launch_quant_rows(dyp, cfg->T, d, dyq, dys, Y.fb, "quant_dy", s));
    if (!L.err) L(launch_scale_gather(dyp, tk_row, topk_w, cfg->T, k, d, dyw, s));
    if (!L.err)
      L(launch_bwd_down_dgrad_mx({dyq, dys, row_src, topk_w, at<uint8_t>(wq, Y.w2b),
                                  at<uint8_t>(wq, Y.w2bs), H, A, dH, dwpart, dhq, dhs, offsets,
                                  sched, d, I, k, Tk, E, Y.fb},
                                 pers, s));
    if (!L.err)
      L(launch_dw_router(dwpart, Y.nIt, tk_row, topk_w, cfg->T, k, d_topk_w, dl_pos, routed, s));
    if (cfg->flags & MOE_FLAG_MXFP8_WGRAD) {
      // both weight gradients in MXFP8, their operands quantised along each expert's positions
      int32_t* poff = at<int32_t>(workspace, Y.poff);
      uint8_t* lq = at<uint8_t>(workspace, Y.lq);
      uint8_t* lqs = at<uint8_t>(workspace, Y.lqs);
      uint8_t* rq = at<uint8_t>(workspace, Y.rq);
      uint8_t* rqs = at<uint8_t>(workspace, Y.rqs);
      if (!L.err) L(launch_seg_offsets(offsets, E, poff, s));
      SegOperand wdy, sa, sdh, sxp;
      wdy.src = dyp;  // w * dY, formed in fp32 and quantised from that
      wdy.row_src = row_src;
      wdy.topk_w = topk_w;
      wdy.k = k;
      sa.src = A;
      sdh.src = dH;
      sxp.src8 = xp8;
      sxp.src8s = xps;
      if (!L.err)
        L(launch_quant_seg(wdy, offsets, poff, E, d, Y.P, lq, lqs, "bwd_down_wgrad_qL", s));
      if (!L.err)
        L(launch_quant_seg(sa, offsets, poff, E, I, Y.P, rq, rqs, "bwd_down_wgrad_qR", s));
      if (!L.err)
        L(launch_mx_wgrad({lq, lqs, rq, rqs, dw2, poff, E, d, I, Y.P, accumulate, bdw,
                           "bwd_down_wgrad"},
                          pers, s));
      if (!L.err)
        L(launch_quant_seg(sdh, offsets, poff, E, 2 * I, Y.P, lq, lqs, "bwd_gate_wgrad_qL", s));
      if (!L.err)
        L(launch_quant_seg(sxp, offsets, poff, E, d, Y.P, rq, rqs, "bwd_gate_wgrad_qR", s));
      if (!L.err)
        L(launch_mx_wgrad({lq, lqs, rq, rqs, dw1, poff, E, 2 * I, d, Y.P, accumulate, bdw,
                           "bwd_gate_wgrad"},
                          pers, s));
    } else {
      if (!L.err)
        L(launch_wgrad({dyw, A, nullptr, nullptr, dw2, offsets, at<int4>(workspace, Y.wg_table2),
                        wg_count + 1, E, d, I, accumulate, bdw, false, "bwd_down_wgrad",
                        "wgrad_sched_down"},
                       s));
      // the gate wgrad goes first: until the gate dgrad writes dXp, that buffer holds the bf16
      // image of the big experts' MX Xp rows for the big-expert wgrad kernel
      if (!L.err)
        L(launch_wgrad({dH, nullptr, xp8, xps, dw1, offsets, at<int4>(workspace, Y.wg_table1),
                        wg_count, E, 2 * I, d, accumulate, bdw, true, "bwd_gate_wgrad",
                        "wgrad_sched_gate", dXp, Y.fb},
                       s));
    }
    if (!L.err)
      L(launch_bwd_gate_dgrad_mx({dhq, dhs, at<uint8_t>(wq, Y.w1b), at<uint8_t>(wq, Y.w1bs), dXp,
                                  offsets, sched, d, I, Tk, E, Y.fb},
                                 pers, s));
  } else {
    if (!L.err) L(launch_scale_gather(dyp, tk_row, topk_w, cfg->T, k, d, dyw, s));
    if (!L.err)
      L(launch_bwd_down_dgrad({dyp, row_src, topk_w, w2p, H, A, dH, dwpart, offsets, sched, d, I,
                               k, Tk, E},
                              pers, s));
    if (!L.err)
      L(launch_dw_router(dwpart, Y.nIt, tk_row, topk_w, cfg->T, k, d_topk_w, dl_pos, routed, s));
    if (!L.err)
      L(launch_wgrad({dyw, A, nullptr, nullptr, dw2, offsets, at<int4>(workspace, Y.wg_table2),
                      wg_count + 1, E, d, I, accumulate, bdw, false, "bwd_down_wgrad",
                      "wgrad_sched_down"},
                     s));
    if (!L.err) L(launch_bwd_gate_dgrad({dH, w1p, dXp, offsets, sched, d, I, Tk, E}, pers, s));
    if (!L.err)
      L(launch_wgrad({dH, xp, nullptr, nullptr, dw1, offsets, at<int4>(workspace, Y.wg_table1),
                      wg_count, E, 2 * I, d, accumulate, bdw, true, "bwd_gate_wgrad",
                      "wgrad_sched_gate"},
                     s));
  }
  if (!L.err)
    L(launch_uncombine(dXp, tk_row, topk_idx, dl_pos,
                       routed ? static_cast<const uint16_t*>(w_router) : nullptr, cfg->T, k, d,
                       static_cast<uint16_t*>(dx), s));
  if (!L.err && routed) L(launch_dwr(dl_pos, xp, xp8, xps, Y.fb, offsets, E, d, dwr, accumulate, s));
  return L.status();
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_RING_TOO_SMALL: return "ring buffer too small for the requested slot";
    case MOE_ERR_UNSUPPORTED: return "unsupported mode";
    case MOE_ERR_HIP: return "HIP runtime error while enqueuing";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace or saved buffer too small";
    default: return "unknown status";
  }
}

}  // extern "C"
