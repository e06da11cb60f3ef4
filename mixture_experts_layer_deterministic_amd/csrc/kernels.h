// Internal launch interface between the C ABI (api.cpp) and the HIP kernels. Every function
// only enqueues on the given stream and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Optional per-launch timing (moe_trace_begin / moe_trace_end): each launch site opens a
// TraceScope, which records a caller-provided event before the launch and another after it,
// both on the launching stream. With tracing off this costs one atomic load.
void trace_pre(const char* name, hipStream_t s);
void trace_post(hipStream_t s);
struct TraceScope {
  hipStream_t s;
  TraceScope(const char* name, hipStream_t st) : s(st) { trace_pre(name, s); }
  ~TraceScope() { trace_post(s); }
};

constexpr int kSchedBM = 128;   // rows per M-tile of the forward/dgrad grouped GEMMs
constexpr int kSchedBigBM = 256;  // rows per M-tile of the big-tile forward GEMMs
constexpr int kDgradBN = 128;   // columns per N-tile of the down dgrad (dw partials per row)
constexpr int kPermRows = 256;  // rows per histogram block of the permutation
constexpr int kMaxTopK = 64;

// router.hip
// w32: scratch of E * d floats for the router weight widened to fp32.
hipError_t launch_router_logits(const uint16_t* x, const uint16_t* wr, float* w32, float* logits,
                                int T, int d, int E, hipStream_t s);
hipError_t launch_router_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                              hipStream_t s);

// permute.hip
// Bytes of the fixed per-device scratch behind moe_permute_static, and its device address on
// the current device (fetched once per device).
constexpr size_t kStaticPermScratchBytes = size_t(4) << 20;
hipError_t static_perm_scratch(void** ptr);
hipError_t launch_perm_hist(const int32_t* idx, int Tk, int E, int32_t* blk_cnt, int32_t* rank,
                            int32_t* blk_flag, hipStream_t s);
hipError_t launch_perm_scan(int32_t* blk_cnt, int nb, int E, const int32_t* blk_flag,
                            int32_t* counts, int32_t* offsets, int32_t* status, hipStream_t s);
// With xp8 non-null the slot receives the MX image of each token (xp8 codes of fbits bits, xps
// scales) instead of the bf16 copy xp.
hipError_t launch_perm_place(const int32_t* idx, const int32_t* rank, const int32_t* blk_base,
                             int Tk, int E, int k, int32_t* row_src, int32_t* tk_row,
                             const uint16_t* x, uint16_t* xp, uint8_t* xp8, uint8_t* xps, int d,
                             int fbits, hipStream_t s);

// gemm.hip
int sched_max_mtiles(int Tk, int E);
int sched_max_big(int Tk);
int sched_max_rem(int Tk, int E);
// int2 entries of the schedule region: the full, big and remainder tables back to back
size_t sched_entries(int Tk, int E);
hipError_t launch_sched_build(const int32_t* offsets, int E, int Tk, int2* sched, hipStream_t s);

struct GemmFwdGateUpArgs {
  const uint16_t* xp;
  const uint16_t* w1;
  uint16_t* H;
  uint16_t* A;
  const int32_t* offsets;
  const int2* sched;
  int d, I, Tk, E;
};
struct GemmFwdDownArgs {
  const uint16_t* A;
  const uint16_t* w2;
  uint16_t* O;
  const int32_t* offsets;
  const int2* sched;
  int d, I, Tk, E;
};
struct GemmBwdDownDgradArgs {
  const uint16_t* dy;
  const int32_t* row_src;
  const float* topk_w;
  const uint16_t* w2;
  const uint16_t* H;
  const uint16_t* A;
  uint16_t* dH;
  float* dwpart;
  const int32_t* offsets;
  const int2* sched;
  int d, I, k, Tk, E;
};
struct GemmBwdGateDgradArgs {
  const uint16_t* dH;
  const uint16_t* w1;
  uint16_t* dXp;
  const int32_t* offsets;
  const int2* sched;
  int d, I, Tk, E;
};
// MX modes: codes with one E8M0 scale (uint8) per 32 along each GEMM's K. fbits 8: E4M3 codes,
// one a byte (MXFP8); fbits 4: E2M1 codes, two a byte, element 2i in the low nibble (MXFP4), so
// a row of n codes takes n * fbits / 8 bytes. The shapes below count codes.
struct GemmMxGateUpArgs {
  const uint8_t* xp8;  // [T*k, d], scales xps [T*k, d/32]
  const uint8_t* xps;
  const uint8_t* w8;   // [E, 2I, d], scales ws [E, 2I, d/32]
  const uint8_t* ws;
  uint16_t* H;
  uint16_t* A;
  uint8_t* aq;         // A quantised along I: [T*k, I], scales aqs [T*k, I/32]
  uint8_t* aqs;
  const int32_t* offsets;
  const int2* sched;
  int d, I, Tk, E, fbits;
};
struct GemmMxDownArgs {
  const uint8_t* aq;
  const uint8_t* aqs;
  const uint8_t* w8;   // [E, d, I], scales [E, d, I/32]
  const uint8_t* ws;
  uint16_t* O;
  const int32_t* offsets;
  const int2* sched;
  int d, I, Tk, E, fbits;
};
struct GemmMxDownDgradArgs {
  const uint8_t* dyq;  // [T, d], scales [T, d/32]
  const uint8_t* dys;
  const int32_t* row_src;
  const float* topk_w;
  const uint8_t* w8;   // W2 transposed [E, I, d], scales [E, I, d/32]
  const uint8_t* ws;
  const uint16_t* H;
  const uint16_t* A;
  uint16_t* dH;
  float* dwpart;
  uint8_t* dhq;        // dH quantised along 2I: [T*k, 2I], scales [T*k, 2I/32]
  uint8_t* dhs;
  const int32_t* offsets;
  const int2* sched;
  int d, I, k, Tk, E, fbits;
};
struct GemmMxGateDgradArgs {
  const uint8_t* dhq;
  const uint8_t* dhs;
  const uint8_t* w8;   // W1 transposed [E, d, 2I], scales [E, d, 2I/32]
  const uint8_t* ws;
  uint16_t* dXp;
  const int32_t* offsets;
  const int2* sched;
  int d, I, Tk, E, fbits;
};
hipError_t launch_fwd_gateup_mx(const GemmMxGateUpArgs& a, bool persistent, hipStream_t s);
hipError_t launch_fwd_down_mx(const GemmMxDownArgs& a, bool persistent, hipStream_t s);
hipError_t launch_bwd_down_dgrad_mx(const GemmMxDownDgradArgs& a, bool persistent, hipStream_t s);
hipError_t launch_bwd_gate_dgrad_mx(const GemmMxGateDgradArgs& a, bool persistent, hipStream_t s);
hipError_t launch_fwd_gateup(const GemmFwdGateUpArgs& a, bool persistent, hipStream_t s);
hipError_t launch_fwd_down(const GemmFwdDownArgs& a, bool persistent, hipStream_t s);
hipError_t launch_bwd_down_dgrad(const GemmBwdDownDgradArgs& a, bool persistent, hipStream_t s);
hipError_t launch_bwd_gate_dgrad(const GemmBwdGateDgradArgs& a, bool persistent, hipStream_t s);

// fused.hip: route, permute and forward in one cooperative launch (BF16)
struct FusedFwdParams {
  const uint16_t* x;
  const uint16_t* wr;
  float* w32;
  float* logits;
  int32_t* topk_idx;
  float* topk_w;
  int32_t* blk_cnt;
  int32_t* rank;
  int32_t* blk_flag;
  int32_t* counts;
  int32_t* offsets;
  int32_t* status;
  int32_t* row_src;
  int32_t* tk_row;
  uint16_t* xp;
  int2* sched;  // the 128-row block table: count, then (expert, first row)
  const uint16_t* w1;
  const uint16_t* w2;
  uint16_t* H;
  uint16_t* A;
  uint16_t* O;
  uint16_t* y;
  int T, d, E, k, I, nb, tpb;
};
hipError_t launch_fused_forward(const FusedFwdParams& p, hipStream_t s);

// wgrad.hip
constexpr int kWgradBM = 256;         // dW rows per task stripe
constexpr int kWgradBN = 128;         // dW columns per tile
constexpr int kWgradTaskSteps = 64;   // K-steps of 32 positions per task (target)
struct WgradArgs {
  const uint16_t* L;  // [T*k, Mdim], position-major
  const uint16_t* R;  // [T*k, Ndim], position-major (bf16), or null when R8 is given
  const uint8_t* R8;  // MX R (gate wgrad only): codes [T*k, Ndim * rbits / 8], or null
  const uint8_t* R8s; // its scales [T*k, Ndim/32]
  void* dw;           // [E, Mdim, Ndim], fp32 or (bf16_dw) bf16
  const int32_t* offsets;
  int4* table;        // task table, wgrad_table_entries(...) entries
  int32_t* count;     // task count (device)
  int E, Mdim, Ndim, accumulate, bf16_dw;
  bool gate;  // dW1 (true) or dW2 (false)
  const char* name;
  const char* name_sched;
  // with an MX R: bf16 scratch [T*k, Ndim] for the exact bf16 image of the big experts' R rows
  // (they then run on the big-expert kernel), or null (every expert on the task kernel)
  uint16_t* Rx = nullptr;
  int rbits = 8;  // an MX R's codes: 8 (E4M3) or 4 (E2M1)
};
size_t wgrad_table_entries(int Tk, int E, int Mdim, int Ndim);
hipError_t launch_wgrad(const WgradArgs& a, hipStream_t s);

// mx.hip
// fbits: 8 for MXFP8 (E4M3 codes, one a byte), 4 for MXFP4 (E2M1 codes, two a byte)
hipError_t launch_quant_rows(const uint16_t* src, long long rows, int cols, uint8_t* dst,
                             uint8_t* sc, int fbits, const char* name, hipStream_t s);
// Both MXFP8 copies of src [B][R][C]: along C into (dq, dqs), along R transposed into (tq, tqs).
hipError_t launch_quant_weight(const uint16_t* src, int B, int R, int C, uint8_t* dq,
                               uint8_t* dqs, uint8_t* tq, uint8_t* tqs, int fbits,
                               const char* name, hipStream_t s);
// MXFP8 weight gradients: expert segments padded to kSegK positions (segment offsets poff
// [E + 1], the padded total in poff[E] <= seg_capacity), and an operand S [T*k, C] quantised
// along each segment's positions into q [C][P] codes and qs [C][P / 32] scales.
constexpr int kSegK = 128;
inline int seg_capacity(int Tk, int E) {
  return (Tk + E * (kSegK - 1) + kSegK - 1) / kSegK * kSegK;
}
hipError_t launch_seg_offsets(const int32_t* offsets, int E, int32_t* poff, hipStream_t s);
// The operand: bf16 rows (src), or the MXFP8 image along C (src8 codes, src8s scales), or
// w * dY gathered in fp32 (src = dY [T, C], row_src, topk_w, k).
struct SegOperand {
  const uint16_t* src = nullptr;
  const uint8_t* src8 = nullptr;
  const uint8_t* src8s = nullptr;
  const int32_t* row_src = nullptr;
  const float* topk_w = nullptr;
  int k = 1;
};
hipError_t launch_quant_seg(const SegOperand& x, const int32_t* offsets, const int32_t* poff,
                            int E, int C, int P, uint8_t* q, uint8_t* qs, const char* name,
                            hipStream_t s);
// dW [E, Mdim, Ndim] (fp32, overwritten or accumulated) = per expert, lq^T rq over its padded
// positions: lq [Mdim][P] and rq [Ndim][P] with scales [.][P / 32], from launch_quant_seg.
struct GemmMxWgradArgs {
  const uint8_t* lq;
  const uint8_t* lqs;
  const uint8_t* rq;
  const uint8_t* rqs;
  void* dw;  // fp32 or (bf16_dw) bf16
  const int32_t* poff;
  int E, Mdim, Ndim, P, accumulate, bf16_dw;
  const char* name;
};
hipError_t launch_mx_wgrad(const GemmMxWgradArgs& a, bool persistent, hipStream_t s);
hipError_t launch_scale_gather(const uint16_t* dy, const int32_t* tk_row, const float* topk_w,
                               int T, int k, int d, uint16_t* dyw, hipStream_t s);

// elementwise.hip
hipError_t launch_combine(const uint16_t* O, const int32_t* tk_row, const float* topk_w, int T,
                          int k, int d, uint16_t* y, hipStream_t s);
hipError_t launch_dw_router(const float* dwpart, int nIt, const int32_t* tk_row,
                            const float* topk_w, int T, int k, float* d_topk_w, float* dl_pos,
                            int routed, hipStream_t s);
hipError_t launch_uncombine(const uint16_t* dXp, const int32_t* tk_row, const int32_t* topk_idx,
                            const float* dl_pos, const uint16_t* wr, int T, int k, int d,
                            uint16_t* dx, hipStream_t s);
// With xp8 non-null, Xp is read as MXFP8 (codes xp8, scales xps) instead of bf16 xp.
// Xp as bf16 rows xp, or (xp8 given) as MX codes xp8 with scales xps: fbits 8 E4M3, 4 E2M1.
hipError_t launch_dwr(const float* dl_pos, const uint16_t* xp, const uint8_t* xp8,
                      const uint8_t* xps, int fbits, const int32_t* offsets, int E, int d,
                      float* dwr, int accumulate, hipStream_t s);

}  // namespace moe
