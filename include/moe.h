/*
 * moe.h - C ABI of a deterministic MoE layer (forward and backward) for one AMD MI355X (gfx950).
 *
 * The layer is the mixture-of-experts step that the pages on Mixture-of-Kittens (MoK) describe.
 * Those pages are the MarkTechPost article "Cursor Open-Sources Mixture-of-Kittens (MoK): A
 * Deterministic MoE Training Megakernel for GB300 NVL72 Racks", the toknow.ai post
 * "Mixture-of-Kittens: Cursor's Open-Source Kernel Trains AI Up to 2.37x Faster" and the aiweekly.co
 * alert "Cursor open-sources MoE megakernel for GB300 NVL72 racks". This library takes one GPU's
 * share of it.
 *
 * Forward: the router, then an expert-grouped permute into a ring slot, then per-expert SwiGLU
 * MLPs, then a weighted combine. Backward: dgrad and wgrad of every GEMM, plus the router-weight
 * gradient, which is computed inside the SwiGLU backward (MarkTechPost, closing paragraph of
 * "Three design decisions that matter").
 *
 * Conventions for every entry point:
 *  - Every pointer argument is DEVICE memory of the current HIP device, owned by the caller. The
 *    library never allocates, frees or synchronises. Each call only enqueues kernels on `stream`
 *    (a hipStream_t; NULL means the null stream) and returns.
 *  - Row-major layouts throughout. bf16 is IEEE bfloat16 stored as uint16. Weights follow the
 *    [out, in] convention: W1 is [E, 2I, d] (rows 0..I-1 gate, I..2I-1 up), W2 is [E, d, I], and
 *    the router weight Wr is [E, d].
 *  - Return value: MOE_OK (0), or a negative moe_status. Arguments are checked on the host before
 *    anything is enqueued. A failed check enqueues nothing. Nothing prints and nothing throws.
 *  - Determinism: every result is a function of the inputs alone. No float atomics are used,
 *    and every reduction runs in a fixed order, so two runs are bitwise identical.
 *  - No host synchronisation: per-expert counts never leave the device. Buffers are sized for
 *    the worst case, so no token is ever dropped, whatever the expert imbalance (MarkTechPost,
 *    "Three design decisions that matter": ring token buffer; "Key Takeaways").
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* moe_stream_t; /* hipStream_t */

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,     /* null pointer, bad shape, misaligned pointer */
    MOE_ERR_RING_TOO_SMALL = -2,  /* ring_bytes < (slot + 1) * ring slot bytes */
    MOE_ERR_UNSUPPORTED = -3,     /* a mode the library does not provide */
    MOE_ERR_HIP = -4,             /* a HIP runtime error while enqueuing */
    MOE_ERR_WORKSPACE_TOO_SMALL = -5
} moe_status;

enum { MOE_PREC_BF16 = 0, MOE_PREC_MXFP8 = 1, MOE_PREC_MXFP4 = 2 };

/* cfg.flags bits */
enum {
    MOE_FLAG_PERSISTENT = 1,  /* grouped GEMMs as persistent grids walking the schedule table */
    MOE_FLAG_MXFP8_WGRAD = 2, /* MXFP8 mode only: the weight gradients in MXFP8 too (below) */
    MOE_FLAG_BF16_DW = 4      /* dw1 and dw2 are bf16 buffers instead of fp32 (below) */
};

/* Device status word (first 4 bytes of the workspace). moe_permute clears it and ORs bits into
 * it; the caller may read it after its own synchronisation. */
enum {
    MOE_DEVICE_BAD_EXPERT_INDEX = 1, /* a topk_idx entry outside [0, E): that row is skipped */
    MOE_DEVICE_BARRIER_TIMEOUT = 2   /* moe_forward_fused: a grid barrier waited ~2 s and gave up
                                        (the results of that call are not valid) */
};

/* Layer shape and mode. Constraints checked on the host: T >= 1; 1 <= k <= E <= 1024; k <= 64;
 * d % 256 == 0 (the GEMMs have no masked K tail: K steps of 64 and 256-wide tiles along d);
 * I % 128 == 0 (128-wide tiles along I); T * k < 2^31; T * E < 2^31; and, because the kernels
 * address rows with 32-bit offsets: T * d < 2^31, T * k * d < 2^31, T * k * 2I < 2^31 (an
 * expert may receive all T * k rows) and 4 * I * d < 2^31 (the bytes of one expert's W1).
 * precision MOE_PREC_BF16, MOE_PREC_MXFP8 or MOE_PREC_MXFP4 (MXFP4 also needs I % 256 == 0: its
 * K steps along I are 256 deep).
 * Every entry point that enqueues work also checks that the current HIP device is a gfx950
 * (MOE_ERR_UNSUPPORTED otherwise, MOE_ERR_HIP when no device can be queried).
 *
 * MXFP8 mode (the pages name BF16 and MXFP8 modes: MarkTechPost, closing paragraph of "Three
 * design decisions that matter") follows the OCP MX v1.0 MXFP8 format. Elements are E4M3; every
 * 32 consecutive elements along a GEMM's reduction axis share one E8M0 scale 2^(code - 127),
 * code = floor(log2 amax) - 8 + 127 clamped to 0..254 (0 for an all-zero block). Elements round
 * to nearest even and saturate to +-448. The forward GEMMs read Xp and W1 quantised along d,
 * and A and W2 along I. The dgrad GEMMs read dY and W2 along d, and dH and W1 along 2I. The
 * weight gradients and dWr read bf16 operands, with Xp taken as the MXFP8 image the ring
 * holds. All accumulation is fp32; outputs are bf16 as in BF16 mode.
 * With MOE_FLAG_MXFP8_WGRAD the two weight gradients take MXFP8 operands as well, quantised
 * along their reduction axis, the positions of each expert: blocks of 32 consecutive positions
 * from the expert's first one, the last block holding what is left. dW2 reads w dY (the fp32
 * product, quantised directly) and A, dW1 reads dH and the ring's MXFP8 image of Xp, each
 * quantised so. dWr is unchanged.
 *
 * MXFP4 mode (the MarkTechPost page, section "MoE layer as the bottleneck", names the team's
 * earlier 4-bit NVFP4 training kernels; this mode takes the OCP MX 4-bit format instead, which
 * gfx950's scaled MFMA reads) follows the OCP MX v1.0 MXFP4 format on the same axes as MXFP8
 * mode: elements are E2M1 (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), stored two to a byte
 * with element 2i in the low nibble; the scale code is floor(log2 amax) - 2 + 127 clamped to
 * 0..254; elements round to nearest even and saturate to +-6. The weight gradients and dWr read
 * bf16 operands, Xp taken as the exact bf16 image of the MXFP4 codes the ring holds.
 * MOE_FLAG_MXFP8_WGRAD is not accepted. Buffers: a ring slot holds Xp's codes [T*k, d/2 bytes]
 * then its scales; moe_quantize_weights writes the four weight copies in E2M1.
 *
 * Weight-gradient precision. The pages do not say in which precision the weight gradients are
 * kept. By default dw1 and dw2 are fp32 (the caller's main gradient, which microbatches
 * accumulate into). With MOE_FLAG_BF16_DW (any precision) they are bf16: each element is
 * the same fp32 sum rounded once to nearest even where it is stored; with accumulate the fp32
 * sum of the stored bf16 value and the new result is rounded once. dwr stays fp32. */
typedef struct moe_cfg {
    int32_t T;         /* tokens entering the layer */
    int32_t d;         /* hidden size */
    int32_t E;         /* experts on this GPU */
    int32_t k;         /* experts per token (top-k) */
    int32_t I;         /* SwiGLU intermediate size */
    int32_t precision; /* MOE_PREC_* */
    int32_t flags;     /* MOE_FLAG_* */
} moe_cfg;

/* Byte sizes of the caller-owned buffers, and the offsets of the intermediates inside them. */
typedef struct moe_sizes {
    size_t ring_slot;      /* one ring slot: the permuted tokens Xp, bf16 [T*k, d] */
    size_t saved;          /* forward activations kept for backward */
    size_t saved_H;        /* offset of H = [g | u], bf16 [T*k, 2I], rows in position order */
    size_t saved_A;        /* offset of A = silu(g) * u, bf16 [T*k, I] */
    size_t workspace;      /* scratch for route/permute/forward/backward (one buffer serves all) */
    size_t ws_O;           /* offset of the expert outputs O, bf16 [T*k, d], valid after forward */
    size_t ws_dH;          /* offset of dH, bf16 [T*k, 2I], valid after backward */
    size_t ws_dXp;         /* offset of dXp, bf16 [T*k, d], valid after backward */
    size_t wq;             /* MX modes: bytes of the quantised-weight buffer (0 in BF16 mode) */
} moe_sizes;

/* Sizes of every caller buffer for `cfg`. Host only; enqueues nothing. (Plumbing of this
 * library, defined by no passage of the pages. The schedule and task tables live inside the
 * workspace, so they have no size of their own here.)
 * In MXFP8 mode a ring slot holds the E4M3 codes of Xp [T*k, d] followed (at the next 256-byte
 * boundary) by their scales [T*k, d/32]; in MXFP4 mode the E2M1 codes [T*k, d/2 bytes] followed
 * by the scales. */
int moe_query(const moe_cfg* cfg, moe_sizes* out);

/*
 * moe_quantize_weights - MX modes only: the quantised expert weights every MXFP8 or MXFP4 forward
 * and backward reads. Call it once per weight update; the result serves any number of batches.
 *
 *   w1  bf16 [E, 2I, d]   in
 *   w2  bf16 [E, d, I]    in
 *   wq  bytes [wq_bytes]  out, wq_bytes >= moe_sizes.wq. It receives four quantised tensors, each
 *       with its per-32 scales: W1 along d [E, 2I, d] and W2 along I [E, d, I] (forward), and W2
 *       along d stored transposed [E, I, d] and W1 along 2I stored transposed [E, d, 2I]
 *       (dgrad), in the mode's element format. The layout inside wq is private to the library.
 * Errors: MOE_ERR_INVALID_ARG in BF16 mode; MOE_ERR_WORKSPACE_TOO_SMALL for a short wq.
 */
int moe_quantize_weights(const moe_cfg* cfg, const void* w1, const void* w2, void* wq,
                         size_t wq_bytes, moe_stream_t stream);

/*
 * moe_route - router logits, top-k selection and renormalised softmax weights.
 *
 * The toknow.ai summary describes an MoE as sending each input to a few experts. The gate used
 * here is the plain top-k softmax:
 *   logits[t,e] = sum_i x[t,i] * w_router[e,i], in fp32. For each (t,e) one accumulator starts
 *       at +0 and gains the exact bf16 x bf16 products for i = 0,1,..,d-1 in ascending order,
 *       rounding after each addition.
 *   topk_idx[t,:] holds the k largest logits in descending order; equal logits go to the lower
 *       expert index. Selection compares logits numerically (-0 == +0; NaN unsupported).
 *   topk_w[t,j] = exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0), in fp32 (l_0 = the largest),
 *       which equals softmax over all E followed by renormalisation over the k selected.
 *
 *   x        bf16 [T, d]    in
 *   w_router bf16 [E, d]    in
 *   logits   fp32 [T, E]    out
 *   topk_idx int32 [T, k]   out
 *   topk_w   fp32 [T, k]    out
 *   workspace bytes [ws_bytes]  scratch (the router weight widened to fp32), the same
 *                               workspace the other calls take
 */
int moe_route(const moe_cfg* cfg, const void* x, const void* w_router, float* logits,
              int32_t* topk_idx, float* topk_w, void* workspace, size_t ws_bytes,
              moe_stream_t stream);

/*
 * moe_permute - expert histogram, exclusive scan, and a stable grouping of the T*k rows by
 * expert into ring slot `slot`.
 *
 * The gather half of the pages' dispatch is the part that stays on one GPU (MarkTechPost, "Three
 * design decisions that matter": pull-based dispatch and the ring token buffer). Row r = t*k + j
 * goes to position pos = offsets[e] + (number of rows r' < r with the same expert e), so inside
 * an expert segment rows ascend by r.
 *
 *   topk_idx int32 [T, k]          in   (from moe_route, or given by the caller; a caller's row
 *                                       may name one expert twice: every row is its own
 *                                       position either way)
 *   x        bf16 [T, d]           in
 *   ring     bytes [ring_bytes]    out: slot `slot` (at slot * ring_slot bytes) receives
 *                                       Xp[pos] = x[row_src[pos] / k], bf16 [T*k, d]; in an MX
 *                                       mode its MX image (codes, then scales)
 *   counts   int32 [E]             out: rows per expert
 *   offsets  int32 [E+1]           out: exclusive scan of counts, offsets[E] = T*k
 *   row_src  int32 [T*k]           out: pos -> r
 *   tk_row   int32 [T*k]           out: r -> pos (-1 for a skipped bad-index row)
 *   workspace bytes [ws_bytes]     scratch; also holds the device status word
 * Errors: MOE_ERR_RING_TOO_SMALL when (slot + 1) * ring_slot > ring_bytes or slot < 0.
 */
int moe_permute(const moe_cfg* cfg, const int32_t* topk_idx, const void* x, void* ring,
                size_t ring_bytes, int32_t slot, int32_t* counts, int32_t* offsets,
                int32_t* row_src, int32_t* tk_row, void* workspace, size_t ws_bytes,
                moe_stream_t stream);

/*
 * moe_permute_static - moe_permute for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same operation, arguments and
 * results as moe_permute, except that:
 *  - there is no workspace argument: the permutation's scratch (per-256-row-block expert counts,
 *    per-row ranks, per-block flags) lives in a fixed array of MOE_STATIC_SCRATCH_BYTES inside
 *    the library, one per GPU, held until the process ends;
 *  - the device status word is written to `device_status` (int32, caller device memory) instead
 *    of the workspace's first word.
 * The call allocates nothing and frees nothing. Its scratch needs 4 * (nb * E + nb + T * k)
 * bytes with nb = ceil(T * k / 256), each part 256-byte aligned; beyond MOE_STATIC_SCRATCH_BYTES
 * it returns MOE_ERR_WORKSPACE_TOO_SMALL and enqueues nothing. Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (concurrent streams, or threads) race and give
 * undefined results. Calls in one stream order are safe; the array keeps the last call's
 * contents, and every word is written before it is read.
 */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)4 << 20)
int moe_permute_static(const moe_cfg* cfg, const int32_t* topk_idx, const void* x, void* ring,
                       size_t ring_bytes, int32_t slot, int32_t* counts, int32_t* offsets,
                       int32_t* row_src, int32_t* tk_row, int32_t* device_status,
                       moe_stream_t stream);

/*
 * moe_forward - grouped SwiGLU expert MLPs over the ring slot, then the weighted combine.
 *
 * The expert-grouped GEMMs are in MarkTechPost, "Three design decisions that matter". For each
 * expert e and each of its positions:
 *   [g | u] = Xp[pos] W1[e]^T   (fp32 accumulate; stored bf16 as H)
 *   A       = silu(g) * u        (from the fp32 g, u; stored bf16)
 *   O[pos]  = A W2[e]^T          (fp32 accumulate; stored bf16 in the workspace)
 * Combine, which is atomic-free and fixed-order:
 *   y[t] = bf16( sum_{j=0..k-1} topk_w[t,j] * O[tk_row[t*k+j]] ), fp32 FMA with j ascending.
 *
 *   ring, ring_bytes, slot   in: the slot written by moe_permute
 *   offsets, tk_row          in: from moe_permute
 *   topk_w   fp32 [T, k]     in
 *   w1       bf16 [E, 2I, d] in
 *   w2       bf16 [E, d, I]  in
 *   wq, wq_bytes             in: MX modes, the buffer moe_quantize_weights filled (ignored in
 *                                BF16 mode, may be NULL)
 *   y        bf16 [T, d]     out
 *   saved    bytes [saved_bytes]   out: H and A at the offsets moe_query reports
 *   workspace bytes [ws_bytes]     scratch
 */
int moe_forward(const moe_cfg* cfg, const void* ring, size_t ring_bytes, int32_t slot,
                const int32_t* offsets, const int32_t* tk_row, const float* topk_w,
                const void* w1, const void* w2, const void* wq, size_t wq_bytes, void* y,
                void* saved, size_t saved_bytes, void* workspace, size_t ws_bytes,
                moe_stream_t stream);

/*
 * moe_forward_fused - moe_route, moe_permute and moe_forward in ONE kernel launch (BF16 mode).
 *
 * The pages' layer is one persistent kernel that fuses all of its steps (MarkTechPost, "Cursor
 * Open-Sources Mixture-of-Kittens (MoK)": introduction, and the closing paragraph of "Three
 * design decisions that matter"). This call runs the router, the permutation into ring slot
 * `slot`, both grouped GEMMs and the combine as phases of one cooperatively launched grid
 * (every workgroup resident) that meet at grid-wide barriers, so a small layer pays one launch
 * instead of about a dozen. It writes everything the three calls write (logits, topk_idx,
 * topk_w, counts, offsets, row_src, tk_row, the ring slot, H and A in `saved`, O in the
 * workspace, y, the device status word), with the same values: bit for bit when no expert
 * receives 256 rows or more; otherwise the down projection of those experts' rows sums its K
 * chunks from another start (the separate path gives such blocks a 256 x 256 tile), which
 * changes their O and y in the last bits only. Arguments and errors are those of the three
 * calls; the MX modes return MOE_ERR_UNSUPPORTED. The grid barriers keep their state in a
 * device variable of the library, one per GPU: fused calls that overlap on one GPU race.
 */
int moe_forward_fused(const moe_cfg* cfg, const void* x, const void* w_router, float* logits,
                      int32_t* topk_idx, float* topk_w, void* ring, size_t ring_bytes,
                      int32_t slot, int32_t* counts, int32_t* offsets, int32_t* row_src,
                      int32_t* tk_row, const void* w1, const void* w2, void* y, void* saved,
                      size_t saved_bytes, void* workspace, size_t ws_bytes, moe_stream_t stream);

/*
 * moe_backward - gradients of L = <y, dy> with respect to x, the router weight, w1, w2 and the
 * routing weights.
 *
 * Per position pos (token t, slot j, expert e, weight w):
 *   dA'      = dy[t] W2[e]                           (fp32, never stored)
 *   dw       = <dA', A[pos]>, which equals <dy[t], A[pos] W2[e]^T>. This is the router-weight
 *              gradient, fused into the SwiGLU backward (MarkTechPost, closing paragraph of
 *              "Three design decisions that matter"). Per-tile partials are summed in
 *              ascending tile order.
 *   dA       = w * dA'
 *   dg, du   = dA * u * s * (1 + g (1 - s)),  dA * silu(g)   (s = sigmoid(g); g, u from H)
 *   dH[pos]  = bf16([dg | du]);  dXp[pos] = bf16(dH[pos] W1[e])
 *   dW2[e]   = sum over pos in e, ascending, of bf16(w dy[t]) (x) A[pos]   (fp32 sums)
 *   dW1[e]   = sum over pos in e, ascending, of dH[pos] (x) Xp[pos]       (fp32 sums)
 * Per token: d_topk_w[t,j] = dw of its row. When w_router is given (the layer routed itself):
 *   dlogit_j = w_j (dw_j - sum_i w_i dw_i), and 0 off the selected set;
 *   dx[t]    = bf16( sum_j dXp[tk_row[t*k+j]] + sum_j dlogit_j Wr[e_j] ), j ascending, fp32;
 *   dWr[e]   = sum over pos in e, ascending, of dlogit(pos) * Xp[pos]          (fp32).
 * When w_router is NULL (routing given), dx[t] = bf16(sum_j dXp[tk_row[t*k+j]]), and dwr is not
 * touched. Experts with no rows get zero dW1/dW2 blocks. With accumulate != 0, dw1, dw2 and dwr
 * are added to (read-modify-write, the sum in fp32) instead of overwritten.
 *
 *   ring, ring_bytes, slot        in: the slot holding this batch's Xp (written by moe_permute)
 *   offsets, row_src, tk_row      in: from moe_permute
 *   topk_idx int32 [T, k], topk_w fp32 [T, k]   in
 *   w_router bf16 [E, d] or NULL  in
 *   w1, w2, wq, wq_bytes          in (as in moe_forward)
 *   saved                         in: from moe_forward of the same batch
 *   dy       bf16 [T, d]          in
 *   dx       bf16 [T, d]          out
 *   dw1      fp32 [E, 2I, d]      out (or accumulated); bf16 with MOE_FLAG_BF16_DW
 *   dw2      fp32 [E, d, I]       out (or accumulated); bf16 with MOE_FLAG_BF16_DW
 *   dwr      fp32 [E, d]          out (or accumulated); ignored when w_router is NULL
 *   d_topk_w fp32 [T, k]          out
 *   workspace bytes [ws_bytes]    scratch (dH and dXp at the offsets moe_query reports)
 */
int moe_backward(const moe_cfg* cfg, const void* ring, size_t ring_bytes, int32_t slot,
                 const int32_t* offsets, const int32_t* row_src, const int32_t* tk_row,
                 const int32_t* topk_idx, const float* topk_w, const void* w_router,
                 const void* w1, const void* w2, const void* wq, size_t wq_bytes,
                 const void* saved, size_t saved_bytes, const void* dy, void* dx, void* dw1,
                 void* dw2, float* dwr, float* d_topk_w, int32_t accumulate, void* workspace,
                 size_t ws_bytes, moe_stream_t stream);

/*
 * Launch tracing, for benchmarks and profilers; the layer never needs it.
 * moe_trace_begin: until moe_trace_end, every kernel the library enqueues is bracketed by two
 * hipEventRecord calls on the kernel's own stream: events[2i] before and events[2i+1] after the
 * i-th launch, for 2i+1 < capacity. names[i] receives the kernel's static name when names is
 * non-NULL. The caller creates the hipEvent_t handles (with timing enabled) and keeps them
 * alive. Not meant for concurrent use from several threads.
 *   events   hipEvent_t [capacity]   host array of caller-created events
 *   names    const char* [capacity/2] host array, or NULL
 * moe_trace_end stops tracing and returns the number of launches seen since moe_trace_begin
 * (launches beyond capacity/2 were counted but not timed).
 */
int moe_trace_begin(void* const* events, int capacity, const char** names);
int moe_trace_end(void);

/* A static string for a moe_status value (plumbing of this library, defined by no passage of
 * the pages). */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
