"""Plain numpy oracle of the deterministic MoE layer (forward and backward). Test infrastructure.

Notation: T tokens, hidden size d, E experts, top-k, SwiGLU intermediate I. A "row" is one
(token t, slot j) pair with flat index r = t*k + j. Rows are grouped by expert into "positions"
pos = 0 .. T*k-1, so every expert owns one contiguous segment.

Each function states the passage or reading it follows. The pages are the MoE training-megakernel
pages on Mixture-of-Kittens (MoK): the ncijnetwork.com copy of the MarkTechPost article, toknow.ai
and aiweekly.co.
"""
from __future__ import annotations

import numpy as np

from . import mx

readings = {
    "gate": "softmax over all E router logits, keep the k largest, renormalise over those k; "
            "no bias, no capacity, no auxiliary loss (toknow.ai summary: each input goes to a "
            "few experts; MarkTechPost 'Three design decisions that matter': no dropped tokens)",
    "logit_order": "fp32 logits, each accumulated over the hidden index i = 0..d-1 in ascending "
                   "order into one fp32 accumulator (products of two bf16 values are exact in "
                   "fp32, so fused multiply-add and multiply-then-add agree)",
    "select": "top-k on the fp32 logits, ties to the lower expert index; slots j ordered by "
              "descending logit (ties lower index first)",
    "weights": "w_j = exp(l_j - l_max) / sum_{i in S} exp(l_i - l_max), equal in exact "
               "arithmetic to softmax-then-renormalise",
    "permutation": "stable counting sort of the rows by expert: inside a segment rows ascend by "
                   "r = t*k + j",
    "expert": "SwiGLU: g = x W_gate^T, u = x W_up^T, a = silu(g) * u, o = a W2^T, no biases; "
              "W1 = [W_gate; W_up] stacked as [2I, d]",
    "combine": "y_t = sum_j w_tj o_tj with j ascending",
    "router_grad": "the router-weight gradient dL/dw_tj = <dY_t, o_tj> (MarkTechPost, closing "
                   "paragraph of 'Three design decisions that matter': computed inside the "
                   "SwiGLU backward), flowing on to the logits, the router weight and the input",
    "storage_bf16": "H = [g|u], A, O, Y, dH, dXp, dX stored as bf16; A is rounded once from "
                    "the unrounded g, u; every later step reads the stored value",
    "mxfp8_wgrad": "MXFP8 weight gradients (an option of MXFP8 mode): both operands of each "
                   "weight-gradient product are MXFP8 images quantised along its reduction "
                   "axis, the positions of one expert segment, in blocks of 32 consecutive "
                   "positions from the segment's first (the last block holds the rest): dW2 "
                   "from (w dY) and A, dW1 from dH and the MXFP8 image of Xp the ring holds "
                   "(quantised again, along the positions)",
    "dw_bf16": "weight gradients stored as bf16, an option (the default stores dW1 and dW2 in "
               "fp32, the caller's main gradient): each element of dW1 and dW2 is its sum "
               "rounded once to bf16 where it is stored; dWr stays fp32",
    "mxfp4": "MXFP4 mode, the 4-bit analogue of MXFP8 mode (MarkTechPost, 'MoE layer as the "
             "bottleneck': the pages' NVFP4 training kernels; OCP MX v1.0 MXFP4): E2M1 elements "
             "with one E8M0 scale per 32, the scale exponent floor(log2 amax) - 2, round to "
             "nearest even, saturate to 6; every expert GEMM of forward and dgrad takes both "
             "operands as MXFP4 images along the same axes as in MXFP8 mode, and the weight "
             "gradients and dWr take Xp as its MXFP4 image",
    "mxfp8": "MXFP8 mode (MarkTechPost, closing paragraph of 'Three design decisions that "
             "matter': BF16 and MXFP8 modes): every expert GEMM of forward and dgrad takes both "
             "operands as MXFP8 images quantised along that GEMM's reduction axis - Xp and W1 "
             "along d, the stored A and W2 along I (forward); dY and W2 along d, the stored dH "
             "and W1 along 2I (dgrad). The router-weight gradient is the fused <dA', A> with dA' "
             "from the quantised dgrad GEMM. The weight gradients stay on bf16 operands, with Xp "
             "taken as its MXFP8 image (the ring holds the quantised tokens); so does dWr",
}


# ----------------------------------------------------------------------------------------------
# bfloat16 rounding

def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16, ties to even; returns float64.

    A bfloat16 keeps 8 significant bits. The float64 significand has 53, so the low 45 bits
    are dropped with round-to-nearest-even on the bit pattern. This holds in bfloat16's normal
    range, the only range the layer's data reaches. Its subnormals and overflow are not
    modelled.
    """
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    u = a.view(np.uint64)
    drop = np.uint64(45)
    half = np.uint64((1 << 44) - 1)
    odd = (u >> drop) & np.uint64(1)
    r = (u + half + odd) & ~np.uint64((1 << 45) - 1)
    return r.view(np.float64)


def _is_bf16(a: np.ndarray) -> bool:
    return bool(np.all(bf16_round(a) == a))


# ----------------------------------------------------------------------------------------------
# Router

def router_logits_fp32(X, Wr) -> np.ndarray:
    """Router logits L[t, e] = sum_i X[t, i] Wr[e, i] in float32, in one fixed order.

    Reading "logit_order": one float32 accumulator per (t, e), starting at +0, gains the
    products for i = 0, 1, ..., d-1 in that order, rounding to nearest after each addition. X
    and Wr hold bfloat16 values, so each product is exact in float32. Its one rounding then
    equals the fused multiply-add's.
    """
    X32 = np.asarray(X, dtype=np.float32)
    W32 = np.asarray(Wr, dtype=np.float32)
    assert _is_bf16(X32) and _is_bf16(W32), "router inputs must hold bfloat16 values"
    T, d = X32.shape
    E = W32.shape[0]
    XT = np.ascontiguousarray(X32.T)  # row i holds x[:, i] (contiguous reads; same values)
    WT = np.ascontiguousarray(W32.T)
    acc = np.zeros((T, E), dtype=np.float32)
    prod = np.empty_like(acc)
    for i in range(d):
        np.multiply.outer(XT[i], WT[i], out=prod)  # exact: bf16 x bf16 fits in fp32
        acc += prod                                # one fp32 rounding per step, i ascending
    return acc


def router_logits_fp64(X, Wr) -> np.ndarray:
    """The same logits in float64 (a plain matrix product); for the exact-math reference."""
    return np.asarray(X, np.float64) @ np.asarray(Wr, np.float64).T


def route_topk(L, k: int):
    """Top-k selection and renormalised softmax weights (readings "select", "weights").

    The k largest logits are taken, in descending order. Equal logits go lower expert index
    first, because a stable sort of -L keeps the ascending index order among equal keys. Then
    w_j = exp(l_j - l_max) / sum over the selected set of exp(l_i - l_max), in float64 from the
    given logits. Returns (idx int32 [T,k], w float64 [T,k]).
    """
    L = np.asarray(L)
    order = np.argsort(-L, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(L, idx, axis=1).astype(np.float64)
    z = np.exp(sel - sel[:, :1])
    w = z / z.sum(axis=1, keepdims=True)
    return idx, w


# ----------------------------------------------------------------------------------------------
# Permutation

def permute(idx, E: int):
    """Expert histogram, exclusive scan and stable grouping of the rows (reading "permutation").

    counts[e] is the number of rows routed to e, and offsets is its exclusive prefix sum
    (E+1 entries). row_src[pos] is the flat row r stored at position pos, and tk_row[r] is its
    inverse. No row is dropped: every one of the T*k rows gets a position (MarkTechPost,
    "Three design decisions that matter", ring token buffer paragraph).
    """
    flat = np.asarray(idx).reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    row_src = np.argsort(flat, kind="stable").astype(np.int32)
    tk_row = np.empty_like(row_src)
    tk_row[row_src] = np.arange(flat.size, dtype=np.int32)
    return counts, offsets, row_src, tk_row


# ----------------------------------------------------------------------------------------------
# Layer

def _silu(z):
    return z / (1.0 + np.exp(-z))


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def _identity(a, axis=-1):
    return a


def _rounder(storage):
    return bf16_round if storage == "bf16" else (lambda a: a)


def expert_forward(x, w1, w2, *, rnd, mxq=_identity):
    """One expert's forward over its rows x [c, d] (readings "expert", "storage_bf16", "mxfp8").

    [g | u] = x W1_e^T, a = silu(g) * u, o = a W2_e^T. With bf16 storage H = [g | u] is stored
    rounded, A is rounded once from the unrounded g and u, and the down projection reads the
    stored A. ``mxq`` is the MXFP8 image taken of both operands of each GEMM (identity in BF16
    mode). Returns (H [c, 2I], A [c, I], O_exact [c, d]); the caller rounds O where it is stored.
    """
    I = w1.shape[0] // 2
    x = mxq(x)
    w1 = mxq(np.asarray(w1, np.float64))
    g = x @ w1[:I].T
    u = x @ w1[I:].T
    h = np.concatenate([rnd(g), rnd(u)], axis=1)
    a = rnd(_silu(g) * u)
    o = mxq(a) @ mxq(np.asarray(w2, np.float64)).T
    return h, a, o


def _mx_images(precision):
    """The MX image taken of the GEMM operands in a precision mode (reading "mxfp8" or "mxfp4"),
    or None in BF16 mode."""
    return {"bf16": None, "mxfp8": mx.qdq, "mxfp4": mx.qdq4}[precision]


def expert_backward(x, dy, wv, h, a, o_used, w1, w2, *, rnd, mxq=None, mx_wgrad=False):
    """One expert's backward over its rows (readings "router_grad", "storage_bf16", "mxfp8",
    "mxfp4").

    x and dy are the rows' tokens and upstream gradients, wv [c, 1] their routing weights, h and
    a the stored forward H and A, o_used the stored O. Per row:
    * dw = <dy, o>, the router-weight gradient; in MXFP8 mode the fused <dA', a> with dA' from
      the quantised dgrad GEMM;
    * dA = w * (dy W2_e); dg = dA * u * s * (1 + g (1 - s)) with s = sigmoid(g), du = dA * silu(g),
      from the stored g and u; dH = [dg | du] is stored (rounded);
    * dXp = dH W1_e, stored (rounded).
    Over the expert's rows: dW2_e = sum (w dy) outer a, dW1_e = sum dH outer x. In an MX mode
    (mxq the MXFP8 or MXFP4 image) both dgrad GEMMs take MX images along their reduction axes and
    x enters dW1 as its MX image. With mx_wgrad (reading "mxfp8_wgrad") both weight-gradient
    products take MXFP8 images of their operands along the expert's positions.
    Returns (dw [c], dH [c, 2I], dXp [c, d], dW1_e [2I, d], dW2_e [d, I]).
    """
    I = h.shape[1] // 2
    w1 = np.asarray(w1, np.float64)
    w2 = np.asarray(w2, np.float64)
    if mxq is not None:
        dAp = mxq(dy) @ mxq(w2.T).T            # W2 [d, I] quantised along d
        dw = np.sum(dAp * a, axis=1)
    else:
        dAp = dy @ w2
        dw = np.sum(dy * o_used, axis=1)
    dA = wv * dAp
    g = h[:, :I]
    u = h[:, I:]
    s = _sigmoid(g)
    dg = dA * u * s * (1.0 + g * (1.0 - s))
    du = dA * (g * s)
    dh = rnd(np.concatenate([dg, du], axis=1))
    if mxq is not None:
        dxp = rnd(mxq(dh) @ mxq(w1.T).T)        # W1 [2I, d] quantised along 2I
    else:
        dxp = rnd(dh @ w1)
    xr = mxq(x) if mxq is not None else x
    if mx_wgrad:
        dW2 = mx.qdq_segment(wv * dy).T @ mx.qdq_segment(a)
        dW1 = mx.qdq_segment(dh).T @ mx.qdq_segment(xr)
    else:
        dW2 = (wv * dy).T @ a
        dW1 = dh.T @ xr
    return dw, dh, dxp, dW1, dW2


def gather_sum(R, w, tk_row, k):
    """out_t = sum_j w_tj R[pos(t, j)], j ascending, unrounded; w = None sums without weights.
    The combine (reading "combine") and the sum of a token's dXp rows in backward."""
    T = len(tk_row) // k
    out = np.zeros((T, R.shape[1]))
    for j in range(k):
        rows = R[tk_row[np.arange(T) * k + j]]
        out += rows if w is None else w[:, j:j + 1] * rows
    return out


def router_backward(w, idx, dw, E):
    """Top-k softmax backward: dlogit_j = w_j (dw_j - sum_{i in S} w_i dw_i) on the selected set
    S, and exactly 0 off it (reading "router_grad": nothing is detached). Returns [T, E]."""
    dl = w * (dw - np.sum(w * dw, axis=1, keepdims=True))
    dlogits = np.zeros((w.shape[0], E))
    np.put_along_axis(dlogits, idx, dl, axis=1)
    return dlogits


def _routing(X, Wr, k, topk_idx, topk_w, logits):
    if topk_idx is None:
        L = router_logits_fp32(X, Wr) if logits == "fp32" else router_logits_fp64(X, Wr)
        idx, w = route_topk(L, k)
        return idx, w, k, L
    idx = np.asarray(topk_idx, np.int32)
    return idx, np.asarray(topk_w, np.float64), idx.shape[1], None


def forward(X, W1, W2, *, Wr=None, k=None, topk_idx=None, topk_w=None,
            storage="bf16", logits="fp32", experts=None, precision="bf16") -> dict:
    """Forward pass of the MoE layer.

    Routing comes from the router (Wr, k) or is given (topk_idx, topk_w). ``experts`` limits
    the expert math to a subset, for bounded CPU timings; rows of the other experts stay NaN.

    Per expert e and each of its rows (``expert_forward``): [g | u] = x W1_e^T,
    a = silu(g) * u, o = a W2_e^T. Then y_t = sum_j w_tj o_tj, j ascending (reading
    "combine"). With precision="mxfp8" (or "mxfp4") the two GEMMs take MXFP8 (MXFP4) images of
    their operands (readings "mxfp8", "mxfp4"). Returns a dict of every intermediate the GPU path
    also produces.
    """
    mxq = _mx_images(precision) or _identity
    X = np.asarray(X, np.float64)
    T, d = X.shape
    E, twoI, _ = W1.shape
    I = twoI // 2
    rnd = _rounder(storage)
    out = {}
    idx, w, k, L = _routing(X, Wr, k, topk_idx, topk_w, logits)
    if L is not None:
        out["logits"] = L
    counts, offsets, row_src, tk_row = permute(idx, E)
    Tk = T * k
    H = np.full((Tk, twoI), np.nan)
    A = np.full((Tk, I), np.nan)
    O = np.full((Tk, d), np.nan)
    O_exact = np.full((Tk, d), np.nan)
    ex = range(E) if experts is None else experts
    for e in ex:
        p0, p1 = int(offsets[e]), int(offsets[e + 1])
        if p1 == p0:
            continue
        tok = row_src[p0:p1] // k
        H[p0:p1], A[p0:p1], O_exact[p0:p1] = expert_forward(X[tok], W1[e], W2[e], rnd=rnd,
                                                            mxq=mxq)
        O[p0:p1] = rnd(O_exact[p0:p1])
    Y = gather_sum(O, w, tk_row, k)
    out.update(idx=idx, w=w, counts=counts, offsets=offsets, row_src=row_src, tk_row=tk_row,
               H=H, A=A, O=O, O_exact=O_exact, Y=rnd(Y), k=k, storage=storage,
               routed=topk_idx is None, precision=precision)
    return out


def backward(fwd: dict, X, W1, W2, dY, *, Wr=None, experts=None, wgrad="bf16",
             dw_dtype="fp32") -> dict:
    """Backward pass: gradients of L = <Y, dY> with respect to every input.

    Per row at position pos (token t, slot j, expert e, weight w), by ``expert_backward``:
    * dw = <dY_t, o>, the router-weight gradient (reading "router_grad");
    * dA = w * (dY_t W2_e);
    * dg = dA * u * s * (1 + g (1 - s)) with s = sigmoid(g), and du = dA * silu(g);
    * dXp = [dg | du] W1_e;
    * dW2_e = sum over rows of (w dY_t) outer a;
    * dW1_e = sum over rows of [dg | du] outer x_t.
    Per token, over its selected set S (``router_backward``):
    * dlogit_j = w_j (dw_j - sum_{i in S} w_i dw_i), and 0 off S;
    * dX_t = sum_j dXp_tj + sum_j dlogit_j Wr_{e_j};
    * dWr = dlogits^T X.
    With bf16 storage, dH, dXp and dX are rounded where the GPU stores them, and the stored H,
    A and dH feed the later steps. Empty experts get all-zero dW1_e and dW2_e blocks.
    ``experts`` limits the expert math to a subset (rows of other experts stay NaN). dW1 and dW2
    then hold one block per listed expert, in the order listed in out["experts"].
    In MXFP8 (MXFP4) mode (readings "mxfp8", "mxfp4") both dgrad GEMMs take MXFP8 (MXFP4)
    images of their operands, dw is
    <dA', A>, and Xp enters dW1 and dWr as its MX image. wgrad="mxfp8" (MXFP8 mode only,
    reading "mxfp8_wgrad") quantises both operands of both weight-gradient products along the
    expert's positions. dw_dtype="bf16" (reading "dw_bf16") rounds each dW1 and dW2 element once
    to bf16.
    """
    mxq = _mx_images(fwd.get("precision", "bf16"))
    assert wgrad in ("bf16", "mxfp8") and (wgrad == "bf16" or fwd.get("precision") == "mxfp8"), \
        "MXFP8 wgrad needs MXFP8 mode"
    assert dw_dtype in ("fp32", "bf16")
    X = np.asarray(X, np.float64)
    dY = np.asarray(dY, np.float64)
    T, d = X.shape
    E, twoI, _ = W1.shape
    I = twoI // 2
    k = fwd["k"]
    rnd = _rounder(fwd["storage"])
    offsets, row_src, tk_row = fwd["offsets"], fwd["row_src"], fwd["tk_row"]
    w_flat = fwd["w"].reshape(-1)
    Tk = T * k
    dw_pos = np.full(Tk, np.nan)
    dH = np.full((Tk, twoI), np.nan)
    dXp = np.full((Tk, d), np.nan)
    ex = list(range(E)) if experts is None else list(experts)
    dW1 = np.zeros((len(ex), twoI, d))
    dW2 = np.zeros((len(ex), d, I))
    for slot, e in enumerate(ex):
        p0, p1 = int(offsets[e]), int(offsets[e + 1])
        if p1 == p0:
            continue
        rows = row_src[p0:p1]
        tok = rows // k
        dw_pos[p0:p1], dH[p0:p1], dXp[p0:p1], dW1[slot], dW2[slot] = expert_backward(
            X[tok], dY[tok], w_flat[rows][:, None], fwd["H"][p0:p1], fwd["A"][p0:p1],
            fwd["O"][p0:p1], W1[e], W2[e], rnd=rnd, mxq=mxq, mx_wgrad=wgrad == "mxfp8")
    if dw_dtype == "bf16":
        dW1, dW2 = bf16_round(dW1), bf16_round(dW2)
    dw = dw_pos[tk_row].reshape(T, k)
    dXsum = gather_sum(dXp, None, tk_row, k)
    out = dict(dw=dw, dH=dH, dXp=dXp, dW1=dW1, dW2=dW2, experts=ex)
    if fwd["routed"]:
        dlogits = router_backward(fwd["w"], fwd["idx"], dw, E)
        dXsum = dXsum + dlogits @ np.asarray(Wr, np.float64)
        out["dlogits"] = dlogits
        out["dWr"] = dlogits.T @ (mxq(X) if mxq is not None else X)
    out["dX"] = rnd(dXsum)
    return out


def layer(X, W1, W2, dY, *, Wr=None, k=None, topk_idx=None, topk_w=None, storage="bf16",
          precision="bf16", on_expert=None, wgrad="bf16", dw_dtype="fp32") -> dict:
    """Forward and backward of the whole layer, one expert at a time.

    The same steps as ``forward`` followed by ``backward``, in the same order and arithmetic,
    but each expert's forward and backward run back to back and its weight gradients are handed
    to ``on_expert(e, dW1_e, dW2_e)`` instead of being kept. Host memory thus stays at the
    per-row intermediates plus one expert's dW, which lets the oracle cover every token of the
    largest workloads. Returns the forward intermediates and the backward results of
    ``forward``/``backward`` (without dW1 and dW2).
    """
    assert dw_dtype in ("fp32", "bf16")
    dwr = bf16_round if dw_dtype == "bf16" else _identity
    mxb = _mx_images(precision)
    mxq = mxb or _identity
    X = np.asarray(X, np.float64)
    dY = np.asarray(dY, np.float64)
    T, d = X.shape
    E, twoI, _ = W1.shape
    I = twoI // 2
    rnd = _rounder(storage)
    idx, w, k, L = _routing(X, Wr, k, topk_idx, topk_w, "fp32")
    counts, offsets, row_src, tk_row = permute(idx, E)
    Tk = T * k
    w_flat = w.reshape(-1)
    H = np.full((Tk, twoI), np.nan)
    A = np.full((Tk, I), np.nan)
    O = np.full((Tk, d), np.nan)
    dw_pos = np.full(Tk, np.nan)
    dH = np.full((Tk, twoI), np.nan)
    dXp = np.full((Tk, d), np.nan)
    for e in range(E):
        p0, p1 = int(offsets[e]), int(offsets[e + 1])
        if p1 == p0:
            if on_expert is not None:
                on_expert(e, np.zeros((twoI, d)), np.zeros((d, I)))
            continue
        rows = row_src[p0:p1]
        tok = rows // k
        w1, w2 = W1[e], W2[e]
        H[p0:p1], A[p0:p1], o = expert_forward(X[tok], w1, w2, rnd=rnd, mxq=mxq)
        O[p0:p1] = rnd(o)
        dw_pos[p0:p1], dH[p0:p1], dXp[p0:p1], dW1, dW2 = expert_backward(
            X[tok], dY[tok], w_flat[rows][:, None], H[p0:p1], A[p0:p1], O[p0:p1], w1, w2,
            rnd=rnd, mxq=mxb, mx_wgrad=wgrad == "mxfp8")
        if on_expert is not None:
            on_expert(e, dwr(dW1), dwr(dW2))
    out = dict(idx=idx, w=w, counts=counts, offsets=offsets, row_src=row_src, tk_row=tk_row,
               H=H, A=A, O=O, Y=rnd(gather_sum(O, w, tk_row, k)), k=k)
    dw = dw_pos[tk_row].reshape(T, k)
    dXsum = gather_sum(dXp, None, tk_row, k)
    out.update(dw=dw, dH=dH, dXp=dXp)
    if L is not None:
        out["logits"] = L
        dlogits = router_backward(w, idx, dw, E)
        dXsum = dXsum + dlogits @ np.asarray(Wr, np.float64)
        out["dlogits"] = dlogits
        out["dWr"] = dlogits.T @ (mxb(X) if mxb is not None else X)
    out["dX"] = rnd(dXsum)
    return out
