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


def forward(X, W1, W2, *, Wr=None, k=None, topk_idx=None, topk_w=None,
            storage="bf16", logits="fp32", experts=None, precision="bf16") -> dict:
    """Forward pass of the MoE layer.

    Routing comes from the router (Wr, k) or is given (topk_idx, topk_w). ``experts`` limits
    the expert math to a subset, for bounded CPU timings; rows of the other experts stay NaN.

    Per expert e and each of its rows (readings "expert", "storage_bf16"):
    [g | u] = x W1_e^T, a = silu(g) * u, o = a W2_e^T. Then y_t = sum_j w_tj o_tj, j ascending
    (reading "combine"). With precision="mxfp8" the two GEMMs take MXFP8 images of their
    operands (reading "mxfp8"). Returns a dict of every intermediate the GPU path also produces.
    """
    mxq = mx.qdq if precision == "mxfp8" else (lambda a, axis=-1: a)
    X = np.asarray(X, np.float64)
    T, d = X.shape
    E, twoI, _ = W1.shape
    I = twoI // 2
    rnd = bf16_round if storage == "bf16" else (lambda a: a)
    out = {}
    if topk_idx is None:
        L = router_logits_fp32(X, Wr) if logits == "fp32" else router_logits_fp64(X, Wr)
        idx, w = route_topk(L, k)
        out["logits"] = L
    else:
        idx = np.asarray(topk_idx, np.int32)
        w = np.asarray(topk_w, np.float64)
        k = idx.shape[1]
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
        x = mxq(X[tok])
        w1 = mxq(np.asarray(W1[e], np.float64))
        g = x @ w1[:I].T
        u = x @ w1[I:].T
        H[p0:p1, :I] = rnd(g)
        H[p0:p1, I:] = rnd(u)
        a = rnd(_silu(g) * u)
        A[p0:p1] = a
        o = mxq(a) @ mxq(np.asarray(W2[e], np.float64)).T
        O_exact[p0:p1] = o
        O[p0:p1] = rnd(o)
    Y = np.zeros((T, d))
    for j in range(k):
        Y += w[:, j:j + 1] * O[tk_row[np.arange(T) * k + j]]
    out.update(idx=idx, w=w, counts=counts, offsets=offsets, row_src=row_src, tk_row=tk_row,
               H=H, A=A, O=O, O_exact=O_exact, Y=rnd(Y), k=k, storage=storage,
               routed=topk_idx is None, precision=precision)
    return out


def backward(fwd: dict, X, W1, W2, dY, *, Wr=None, experts=None) -> dict:
    """Backward pass: gradients of L = <Y, dY> with respect to every input.

    Per row at position pos (token t, slot j, expert e, weight w):
    * dw = <dY_t, o>, the router-weight gradient (reading "router_grad");
    * dA = w * (dY_t W2_e);
    * dg = dA * u * s * (1 + g (1 - s)) with s = sigmoid(g), and du = dA * silu(g);
    * dXp = [dg | du] W1_e;
    * dW2_e = sum over rows of (w dY_t) outer a;
    * dW1_e = sum over rows of [dg | du] outer x_t.
    Per token, over its selected set S:
    * dlogit_j = w_j (dw_j - sum_{i in S} w_i dw_i), and 0 off S;
    * dX_t = sum_j dXp_tj + sum_j dlogit_j Wr_{e_j};
    * dWr = dlogits^T X.
    With bf16 storage, dH, dXp and dX are rounded where the GPU stores them, and the stored H,
    A and dH feed the later steps. Empty experts get all-zero dW1_e and dW2_e blocks.
    ``experts`` limits the expert math to a subset (rows of other experts stay NaN). dW1 and dW2
    then hold one block per listed expert, in the order listed in out["experts"].
    In MXFP8 mode (reading "mxfp8") both dgrad GEMMs take MXFP8 images of their operands, dw is
    <dA', A>, and Xp enters dW1 and dWr as its MXFP8 image.
    """
    mxmode = fwd.get("precision", "bf16") == "mxfp8"
    X = np.asarray(X, np.float64)
    dY = np.asarray(dY, np.float64)
    T, d = X.shape
    E, twoI, _ = W1.shape
    I = twoI // 2
    k = fwd["k"]
    rnd = bf16_round if fwd["storage"] == "bf16" else (lambda a: a)
    offsets, row_src, tk_row = fwd["offsets"], fwd["row_src"], fwd["tk_row"]
    w_flat = fwd["w"].reshape(-1)
    O_used = fwd["O"]
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
        wv = w_flat[rows][:, None]
        dy = dY[tok]
        w2 = np.asarray(W2[e], np.float64)
        w1 = np.asarray(W1[e], np.float64)
        if mxmode:
            dAp = mx.qdq(dy) @ mx.qdq(w2.T).T      # W2 [d, I] quantised along d
            dw_pos[p0:p1] = np.sum(dAp * fwd["A"][p0:p1], axis=1)
        else:
            dAp = dy @ w2
            dw_pos[p0:p1] = np.sum(dy * O_used[p0:p1], axis=1)
        dA = wv * dAp
        g = fwd["H"][p0:p1, :I]
        u = fwd["H"][p0:p1, I:]
        s = _sigmoid(g)
        dg = dA * u * s * (1.0 + g * (1.0 - s))
        du = dA * (g * s)
        dh = rnd(np.concatenate([dg, du], axis=1))
        dH[p0:p1] = dh
        if mxmode:
            dXp[p0:p1] = rnd(mx.qdq(dh) @ mx.qdq(w1.T).T)  # W1 [2I, d] quantised along 2I
        else:
            dXp[p0:p1] = rnd(dh @ w1)
        dW2[slot] = (wv * dy).T @ fwd["A"][p0:p1]
        dW1[slot] = dh.T @ (mx.qdq(X[tok]) if mxmode else X[tok])
    dw = dw_pos[tk_row].reshape(T, k)
    dXsum = np.zeros((T, d))
    for j in range(k):
        dXsum += dXp[tk_row[np.arange(T) * k + j]]
    out = dict(dw=dw, dH=dH, dXp=dXp, dW1=dW1, dW2=dW2, experts=ex)
    if fwd["routed"]:
        w = fwd["w"]
        idx = fwd["idx"]
        dl = w * (dw - np.sum(w * dw, axis=1, keepdims=True))
        dlogits = np.zeros((T, E))
        np.put_along_axis(dlogits, idx, dl, axis=1)
        Wr64 = np.asarray(Wr, np.float64)
        dXsum = dXsum + dlogits @ Wr64
        out["dlogits"] = dlogits
        out["dWr"] = dlogits.T @ (mx.qdq(X) if mxmode else X)
    out["dX"] = rnd(dXsum)
    return out
