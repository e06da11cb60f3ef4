"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

At these sizes the oracle cannot redo the whole layer in seconds, so each output is checked
where the oracle can compute it piece by piece:
* Routing (fp32 logits in the stated order, top-k, weights) and the permutation maps are
  recomputed for every token and compared bit for bit (weights within 1e-6). So is the permuted
  token copy.
* Y, dX, d_topk_w and the saved H and A rows are checked on sampled tokens. Each depends only on
  its own token, so the oracle runs on those tokens alone.
* dW1 and dW2 are checked on sampled experts. The oracle routes every token but does the
  expert math of those experts only.
* dWr is checked against dlogits^T X, formed in float64 from the layer's own d_topk_w, whose
  sampled rows are oracle-checked, and from its routing weights.
Two runs, and the persistent grid, must agree bitwise at the DeepSeek-V3 shape.
"""
import numpy as np
import pytest
import torch

import oracle
import workload
from tests._gpu import (DEV, MoeLayer, _announce, _np, assert_bitwise_equal, m, outputs,
                        run_gpu)
from tests._util import assert_act, assert_grad

pytestmark = pytest.mark.gpu


def _sample(n_total, n, seed):
    rng = np.random.default_rng(seed)
    pick = rng.choice(n_total, size=min(n, n_total), replace=False)
    return np.unique(np.concatenate([[0, n_total - 1], pick])).astype(np.int64)


def _check_routing_and_permutation(L, inp, X):
    cfg = inp["cfg"]
    E, k = cfg["E"], cfg["k"]
    if "Wr" in inp:
        logits = oracle.router_logits_fp32(X, _np(inp["Wr"]))
        np.testing.assert_array_equal(_np(L.logits), logits)
        idx, w = oracle.route_topk(logits, k)
        np.testing.assert_array_equal(_np(L.topk_idx), idx)
        np.testing.assert_allclose(_np(L.topk_w), w, rtol=0, atol=1e-6)
    else:
        idx = _np(inp["topk_idx"])
    counts, offsets, row_src, tk_row = oracle.permute(idx, E)
    np.testing.assert_array_equal(_np(L.counts), counts)
    np.testing.assert_array_equal(_np(L.offsets), offsets)
    np.testing.assert_array_equal(_np(L.row_src), row_src)
    np.testing.assert_array_equal(_np(L.tk_row), tk_row)
    return counts


def _check_xp(L, X_dev, k, slot=0):
    src = L.row_src.long() // k
    assert torch.equal(L.xp(slot).view(torch.int16), X_dev[src].view(torch.int16))


def _check_tokens(L, inp, X, dY, tok, W1h, W2h):
    """Per-token outputs on the sampled tokens against the oracle run on those tokens alone."""
    k = inp["cfg"]["k"]
    if "Wr" in inp:
        Wr = _np(inp["Wr"])
        f = oracle.forward(X[tok], W1h, W2h, Wr=Wr, k=k)
        b = oracle.backward(f, X[tok], W1h, W2h, dY[tok], Wr=Wr)
    else:
        f = oracle.forward(X[tok], W1h, W2h, topk_idx=_np(inp["topk_idx"])[tok],
                           topk_w=_np(inp["topk_w"])[tok])
        b = oracle.backward(f, X[tok], W1h, W2h, dY[tok])
    t_dev = torch.from_numpy(tok).to(DEV)
    assert_act("Y[tokens]", _np(L.y[t_dev]), f["Y"])
    assert_act("dX[tokens]", _np(L.dx[t_dev]), b["dX"])
    assert_grad("d_topk_w[tokens]", _np(L.d_topk_w[t_dev]), b["dw"])
    rows = (tok[:, None] * k + np.arange(k)).reshape(-1)
    pos = L.tk_row[torch.from_numpy(rows).to(DEV)].long()
    sub = f["tk_row"][np.arange(len(tok) * k)]
    assert_act("H[rows]", _np(L.H()[pos]), f["H"][sub])
    assert_act("A[rows]", _np(L.A()[pos]), f["A"][sub])


def _check_experts(L, inp, X, dY, experts, W1h, W2h):
    """dW1 and dW2 of the listed experts against the oracle (all tokens routed, expert math of
    those experts only)."""
    k = inp["cfg"]["k"]
    if "Wr" in inp:
        Wr = _np(inp["Wr"])
        f = oracle.forward(X, W1h, W2h, Wr=Wr, k=k, experts=experts)
        b = oracle.backward(f, X, W1h, W2h, dY, Wr=Wr, experts=experts)
    else:
        f = oracle.forward(X, W1h, W2h, topk_idx=_np(inp["topk_idx"]),
                           topk_w=_np(inp["topk_w"]), experts=experts)
        b = oracle.backward(f, X, W1h, W2h, dY, experts=experts)
    for i, e in enumerate(experts):
        assert_grad(f"dW1[{e}]", _np(L.dw1[e]), b["dW1"][i])
        assert_grad(f"dW2[{e}]", _np(L.dw2[e]), b["dW2"][i])
    return b


def _check_dwr(L, X):
    """dWr = dlogits^T X, with dlogit_j = w_j (dw_j - sum_i w_i dw_i) from the layer's own
    (sample-checked) d_topk_w and routing weights, in float64."""
    w = _np(L.topk_w).astype(np.float64)
    dw = _np(L.d_topk_w).astype(np.float64)
    idx = _np(L.topk_idx)
    dl = w * (dw - np.sum(w * dw, axis=1, keepdims=True))
    E = L.E
    dlogits = np.zeros((X.shape[0], E))
    np.put_along_axis(dlogits, idx, dl, axis=1)
    assert_grad("dWr", _np(L.dwr), dlogits.T @ X.astype(np.float64))


def test_dsv3_full_size_parity():
    _announce("[full] dsv3 T=2048 d=7168 E=256 k=8 I=2048 seed 0, one-shot grids")
    inp = workload.make_inputs("dsv3", seed=0, device=DEV)
    L = run_gpu(inp)
    X, dY = _np(inp["X"]), _np(inp["dY"])
    counts = _check_routing_and_permutation(L, inp, X)
    _check_xp(L, inp["X"], inp["cfg"]["k"])
    W1h, W2h = workload.HostExperts(inp["W1"]), workload.HostExperts(inp["W2"])
    _check_tokens(L, inp, X, dY, _sample(X.shape[0], 10, seed=1), W1h, W2h)
    heavy = int(np.argmax(counts))
    light = int(np.argmin(np.where(counts > 0, counts, 1 << 30)))
    _check_experts(L, inp, X, dY, sorted({heavy, light, 0}), W1h, W2h)
    _check_dwr(L, X)


def test_dsv3_two_runs_and_persistent_grid_are_bitwise_identical():
    _announce("[full] dsv3 determinism: one-shot twice, then persistent")
    inp = workload.make_inputs("dsv3", seed=3, device=DEV)
    L = run_gpu(inp)
    ref = outputs(L, True)
    del L
    torch.cuda.empty_cache()
    L = run_gpu(inp)
    assert_bitwise_equal(ref, outputs(L, True, clone=False))
    del L
    torch.cuda.empty_cache()
    L = run_gpu(inp, persistent=True)
    assert_bitwise_equal(ref, outputs(L, True, clone=False))


def test_local_zipf_full_size_parity():
    _announce("[full] local_zipf 16384 rows d=7168 E=8 k=1 I=2048 seed 0")
    inp = workload.make_inputs("local_zipf", seed=0, device=DEV)
    L = run_gpu(inp)
    X, dY = _np(inp["X"]), _np(inp["dY"])
    counts = _check_routing_and_permutation(L, inp, X)
    assert counts.sum() == X.shape[0] and np.count_nonzero(counts == 0) == 3
    _check_xp(L, inp["X"], 1)
    W1h, W2h = workload.HostExperts(inp["W1"]), workload.HostExperts(inp["W2"])
    _check_tokens(L, inp, X, dY, _sample(X.shape[0], 12, seed=2), W1h, W2h)
    nonempty = np.flatnonzero(counts)
    light = int(nonempty[np.argmin(counts[nonempty])])
    empty = int(np.flatnonzero(counts == 0)[0])
    _check_experts(L, inp, X, dY, sorted({light, empty}), W1h, W2h)
    assert torch.count_nonzero(L.dw1[empty]) == 0 and torch.count_nonzero(L.dw2[empty]) == 0


def test_stream_full_size_ring_walk():
    """8 microbatches of 2368 tokens through a 512 MiB ring (2 slots). Forward runs 0..7;
    backward runs 7..0, re-permuting microbatches whose slot was overwritten, and accumulates
    the weight gradients."""
    _announce("[full] stream 8 x T=2368 d=4096 E=512 k=10 I=1024, 512 MiB ring, seed 0")
    inp = workload.make_inputs("stream", seed=0, device=DEV)
    cfg = inp["cfg"]
    T, d, E, k, I, nmb = cfg["T"], cfg["d"], cfg["E"], cfg["k"], cfg["I"], cfg["microbatches"]
    S = cfg["ring_bytes"] // m.moe_query(m.make_cfg(T, d, E, k, I)).ring_slot
    assert S == 2
    L = MoeLayer(T, d, E, k, I, device=DEV, ring_slots=S)
    assert L.ring.numel() <= cfg["ring_bytes"]
    saved = [torch.empty_like(L.saved) for _ in range(nmb)]
    routing, ys = [], []
    for i in range(nmb):
        L.route(inp["X"][i], inp["Wr"])
        L.permute(inp["X"][i], slot=i % S)
        L.forward(inp["W1"], inp["W2"], slot=i % S, saved=saved[i])
        ys.append(L.y.clone())
        routing.append(tuple(t.clone() for t in (L.topk_idx, L.topk_w, L.counts, L.offsets,
                                                  L.row_src, L.tk_row)))
    dxs, dtws = [None] * nmb, [None] * nmb
    for i in reversed(range(nmb)):
        for dst, src in zip((L.topk_idx, L.topk_w, L.counts, L.offsets, L.row_src, L.tk_row),
                            routing[i]):
            dst.copy_(src)
        if i < nmb - S:
            L.permute(inp["X"][i], slot=i % S)  # replay: the slot was overwritten
        L.backward(inp["Wr"], inp["W1"], inp["W2"], inp["dY"][i], slot=i % S,
                   accumulate=(i != nmb - 1), saved=saved[i])
        dxs[i] = L.dx.clone()
        dtws[i] = L.d_topk_w.clone()
    torch.cuda.synchronize()
    Wr = _np(inp["Wr"])
    W1h, W2h = workload.HostExperts(inp["W1"]), workload.HostExperts(inp["W2"])
    experts = None
    dW1 = dW2 = None
    for i in range(nmb):
        X, dY = _np(inp["X"][i]), _np(inp["dY"][i])
        tok = _sample(T, 4, seed=10 + i)
        f = oracle.forward(X[tok], W1h, W2h, Wr=Wr, k=k)
        b = oracle.backward(f, X[tok], W1h, W2h, dY[tok], Wr=Wr)
        t_dev = torch.from_numpy(tok).to(DEV)
        np.testing.assert_array_equal(_np(routing[i][0][t_dev]), f["idx"])
        assert_act(f"Y[{i}][tokens]", _np(ys[i][t_dev]), f["Y"])
        assert_act(f"dX[{i}][tokens]", _np(dxs[i][t_dev]), b["dX"])
        assert_grad(f"d_topk_w[{i}][tokens]", _np(dtws[i][t_dev]), b["dw"])
        if experts is None:
            c = _np(routing[0][2])
            experts = sorted({int(np.argmax(c)), 0})
        fe = oracle.forward(X, W1h, W2h, Wr=Wr, k=k, experts=experts)
        np.testing.assert_array_equal(_np(routing[i][0]), fe["idx"])
        be = oracle.backward(fe, X, W1h, W2h, dY, Wr=Wr, experts=experts)
        dW1 = be["dW1"] if dW1 is None else dW1 + be["dW1"]
        dW2 = be["dW2"] if dW2 is None else dW2 + be["dW2"]
    for j, e in enumerate(experts):
        assert_grad(f"dW1[{e}] (sum of 8)", _np(L.dw1[e]), dW1[j])
        assert_grad(f"dW2[{e}] (sum of 8)", _np(L.dw2[e]), dW2[j])
