"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

The oracle walks the experts one at a time (``oracle.layer``): it keeps every per-row
intermediate and hands over one expert's weight gradients at a time, so it covers every token
of the full workloads in host memory:
* routing (fp32 logits in the stated order, top-k, weights) and the permutation maps, bit for
  bit (weights within 1e-6), and the permuted token copy;
* every token's Y, dX and d_topk_w, and every row's H, A, O, dH and dXp;
* dWr against the oracle's own dlogits^T X;
* dW1 and dW2 of sampled experts (all experts of the local slice).
Two runs, and the persistent grid, must agree bitwise at the DeepSeek-V3 shape; two runs must
agree bitwise on the local slice and on the streaming macrobatch as well.
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


def _check_xp(L, X_dev, k, slot=0):
    src = L.row_src.long() // k
    assert torch.equal(L.xp(slot).view(torch.int16), X_dev[src].view(torch.int16))


def _whole_layer(L, inp, check_experts, tol_act=None, tol_grad=None):
    """Every output of one GPU step against oracle.layer on the same inputs."""
    cfg = inp["cfg"]
    k = cfg["k"]
    X, dY = _np(inp["X"]), _np(inp["dY"])
    W1h, W2h = workload.HostExperts(inp["W1"]), workload.HostExperts(inp["W2"])
    kw = dict(Wr=_np(inp["Wr"]), k=k) if "Wr" in inp else dict(
        topk_idx=_np(inp["topk_idx"]), topk_w=_np(inp["topk_w"]))
    prec = "mxfp8" if cfg.get("precision") == "mxfp8" else "bf16"
    ta = {} if tol_act is None else {"tol": tol_act}
    tg = {} if tol_grad is None else {"tol": tol_grad}
    checked = []

    def on_expert(e, dW1, dW2):
        if e in check_experts:
            assert_grad(f"dW1[{e}]", _np(L.dw1[e]), dW1, **tg)
            assert_grad(f"dW2[{e}]", _np(L.dw2[e]), dW2, **tg)
            checked.append(e)
        if e % 32 == 31:
            _announce(f"  oracle: experts 0..{e} done")

    lay = oracle.layer(X, W1h, W2h, dY, precision=prec, on_expert=on_expert, **kw)
    assert sorted(checked) == sorted(check_experts)
    if "Wr" in inp:
        np.testing.assert_array_equal(_np(L.logits), lay["logits"])
        np.testing.assert_array_equal(_np(L.topk_idx), lay["idx"])
        np.testing.assert_allclose(_np(L.topk_w), lay["w"], rtol=0, atol=1e-6)
    for n in ("counts", "offsets", "row_src", "tk_row"):
        np.testing.assert_array_equal(_np(getattr(L, n)), lay[n], err_msg=n)
    _announce("  routing and permutation bit-exact over every token")
    for n, got in (("H", L.H()), ("A", L.A()), ("O", L.O()), ("dH", L.dH()), ("dXp", L.dXp())):
        assert_act(f"{n} (every row)", _np(got), lay[n], **ta)
    assert_act("Y (every token)", _np(L.y), lay["Y"], **ta)
    assert_act("dX (every token)", _np(L.dx), lay["dX"], **ta)
    assert_grad("d_topk_w (every token)", _np(L.d_topk_w), lay["dw"], **tg)
    if "Wr" in inp:
        assert_grad("dWr (oracle dlogits)", _np(L.dwr), lay["dWr"], **tg)
    return lay


def test_dsv3_every_token_against_the_oracle():
    _announce("[full] dsv3 T=2048 d=7168 E=256 k=8 I=2048 seed 0, one-shot grids, every token")
    inp = workload.make_inputs("dsv3", seed=0, device=DEV)
    L = run_gpu(inp)
    _check_xp(L, inp["X"], inp["cfg"]["k"])
    counts = _np(L.counts)
    heavy = int(np.argmax(counts))
    light = int(np.argmin(np.where(counts > 0, counts, 1 << 30)))
    experts = sorted({heavy, light} | set(range(0, 256, 16)))
    _whole_layer(L, inp, experts)


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


def test_local_zipf_every_row_against_the_oracle():
    _announce("[full] local_zipf 16384 rows d=7168 E=8 k=1 I=2048 seed 0, every row")
    inp = workload.make_inputs("local_zipf", seed=0, device=DEV)
    L = run_gpu(inp)
    counts = _np(L.counts)
    assert counts.sum() == inp["cfg"]["T"] and np.count_nonzero(counts == 0) == 3
    assert counts.max() > 0.4 * inp["cfg"]["T"]
    _check_xp(L, inp["X"], 1)
    _whole_layer(L, inp, list(range(8)))
    for e in np.flatnonzero(counts == 0):
        assert torch.count_nonzero(L.dw1[e]) == 0 and torch.count_nonzero(L.dw2[e]) == 0


def test_local_zipf_two_runs_are_bitwise_identical():
    _announce("[full] local_zipf determinism: two runs")
    inp = workload.make_inputs("local_zipf", seed=4, device=DEV)
    ref = outputs(run_gpu(inp), False)
    torch.cuda.empty_cache()
    assert_bitwise_equal(ref, outputs(run_gpu(inp), False, clone=False))


def _stream_run(inp):
    """8 microbatches through a 2-slot ring: forward 0..7, then backward 7..0, re-permuting the
    microbatches whose slot was overwritten (replay), with the weight gradients accumulated.
    Returns the layer, the per-microbatch routing, Y, dX and d_topk_w."""
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
    return L, routing, ys, dxs, dtws


def test_stream_full_size_ring_walk():
    """8 microbatches of 2368 tokens through a 512 MiB ring (2 slots), backward in reverse with
    replay and accumulated weight gradients, against the oracle on sampled tokens and experts."""
    _announce("[full] stream 8 x T=2368 d=4096 E=512 k=10 I=1024, 512 MiB ring, seed 0")
    inp = workload.make_inputs("stream", seed=0, device=DEV)
    cfg = inp["cfg"]
    T, k, nmb = cfg["T"], cfg["k"], cfg["microbatches"]
    L, routing, ys, dxs, dtws = _stream_run(inp)
    Wr = _np(inp["Wr"])
    W1h, W2h = workload.HostExperts(inp["W1"]), workload.HostExperts(inp["W2"])
    experts = None
    dW1 = dW2 = dWr = None
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
        # dWr sums every microbatch's dlogits^T X: the oracle's dlogits need every row's dw, so
        # this uses the GPU's d_topk_w, which the sampled tokens above pin to the oracle's
        w = _np(routing[i][1]).astype(np.float64)
        dl = oracle.router_backward(w, _np(routing[i][0]), _np(dtws[i]).astype(np.float64),
                                    cfg["E"])
        dWr = dl.T @ X if dWr is None else dWr + dl.T @ X
        _announce(f"  microbatch {i} checked")
    for j, e in enumerate(experts):
        assert_grad(f"dW1[{e}] (sum of 8)", _np(L.dw1[e]), dW1[j])
        assert_grad(f"dW2[{e}] (sum of 8)", _np(L.dw2[e]), dW2[j])
    assert_grad("dWr (sum of 8)", _np(L.dwr), dWr)


def test_stream_two_macrobatch_runs_are_bitwise_identical():
    _announce("[full] stream determinism: the whole 8-microbatch ring walk twice")
    inp = workload.make_inputs("stream", seed=1, device=DEV)
    runs = []
    for _ in range(2):
        L, routing, ys, dxs, dtws = _stream_run(inp)
        flat = [t for r in routing for t in r] + ys + dxs + dtws
        flat += [L.dw1.clone(), L.dw2.clone(), L.dwr.clone()]
        runs.append(flat)
        del L
        torch.cuda.empty_cache()
    assert_bitwise_equal(runs[0], runs[1])
