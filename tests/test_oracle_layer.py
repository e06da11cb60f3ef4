"""Pins of the oracle's forward and backward against independent computations.

* Forward: a dense evaluation of every token through every expert, masked. It equals the
  sparse permute/gather path (no row lost or mixed up). Two special cases reduce to a plain
  SwiGLU MLP built from torch's functional ops: E=1 with k=1, and all experts identical.
* Backward: central finite differences in float64, and torch autograd on an independent dense
  torch formulation. Invariants: the router-weight-gradient identity
  <dY, o> = <dY W2, a> (the SonicMoE-style fused form), and every dlogits row summing to 0.
"""
import numpy as np
import pytest
import torch

import oracle

torch.set_default_dtype(torch.float64)


def _rand_layer(T, d, E, k, I, seed, scale_w=0.3):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, d))
    Wr = rng.standard_normal((E, d)) * scale_w
    W1 = rng.standard_normal((E, 2 * I, d)) * scale_w
    W2 = rng.standard_normal((E, d, I)) * scale_w
    dY = rng.standard_normal((T, d))
    return X, Wr, W1, W2, dY


def _ffn_torch(x, w1, w2):
    I = w1.shape[0] // 2
    g = torch.nn.functional.linear(x, w1[:I])
    u = torch.nn.functional.linear(x, w1[I:])
    return torch.nn.functional.linear(torch.nn.functional.silu(g) * u, w2)


def _fwd_exact(X, Wr, W1, W2, k):
    return oracle.forward(X, W1, W2, Wr=Wr, k=k, storage="exact", logits="fp64")


# --- forward --------------------------------------------------------------------------------

@pytest.mark.parametrize("T,d,E,k,I", [(40, 16, 6, 2, 8), (33, 32, 8, 3, 16), (20, 8, 4, 4, 4)])
def test_forward_equals_dense_masked_evaluation(T, d, E, k, I):
    X, Wr, W1, W2, _ = _rand_layer(T, d, E, k, I, seed=T * d)
    f = _fwd_exact(X, Wr, W1, W2, k)
    Wd = np.zeros((T, E))
    np.put_along_axis(Wd, f["idx"], f["w"], axis=1)
    Xt = torch.from_numpy(X)
    Y = torch.zeros(T, d)
    for e in range(E):
        Y += torch.from_numpy(Wd[:, e:e + 1]) * _ffn_torch(Xt, torch.from_numpy(W1[e]),
                                                         torch.from_numpy(W2[e]))
    np.testing.assert_allclose(f["Y"], Y.numpy(), rtol=1e-12, atol=1e-12)


def test_single_expert_top1_is_textbook_swiglu():
    X, Wr, W1, W2, _ = _rand_layer(25, 16, 1, 1, 8, seed=11)
    f = _fwd_exact(X, Wr, W1, W2, 1)
    np.testing.assert_array_equal(f["w"], np.ones((25, 1)))
    want = _ffn_torch(torch.from_numpy(X), torch.from_numpy(W1[0]), torch.from_numpy(W2[0]))
    np.testing.assert_allclose(f["Y"], want.numpy(), rtol=1e-13, atol=1e-13)


def test_identical_experts_give_the_plain_ffn():
    X, Wr, W1, W2, _ = _rand_layer(30, 16, 5, 3, 8, seed=12)
    W1[:] = W1[0]
    W2[:] = W2[0]
    f = _fwd_exact(X, Wr, W1, W2, 3)
    want = _ffn_torch(torch.from_numpy(X), torch.from_numpy(W1[0]), torch.from_numpy(W2[0]))
    np.testing.assert_allclose(f["Y"], want.numpy(), rtol=1e-12, atol=1e-12)


def test_bf16_storage_rounds_where_stated_and_stays_close():
    rng = np.random.default_rng(13)
    bf = lambda a: oracle.bf16_round(a)
    T, d, E, k, I = 64, 64, 8, 2, 32
    X = bf(rng.standard_normal((T, d)))
    Wr = bf(rng.standard_normal((E, d)) * 0.02)
    W1 = bf(rng.standard_normal((E, 2 * I, d)) * 0.1)
    W2 = bf(rng.standard_normal((E, d, I)) * 0.1)
    dY = bf(rng.standard_normal((T, d)))
    fb = oracle.forward(X, W1, W2, Wr=Wr, k=k)
    fe = oracle.forward(X, W1, W2, Wr=Wr, k=k, storage="exact")
    np.testing.assert_array_equal(fb["idx"], fe["idx"])
    for key in ("H", "A", "O", "Y"):
        np.testing.assert_array_equal(bf(fb[key]), fb[key])
        rel = np.sqrt(np.mean((fb[key] - fe[key]) ** 2) / np.mean(fe[key] ** 2))
        assert 0 < rel < 1e-2, (key, rel)
    bb = oracle.backward(fb, X, W1, W2, dY, Wr=Wr)
    for key in ("dH", "dXp", "dX"):
        np.testing.assert_array_equal(bf(bb[key]), bb[key])


# --- backward -------------------------------------------------------------------------------

def _loss(X, Wr, W1, W2, dY, k, idx_ref):
    f = _fwd_exact(X, Wr, W1, W2, k)
    assert np.array_equal(f["idx"], idx_ref), "routing changed under the perturbation"
    return float(np.sum(f["Y"] * dY))


def _fd_grad(param, fn, h=1e-6):
    g = np.zeros_like(param)
    it = np.nditer(param, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = param[i]
        param[i] = old + h
        fp = fn()
        param[i] = old - h
        fm = fn()
        param[i] = old
        g[i] = (fp - fm) / (2 * h)
    return g


def test_backward_matches_central_finite_differences():
    T, d, E, k, I = 6, 16, 4, 2, 8
    X, Wr, W1, W2, dY = _rand_layer(T, d, E, k, I, seed=21)
    f = _fwd_exact(X, Wr, W1, W2, k)
    b = oracle.backward(f, X, W1, W2, dY, Wr=Wr)
    fn = lambda: _loss(X, Wr, W1, W2, dY, k, f["idx"])
    for name, param, got in (("X", X, b["dX"]), ("Wr", Wr, b["dWr"]),
                             ("W1", W1, b["dW1"]), ("W2", W2, b["dW2"])):
        want = _fd_grad(param, fn)
        scale = np.max(np.abs(want))
        assert scale > 0
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-6 * scale, err_msg=name)


def test_given_routing_weight_gradient_matches_finite_differences():
    T, d, E, I = 10, 16, 4, 8
    X, _, W1, W2, dY = _rand_layer(T, d, E, 1, I, seed=22)
    rng = np.random.default_rng(23)
    idx = rng.integers(0, E, size=(T, 1)).astype(np.int32)
    idx[:, 0] = np.where(idx[:, 0] == 2, 3, idx[:, 0])        # expert 2 left empty
    w = rng.random((T, 1))
    fwd = lambda: oracle.forward(X, W1, W2, topk_idx=idx, topk_w=w, storage="exact")
    f = fwd()
    b = oracle.backward(f, X, W1, W2, dY)
    assert "dWr" not in b
    np.testing.assert_array_equal(b["dW1"][2], 0)
    np.testing.assert_array_equal(b["dW2"][2], 0)
    want = _fd_grad(w, lambda: float(np.sum(fwd()["Y"] * dY)))
    np.testing.assert_allclose(b["dw"], want, rtol=0, atol=1e-7 * np.max(np.abs(want)))
    wantX = _fd_grad(X, lambda: float(np.sum(fwd()["Y"] * dY)))
    np.testing.assert_allclose(b["dX"], wantX, rtol=0, atol=1e-6 * np.max(np.abs(wantX)))


@pytest.mark.parametrize("T,d,E,k,I", [(24, 16, 6, 2, 8), (16, 32, 8, 4, 16)])
def test_backward_matches_torch_autograd_dense(T, d, E, k, I):
    X, Wr, W1, W2, dY = _rand_layer(T, d, E, k, I, seed=31 + k)
    f = _fwd_exact(X, Wr, W1, W2, k)
    b = oracle.backward(f, X, W1, W2, dY, Wr=Wr)
    tX, tWr, tW1, tW2 = (torch.tensor(a, requires_grad=True) for a in (X, Wr, W1, W2))
    L = tX @ tWr.T
    sel = torch.topk(L.detach(), k, dim=1).indices
    assert np.array_equal(np.sort(sel.numpy(), 1), np.sort(f["idx"], 1))
    mask = torch.zeros(T, E, dtype=torch.bool).scatter_(1, sel, True)
    wfull = torch.softmax(L.masked_fill(~mask, float("-inf")), dim=1)
    wfull.retain_grad()
    Y = torch.zeros(T, d)
    for e in range(E):
        Y = Y + wfull[:, e:e + 1] * _ffn_torch(tX, tW1[e], tW2[e])
    (Y * torch.from_numpy(dY)).sum().backward()
    np.testing.assert_allclose(b["dX"], tX.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(b["dWr"], tWr.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(b["dW1"], tW1.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(b["dW2"], tW2.grad.numpy(), rtol=1e-10, atol=1e-12)
    # The gradient reaching each selected weight: dL/dw_tj = <dY_t, o_tj>.
    dwfull = wfull.grad.numpy()
    np.testing.assert_allclose(b["dw"], np.take_along_axis(dwfull, f["idx"], 1),
                               rtol=1e-10, atol=1e-12)


def test_router_weight_gradient_identity_and_dlogit_rows_sum_to_zero():
    T, d, E, k, I = 30, 24, 6, 3, 12
    X, Wr, W1, W2, dY = _rand_layer(T, d, E, k, I, seed=41)
    f = _fwd_exact(X, Wr, W1, W2, k)
    b = oracle.backward(f, X, W1, W2, dY, Wr=Wr)
    # <dY_t, o_tj> == <dY_t W2_e, a_tj>: the fused (SonicMoE-style) form used by the GPU path.
    for t in range(T):
        for j in range(k):
            e = f["idx"][t, j]
            pos = f["tk_row"][t * k + j]
            fused = np.dot(dY[t] @ W2[e], f["A"][pos])
            assert abs(fused - b["dw"][t, j]) <= 1e-12 * max(1.0, abs(fused))
    np.testing.assert_allclose(b["dlogits"].sum(1), 0, atol=1e-13)
    off = np.ones((T, E), bool)
    np.put_along_axis(off, f["idx"], False, axis=1)
    assert np.all(b["dlogits"][off] == 0)
