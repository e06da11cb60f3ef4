"""Pins of the oracle's bf16 storage points, and of its one-expert-at-a-time layer driver.

The oracle in storage="bf16" mode rounds to bfloat16 exactly where the GPU path stores a
bf16 tensor: H = [g | u], A (rounded once from the unrounded g and u), O, Y, dH, dXp and dX;
every later step reads the stored value. The pin is an independent dense torch formulation
(float64 math, ``Tensor.to(torch.bfloat16)`` as the rounding, torch autograd for the softmax
backward) that casts at those points and nowhere else:
* every stored tensor must agree BIT FOR BIT with the oracle (the two sides differ only in the
  last float64 bit before a rounding, which moves a bf16 result only when a value sits within
  about 1e-16 of a rounding midpoint);
* the unrounded results (dw, the weight and router gradients) must agree to 1e-12 relative;
* each plausible misplacement of a rounding point (A taken from the rounded H, O left unrounded
  before the combine, the SwiGLU backward reading the unrounded g and u, dXp left unrounded
  before the token sum, dH not rounded) changes some stored value, so the bitwise comparison
  would catch it.
With dw_dtype="bf16" the weight gradients are stored as bf16 too: the formulation's dW1 and
dW2 cast once with torch's cast must equal the oracle's bit for bit, and leaving them unrounded
must not.
``oracle.layer`` (forward and backward one expert at a time) must equal ``oracle.forward``
followed by ``oracle.backward`` bit for bit: it is the same arithmetic in the same order.
"""
import numpy as np
import pytest
import torch

import oracle

F = torch.nn.functional


def _bf(t):
    return t.to(torch.bfloat16).to(torch.float64)


def _inputs(T, d, E, k, I, seed):
    rng = np.random.default_rng(seed)
    bf = oracle.bf16_round
    X = bf(rng.standard_normal((T, d)))
    Wr = bf(rng.standard_normal((E, d)) * 0.2)
    W1 = bf(rng.standard_normal((E, 2 * I, d)) * 0.2)
    W2 = bf(rng.standard_normal((E, d, I)) * 0.2)
    dY = bf(rng.standard_normal((T, d)))
    return X, Wr, W1, W2, dY


def _torch_layer(X, Wr, W1, W2, dY, L, k, mutant=None):
    """Dense per-row torch formulation with bf16 casts at the stated storage points.

    L: the fp32 router logits (their order is pinned by tests/test_oracle_router.py).
    ``mutant`` names one deliberate misplacement of a rounding point."""
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    X, Wr, W1, W2, dY = t(X), t(Wr), t(W1), t(W2), t(dY)
    T, d = X.shape
    E, twoI, _ = W1.shape
    I = twoI // 2
    logits = t(L).requires_grad_(True)
    sel = torch.topk(logits.detach(), k, dim=1).indices          # [T, k], descending
    wsel = torch.softmax(torch.gather(logits, 1, sel), dim=1)    # renormalised top-k softmax
    w = wsel.detach()
    W1g, W2g = W1[sel], W2[sel]                                  # [T, k, 2I, d], [T, k, d, I]
    gu = torch.einsum("tkod,td->tko", W1g, X)
    g, u = gu[..., :I], gu[..., I:]
    H = torch.cat([_bf(g), _bf(u)], dim=-1)
    if mutant == "A_from_rounded_H":
        A = _bf(F.silu(H[..., :I]) * H[..., I:])
    else:
        A = _bf(F.silu(g) * u)
    o_exact = torch.einsum("tkdi,tki->tkd", W2g, A)
    O = o_exact if mutant == "O_unrounded" else _bf(o_exact)
    Ysum = torch.zeros(T, d, dtype=torch.float64)
    for j in range(k):
        Ysum = Ysum + w[:, j:j + 1] * O[:, j]
    Y = _bf(Ysum)
    # backward
    dw = torch.einsum("td,tkd->tk", dY, O)
    dA = w[..., None] * torch.einsum("tkdi,td->tki", W2g, dY)
    if mutant == "swiglu_bwd_from_unrounded":
        gs, us = g, u
    else:
        gs, us = H[..., :I], H[..., I:]
    s = torch.sigmoid(gs)
    dgu = torch.cat([dA * us * s * (1 + gs * (1 - s)), dA * F.silu(gs)], dim=-1)
    dH = dgu if mutant == "dH_unrounded" else _bf(dgu)
    dxp_exact = torch.einsum("tko,tkod->tkd", dH, W1g)
    dXp = dxp_exact if mutant == "dXp_unrounded" else _bf(dxp_exact)
    (wsel * dw).sum().backward()                                 # dlogits by autograd
    dlogits = logits.grad
    dXsum = torch.zeros(T, d, dtype=torch.float64)
    for j in range(k):
        dXsum = dXsum + dXp[:, j]
    dX = _bf(dXsum + dlogits @ Wr)
    flat = sel.reshape(-1)
    dW1 = torch.zeros(E, twoI, d, dtype=torch.float64).index_add_(
        0, flat, torch.einsum("tko,td->tkod", dH, X).reshape(-1, twoI, d))
    dW2 = torch.zeros(E, d, I, dtype=torch.float64).index_add_(
        0, flat, torch.einsum("tkd,tki->tkdi", w[..., None] * dY[:, None, :], A).reshape(-1, d, I))
    dWr = dlogits.T @ X
    return dict(idx=sel.numpy(), H=H.numpy(), A=A.numpy(), O=O.numpy(), Y=Y.numpy(),
                dw=dw.numpy(), dH=dH.numpy(), dXp=dXp.numpy(), dX=dX.numpy(),
                dW1=dW1.numpy(), dW2=dW2.numpy(), dWr=dWr.numpy())


def _oracle_rows(f, b, T, k):
    """Oracle per-row tensors in (token, slot) order, to match the dense formulation."""
    pos = f["tk_row"].reshape(T, k)
    return {n: src[n][pos] for src, names in ((f, ("H", "A", "O")), (b, ("dH", "dXp")))
            for n in names}


SHAPES = [(40, 32, 6, 2, 16, 1), (24, 64, 5, 3, 8, 2), (16, 32, 4, 4, 16, 3)]


@pytest.mark.parametrize("T,d,E,k,I,seed", SHAPES)
def test_bf16_storage_points_match_an_independent_torch_formulation(T, d, E, k, I, seed):
    X, Wr, W1, W2, dY = _inputs(T, d, E, k, I, seed)
    f = oracle.forward(X, W1, W2, Wr=Wr, k=k)
    b = oracle.backward(f, X, W1, W2, dY, Wr=Wr)
    ref = _torch_layer(X, Wr, W1, W2, dY, f["logits"], k)
    np.testing.assert_array_equal(ref["idx"], f["idx"])
    rows = _oracle_rows(f, b, T, k)
    for n in ("H", "A", "O", "dH", "dXp"):
        np.testing.assert_array_equal(rows[n], ref[n], err_msg=n)
    np.testing.assert_array_equal(f["Y"], ref["Y"])
    np.testing.assert_array_equal(b["dX"], ref["dX"])
    for n in ("dw", "dW1", "dW2", "dWr"):
        np.testing.assert_allclose(b[n], ref[n], rtol=1e-12, atol=1e-12 * np.abs(ref[n]).max(),
                                   err_msg=n)
    b16 = oracle.backward(f, X, W1, W2, dY, Wr=Wr, dw_dtype="bf16")
    for n in ("dW1", "dW2"):
        want = _bf(torch.from_numpy(ref[n])).numpy()
        np.testing.assert_array_equal(b16[n], want, err_msg=n)
        assert not np.array_equal(b16[n], ref[n])  # the unrounded sums differ from the stored
    for n in ("dw", "dH", "dXp", "dX", "dWr"):
        np.testing.assert_array_equal(b16[n], b[n], err_msg=n)  # nothing else changes


@pytest.mark.parametrize("mutant,affected", [
    ("A_from_rounded_H", ("A", "O", "Y")),
    ("O_unrounded", ("O", "Y")),
    ("swiglu_bwd_from_unrounded", ("dH", "dXp", "dX")),
    ("dH_unrounded", ("dH", "dXp", "dX")),
    ("dXp_unrounded", ("dXp", "dX")),
])
def test_each_misplaced_rounding_point_changes_a_stored_value(mutant, affected):
    T, d, E, k, I, seed = SHAPES[0]
    X, Wr, W1, W2, dY = _inputs(T, d, E, k, I, seed)
    f = oracle.forward(X, W1, W2, Wr=Wr, k=k)
    b = oracle.backward(f, X, W1, W2, dY, Wr=Wr)
    got = _torch_layer(X, Wr, W1, W2, dY, f["logits"], k, mutant=mutant)
    have = dict(_oracle_rows(f, b, T, k), Y=f["Y"], dX=b["dX"])
    for n in affected:
        assert not np.array_equal(have[n], got[n]), (mutant, n)


def _layer_cases():
    rng = np.random.default_rng(5)
    T, d, E, I = 48, 64, 6, 32
    idx = rng.integers(0, E, size=(T, 1)).astype(np.int32)
    idx[idx == 3] = 4                                        # expert 3 left empty
    return [("routed", dict(k=2), "bf16"), ("routed", dict(k=3), "mxfp8"),
            ("given", dict(topk_idx=idx, topk_w=rng.random((T, 1))), "bf16")], (T, d, E, I)


@pytest.mark.parametrize("case", range(3))
@pytest.mark.parametrize("dw_dtype", ["fp32", "bf16"])
def test_layer_driver_equals_forward_then_backward_bitwise(case, dw_dtype):
    cases, (T, d, E, I) = _layer_cases()
    mode, kw, prec = cases[case]
    X, Wr, W1, W2, dY = _inputs(T, d, E, kw.get("k", 1), I, 40 + case)
    if mode == "routed":
        kw = dict(kw, Wr=Wr)
    f = oracle.forward(X, W1, W2, precision=prec, **kw)
    b = oracle.backward(f, X, W1, W2, dY, Wr=kw.get("Wr"), dw_dtype=dw_dtype)
    seen = {}
    lay = oracle.layer(X, W1, W2, dY, precision=prec, dw_dtype=dw_dtype,
                       on_expert=lambda e, a, c: seen.__setitem__(e, (a, c)), **kw)
    assert sorted(seen) == list(range(E))
    for n in ("idx", "w", "counts", "offsets", "row_src", "tk_row", "H", "A", "O", "Y"):
        np.testing.assert_array_equal(lay[n], f[n], err_msg=n)
    for n in ("dw", "dH", "dXp", "dX") + (("dlogits", "dWr") if mode == "routed" else ()):
        np.testing.assert_array_equal(lay[n], b[n], err_msg=n)
    for e in range(E):
        np.testing.assert_array_equal(seen[e][0], b["dW1"][e])
        np.testing.assert_array_equal(seen[e][1], b["dW2"][e])
    if mode == "given":
        assert not np.any(seen[3][0]) and not np.any(seen[3][1])
