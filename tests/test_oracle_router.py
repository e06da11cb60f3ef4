"""Pins of the oracle's routing steps against things other than the oracle itself.

The pins are:
* a hand-worked fp32 summation example (golden file);
* the floating-point error bound of recursive summation;
* exact integer arithmetic;
* brute force over all k-subsets;
* the closed forms Wr = 0 and k = E;
* a tie between duplicate router rows;
* a brute-force counting sort.
"""
import itertools
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle.moe import router_logits_fp64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()


# --- bf16 rounding -----------------------------------------------------------------------------

def test_bf16_round_matches_torch_cast_on_float32_values():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(100000).astype(np.float32) * s
                        for s in (1e-3, 1.0, 37.0, 1e4)])
    ours = oracle.bf16_round(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(ours, ref)


def test_bf16_round_ties_to_even_by_hand():
    # Near 1 the bf16 spacing is 2^-7. 1 + 2^-8 is a tie between 1 (even) and 1 + 2^-7 (odd).
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 (odd) and 1 + 2^-6 (even).
    x = np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 1 + 2**-8 + 2**-30, 255.5])
    want = np.array([1.0, 1 + 2**-6, -1.0, 1 + 2**-7, 256.0])
    np.testing.assert_array_equal(oracle.bf16_round(x), want)


# --- router logits ------------------------------------------------------------------------------

def _golden_logit_cases():
    cases = []
    with open(os.path.join(GOLDEN, "logit_order.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            name, xs, ws, exp = [s.strip() for s in line.split("|")]
            x = np.array([float.fromhex(t) for t in xs.split()], np.float32)
            w = np.array([float.fromhex(t) for t in ws.split()], np.float32)
            cases.append((name, x, w, np.float32(float.fromhex(exp))))
    return cases


@pytest.mark.parametrize("case", _golden_logit_cases(), ids=lambda c: c[0])
def test_logits_hand_worked_summation_order(case):
    name, x, w, expected = case
    L = oracle.router_logits_fp32(x[None, :], w[None, :])
    assert L.dtype == np.float32
    assert L[0, 0] == expected, (name, L[0, 0].hex() if hasattr(L[0, 0], "hex") else L[0, 0])


@pytest.mark.parametrize("T,d,E", [(64, 256, 8), (16, 7168, 32)])
def test_logits_within_recursive_summation_bound(T, d, E):
    # Recursive summation of d exact products: |fl(sum) - sum| <= gamma_{d-1} * sum |p_i|,
    # gamma_n = n u / (1 - n u), u = 2^-24 (Higham, Accuracy and Stability, eq. 4.4).
    rng = np.random.default_rng(1)
    X = _bf16(rng.standard_normal((T, d)))
    Wr = _bf16(rng.standard_normal((E, d)) * 0.02)
    L32 = oracle.router_logits_fp32(X, Wr).astype(np.float64)
    L64 = router_logits_fp64(X, Wr)
    absdot = np.abs(X.astype(np.float64)) @ np.abs(Wr.astype(np.float64)).T
    u = 2.0 ** -24
    gamma = (d - 1) * u / (1 - (d - 1) * u)
    assert np.all(np.abs(L32 - L64) <= gamma * absdot)
    # A transposed or shifted operand would break agreement far beyond the bound.
    assert np.max(np.abs(L32 - L64)) < 1e-3 * np.max(np.abs(L64))


def test_logits_exact_for_small_integers():
    # Small integers keep every partial sum exact in fp32, so the result is the integer dot.
    rng = np.random.default_rng(2)
    X = rng.integers(-8, 9, size=(12, 64)).astype(np.float32)
    Wr = rng.integers(-8, 9, size=(5, 64)).astype(np.float32)
    L = oracle.router_logits_fp32(X, Wr)
    want = X.astype(np.int64) @ Wr.astype(np.int64).T
    np.testing.assert_array_equal(L, want.astype(np.float32))


def test_logits_equivariant_and_duplicate_rows_tie_bitwise():
    rng = np.random.default_rng(3)
    X = _bf16(rng.standard_normal((20, 128)))
    Wr = _bf16(rng.standard_normal((6, 128)) * 0.02)
    Wr[4] = Wr[1]
    L = oracle.router_logits_fp32(X, Wr)
    np.testing.assert_array_equal(L[:, 4], L[:, 1])
    perm = rng.permutation(6)
    np.testing.assert_array_equal(oracle.router_logits_fp32(X, Wr[perm]), L[:, perm])
    tperm = rng.permutation(20)
    np.testing.assert_array_equal(oracle.router_logits_fp32(X[tperm], Wr), L[tperm])


# --- top-k ----------------------------------------------------------------------------------

def _brute_topk(row, k):
    """The unique k-subset whose every member beats every non-member under (value desc, index
    asc), listed in that order."""
    E = len(row)
    beats = lambda a, b: row[a] > row[b] or (row[a] == row[b] and a < b)
    winners = []
    for S in itertools.combinations(range(E), k):
        rest = [e for e in range(E) if e not in S]
        if all(beats(a, b) for a in S for b in rest):
            winners.append(S)
    assert len(winners) == 1
    S = list(winners[0])
    S.sort(key=lambda e: (-row[e], e))
    return S


@pytest.mark.parametrize("E,k", [(6, 1), (6, 3), (7, 4), (5, 5)])
def test_topk_brute_force_with_many_ties(E, k):
    rng = np.random.default_rng(E * 10 + k)
    L = rng.integers(-2, 3, size=(200, E)).astype(np.float32)   # heavy ties
    idx, w = oracle.route_topk(L, k)
    for t in range(L.shape[0]):
        assert list(idx[t]) == _brute_topk(list(L[t]), k)


def test_topk_zero_router_gives_first_k_experts_uniform():
    X = _bf16(np.random.default_rng(4).standard_normal((9, 64)))
    L = oracle.router_logits_fp32(X, np.zeros((8, 64), np.float32))
    idx, w = oracle.route_topk(L, 3)
    np.testing.assert_array_equal(idx, np.tile(np.arange(3, dtype=np.int32), (9, 1)))
    np.testing.assert_array_equal(w, np.full((9, 3), 1.0 / 3.0))


def test_topk_with_k_equal_E_is_full_softmax():
    rng = np.random.default_rng(5)
    L = rng.standard_normal((50, 8)).astype(np.float32) * 3
    idx, w = oracle.route_topk(L, 8)
    full = scipy.special.softmax(L.astype(np.float64), axis=1)
    got = np.zeros_like(full)
    np.put_along_axis(got, idx, w, axis=1)
    np.testing.assert_allclose(got, full, rtol=1e-13, atol=1e-16)


def test_topk_weights_equal_softmax_then_renormalise():
    rng = np.random.default_rng(6)
    L = rng.standard_normal((40, 16)).astype(np.float32)
    idx, w = oracle.route_topk(L, 4)
    p = scipy.special.softmax(L.astype(np.float64), axis=1)
    sel = np.take_along_axis(p, idx, axis=1)
    np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-13)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-15)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_duplicate_router_rows_tie_goes_to_lower_expert():
    rng = np.random.default_rng(7)
    X = _bf16(rng.standard_normal((300, 64)))
    Wr = _bf16(rng.standard_normal((8, 64)) * 0.02)
    Wr[6] = Wr[2]
    L = oracle.router_logits_fp32(X, Wr)
    idx, _ = oracle.route_topk(L, 3)
    seen_boundary = 0
    for t in range(300):
        row = list(idx[t])
        if 6 in row:
            assert 2 in row and row.index(2) < row.index(6)
        if 2 in row and 6 not in row:
            seen_boundary += 1   # the tie sat on the selection boundary; the lower id won
    assert seen_boundary > 0


# --- permutation ----------------------------------------------------------------------------

def _brute_counting_sort(flat, E):
    buckets = [[] for _ in range(E)]
    for r, e in enumerate(flat):
        buckets[e].append(r)
    return [r for b in buckets for r in b], [len(b) for b in buckets]


@pytest.mark.parametrize("T,E,k", [(50, 8, 2), (37, 16, 4), (64, 4, 1)])
def test_permutation_invariants_and_brute_force(T, E, k):
    rng = np.random.default_rng(T + E + k)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, row_src, tk_row = oracle.permute(idx, E)
    assert counts.sum() == T * k
    assert offsets[0] == 0 and offsets[-1] == T * k
    np.testing.assert_array_equal(np.sort(row_src), np.arange(T * k))
    np.testing.assert_array_equal(tk_row[row_src], np.arange(T * k))
    np.testing.assert_array_equal(row_src[tk_row], np.arange(T * k))
    flat = idx.reshape(-1)
    for e in range(E):
        seg = row_src[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)
    want_src, want_counts = _brute_counting_sort(list(flat), E)
    np.testing.assert_array_equal(row_src, want_src)
    np.testing.assert_array_equal(counts, want_counts)


def test_permutation_with_empty_experts():
    idx = np.array([[3], [3], [1], [3]], np.int32)
    counts, offsets, row_src, tk_row = oracle.permute(idx, 5)
    np.testing.assert_array_equal(counts, [0, 1, 0, 3, 0])
    np.testing.assert_array_equal(offsets, [0, 0, 1, 1, 4, 4])
    np.testing.assert_array_equal(row_src, [2, 0, 1, 3])
    np.testing.assert_array_equal(tk_row, [1, 2, 0, 3])
