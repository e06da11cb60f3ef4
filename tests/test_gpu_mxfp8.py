"""GPU parity of the MXFP8 mode against the oracle that emulates the same quantisation.

* The quantised weights and the permuted tokens are integer codes: they must equal the oracle's
  quantiser bit for bit.
* Routing and the permutation maps are bit-exact, as in BF16 mode.
* Floating outputs and gradients must be within 6e-2 of the MXFP8-emulating oracle. Y and dX
  are checked as max-abs and RMS relative error; the weight, router and routing-weight
  gradients as relative Frobenius error.
* Two runs are bitwise identical, at a small shape and at the DeepSeek-V3 shape (sampled
  checks there, as in tests/test_gpu_sizes_full.py).
"""
import numpy as np
import pytest
import torch

import oracle
import workload
from tests._gpu import (DEV, MoeLayer, _announce, _np, assert_bitwise_equal, check_parity, m,
                        outputs, run_gpu, run_oracle)
from tests._util import assert_act, assert_grad

pytestmark = pytest.mark.gpu

TOL_MX = 6e-2


def _up(v):
    return (v + 255) // 256 * 256


def _wq_parts(L):
    """The four MXFP8 weight tensors and their scales inside L.wq, in the order the header
    lists them: W1 along d, W2 along I, W2 transposed along d, W1 transposed along 2I."""
    E, d, I = L.E, L.d, L.I
    shapes = [(E, 2 * I, d), (E, d, I), (E, I, d), (E, d, 2 * I)]
    out, o = [], 0
    for sh in shapes:
        n = sh[0] * sh[1] * sh[2]
        codes = L.wq[o:o + n].view(*sh)
        o += _up(n)
        sc = L.wq[o:o + n // 32].view(sh[0], sh[1], sh[2] // 32)
        o += _up(n // 32)
        out.append((codes, sc))
    return out


def _mx_inputs(name="tiny", seed=0, **over):
    return workload.make_inputs(name, seed=seed, device=DEV, precision="mxfp8", **over)


def test_weight_quantisation_is_bit_exact():
    _announce("[mxfp8] quantised weights, tiny shape")
    inp = _mx_inputs(seed=0, E=4)
    L = run_gpu(inp)
    W1, W2 = _np(inp["W1"]), _np(inp["W2"])
    refs = [oracle.mx.quantize(W1), oracle.mx.quantize(W2),
            oracle.mx.quantize(np.swapaxes(W2, 1, 2)), oracle.mx.quantize(np.swapaxes(W1, 1, 2))]
    for i, ((codes, sc), (q, s)) in enumerate(zip(_wq_parts(L), refs)):
        np.testing.assert_array_equal(_np(sc), s, err_msg=f"scales of part {i}")
        np.testing.assert_array_equal(_np(codes), q, err_msg=f"codes of part {i}")


MX_CASES = {
    "tiny": dict(name="tiny"),
    "ragged": dict(name="tiny", T=300, E=16, k=3, d=512, I=256),
    "multi_mtile": dict(name="tiny", T=1024, E=4, k=2, d=512, I=256),
    "zipf_local": dict(name="local_zipf", T=2048, d=256, I=256),
}


@pytest.mark.parametrize("case", list(MX_CASES))
def test_mxfp8_layer_parity(case):
    spec = dict(MX_CASES[case])
    name = spec.pop("name")
    _announce(f"[mxfp8] case={case} shape={spec} seed=0")
    inp = _mx_inputs(name, seed=0, **spec)
    L = run_gpu(inp)
    f, b = run_oracle(inp)
    check_parity(L, inp, f, b, tol_act=TOL_MX, tol_grad=TOL_MX)


def test_mxfp8_two_runs_are_bitwise_identical():
    _announce("[mxfp8] determinism, multi-m-tile shape")
    inp = _mx_inputs("tiny", seed=2, T=1024, E=8, k=2, d=512, I=256)
    a = outputs(run_gpu(inp), True)
    b = outputs(run_gpu(inp, persistent=True), True)
    assert_bitwise_equal(a, b)


def test_mxfp8_full_size_sampled_parity_and_determinism():
    """At the DeepSeek-V3 shape the oracle's quantiser costs seconds per expert, so this checks
    one sampled token (its 8 experts) and the heaviest expert's weights and weight gradients."""
    _announce("[mxfp8] dsv3_mxfp8 T=2048 d=7168 E=256 k=8 I=2048 seed 0")
    inp = workload.make_inputs("dsv3_mxfp8", seed=0, device=DEV)
    L = run_gpu(inp)
    X, dY, Wr = _np(inp["X"]), _np(inp["dY"]), _np(inp["Wr"])
    k = inp["cfg"]["k"]
    logits = oracle.router_logits_fp32(X, Wr)
    np.testing.assert_array_equal(_np(L.logits), logits)
    idx, _ = oracle.route_topk(logits, k)
    np.testing.assert_array_equal(_np(L.topk_idx), idx)
    counts, offsets, row_src, tk_row = oracle.permute(idx, inp["cfg"]["E"])
    np.testing.assert_array_equal(_np(L.row_src), row_src)
    _announce("  routing and permutation bit-exact")
    pos = np.unique(np.concatenate([[0, len(row_src) - 1],
                                    np.random.default_rng(5).choice(len(row_src), 64)]))
    codes, scales = L.xp()
    q, sc = oracle.mx.quantize(X[row_src[pos] // k])
    p_dev = torch.from_numpy(pos).to(DEV)
    np.testing.assert_array_equal(_np(codes[p_dev]), q)
    np.testing.assert_array_equal(_np(scales[p_dev]), sc)
    _announce("  ring codes and scales bit-exact on sampled positions")
    heavy = int(np.argmax(counts))
    W1e, W2e = _np(inp["W1"][heavy]), _np(inp["W2"][heavy])
    refs = [oracle.mx.quantize(W1e), oracle.mx.quantize(W2e),
            oracle.mx.quantize(W2e.T), oracle.mx.quantize(W1e.T)]
    for i, ((cq, cs), (rq, rs)) in enumerate(zip(_wq_parts(L), refs)):
        np.testing.assert_array_equal(_np(cs[heavy]), rs, err_msg=f"scales of part {i}")
        np.testing.assert_array_equal(_np(cq[heavy]), rq, err_msg=f"codes of part {i}")
    _announce(f"  quantised weights of expert {heavy} bit-exact")
    W1h, W2h = workload.HostExperts(inp["W1"]), workload.HostExperts(inp["W2"])
    tok = np.array([int(np.random.default_rng(6).integers(X.shape[0]))])
    f = oracle.forward(X[tok], W1h, W2h, Wr=Wr, k=k, precision="mxfp8")
    _announce("  oracle forward of the sampled token done")
    bk = oracle.backward(f, X[tok], W1h, W2h, dY[tok], Wr=Wr)
    t_dev = torch.from_numpy(tok).to(DEV)
    assert_act("Y[token]", _np(L.y[t_dev]), f["Y"], TOL_MX)
    assert_act("dX[token]", _np(L.dx[t_dev]), bk["dX"], TOL_MX)
    assert_grad("d_topk_w[token]", _np(L.d_topk_w[t_dev]), bk["dw"], TOL_MX)
    fe = oracle.forward(X, W1h, W2h, Wr=Wr, k=k, experts=[heavy], precision="mxfp8")
    _announce("  oracle forward of the heavy expert done")
    be = oracle.backward(fe, X, W1h, W2h, dY, Wr=Wr, experts=[heavy])
    assert_grad(f"dW1[{heavy}]", _np(L.dw1[heavy]), be["dW1"][0], TOL_MX)
    assert_grad(f"dW2[{heavy}]", _np(L.dw2[heavy]), be["dW2"][0], TOL_MX)
    ref = outputs(L, True)
    del L
    torch.cuda.empty_cache()
    assert_bitwise_equal(ref, outputs(run_gpu(inp), True, clone=False))
    _announce("  two full-size runs bitwise identical")


def _special_blocks(rows, cols, seed):
    """bf16 values [rows, cols] whose 32-blocks along the row exercise the edges of the MXFP8
    quantiser: all +0 and all -0 blocks, blocks of bf16 subnormals, blocks at the top of the
    bf16 range, exact powers of two, E4M3 rounding ties at unit scale, values in (448, 512)
    after scaling (saturation), one large value over tiny ones (underflow to zero), and plain
    normal values."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    nb = cols // 32
    for r in range(rows):
        for b in range(nb):
            kind = (r * nb + b) % 10
            blk = x[r, 32 * b:32 * b + 32]
            if kind == 0:
                blk[:] = 0.0
            elif kind == 1:
                blk[:] = -0.0
            elif kind == 2:  # bf16 subnormals, mixed signs
                blk[:] = rng.choice([-1, 1], 32) * rng.integers(1, 128, 32) * 2.0 ** -133
            elif kind == 3:  # near the top of the bf16 range
                blk[:] = rng.choice([-1, 1], 32) * rng.uniform(1.0, 1.99, 32) * 2.0 ** 127
            elif kind == 4:  # exact powers of two
                blk[:] = rng.choice([-1, 1], 32) * 2.0 ** rng.integers(-20, 20, 32)
            elif kind == 5:  # amax 256 -> scale 1; ties between E4M3 neighbours
                blk[:] = [256.0] + [1.0625, 1.1875, 3.25, 9.5, 0.015625 * 1.5, 2.0 ** -9 * 1.5,
                                    -1.0625, -3.75, 17.0, 232.0, 240.0, 248.0] + [0.5] * 19
            elif kind == 6:  # block max in (448, 512) after scaling: saturates
                blk[:] = rng.uniform(-1, 1, 32) * 256.0
                blk[0] = 480.0
                blk[1] = -500.0
            elif kind == 7:  # one large value over tiny ones
                blk[:] = rng.standard_normal(32) * 1e-6
                blk[5] = 3.0e4
    return torch.from_numpy(x).to(torch.bfloat16)


def test_mxfp8_quantiser_edge_values_are_bit_exact():
    """Weights and tokens built from the quantiser's edge cases: the GPU codes and scales of
    W1, W2 (both axes) and of the permuted tokens equal the oracle's quantiser bit for bit."""
    _announce("[mxfp8] quantiser edge values, E=4 d=256 I=128 T=64 k=2")
    T, d, E, k, I = 64, 256, 4, 2, 128
    W1 = _special_blocks(E * 2 * I, d, 1).reshape(E, 2 * I, d).to(DEV)
    W2 = _special_blocks(E * d, I, 2).reshape(E, d, I).to(DEV)
    X = _special_blocks(T, d, 3).to(DEV)
    L = MoeLayer(T, d, E, k, I, device=DEV, precision=m.MOE_PREC_MXFP8)
    L.quantize_weights(W1, W2)
    idx = torch.tensor([[t % E, (t + 1) % E] for t in range(T)], dtype=torch.int32)
    L.set_routing(idx.to(DEV), torch.full((T, k), 0.5, dtype=torch.float32, device=DEV))
    L.permute(X)
    torch.cuda.synchronize()
    W1n, W2n, Xn = _np(W1), _np(W2), _np(X)
    refs = [oracle.mx.quantize(W1n), oracle.mx.quantize(W2n),
            oracle.mx.quantize(np.swapaxes(W2n, 1, 2)), oracle.mx.quantize(np.swapaxes(W1n, 1, 2))]
    for i, ((codes, sc), (q, s)) in enumerate(zip(_wq_parts(L), refs)):
        np.testing.assert_array_equal(_np(sc), s, err_msg=f"scales of part {i}")
        np.testing.assert_array_equal(_np(codes), q, err_msg=f"codes of part {i}")
    row_src = _np(L.row_src)
    codes, scales = L.xp()
    q, sc = oracle.mx.quantize(Xn[row_src // k])
    np.testing.assert_array_equal(_np(scales), sc)
    np.testing.assert_array_equal(_np(codes), q)


def test_mxfp8_big_expert_wgrad_with_accumulation():
    """One expert of 700 rows (the gate wgrad's big-expert kernel, fed the exact bf16 image of
    the ring's fp8 rows through the dXp buffer), beside small and empty experts, in MXFP8 mode:
    parity with the MXFP8 oracle, then a second backward with accumulate=1 must double every
    weight gradient exactly."""
    counts = [700, 300, 0, 24]
    _announce(f"[mxfp8] big expert {counts}, d=512 I=256 k=1, accumulate")
    E, d, I = len(counts), 512, 256
    T = sum(counts)
    inp = workload.make_inputs("local_zipf", seed=13, device=DEV, T=T, d=d, E=E, I=I,
                               precision="mxfp8")
    idx = np.repeat(np.arange(E, dtype=np.int32), counts)
    np.random.default_rng(13).shuffle(idx)
    inp["topk_idx"] = torch.from_numpy(idx.reshape(T, 1)).to(DEV)
    L = run_gpu(inp)
    f, b = run_oracle(inp)
    assert list(f["counts"]) == counts
    check_parity(L, inp, f, b, tol_act=TOL_MX, tol_grad=TOL_MX)
    first = [g.clone() for g in (L.dw1, L.dw2)]
    L.backward(None, inp["W1"], inp["W2"], inp["dY"], accumulate=True)
    torch.cuda.synchronize()
    for g0, g in zip(first, (L.dw1, L.dw2)):
        assert torch.equal(g, 2 * g0)


def test_mxfp8_expert_sizes_at_the_256_row_block_boundaries():
    """Experts of 0, 1, 128, 255, 256, 257, 384, 511, 512 and 513 rows in MXFP8 mode: each of the
    four MXFP8 GEMMs splits an expert into full 256-row blocks (the direct-to-LDS 256 x 256
    kernels) and 128-row remainder tiles. Parity against the MXFP8 oracle, with d = 512 (four K
    steps of the gate/up GEMM, two column tiles of the down GEMM and the gate dgrad) and
    I = 512 (two column tiles of the down dgrad); persistent grids bitwise equal to one-shot
    grids."""
    counts = [255, 256, 257, 0, 511, 512, 513, 1, 128, 384]
    _announce(f"[mxfp8] expert sizes {counts}, d=512 I=512 k=1")
    E, d, I = len(counts), 512, 512
    T = sum(counts)
    inp = workload.make_inputs("local_zipf", seed=9, device=DEV, T=T, d=d, E=E, I=I,
                               precision="mxfp8")
    idx = np.repeat(np.arange(E, dtype=np.int32), counts)
    np.random.default_rng(9).shuffle(idx)
    inp["topk_idx"] = torch.from_numpy(idx.reshape(T, 1)).to(DEV)
    L = run_gpu(inp)
    f, b = run_oracle(inp)
    assert list(f["counts"]) == counts
    check_parity(L, inp, f, b, tol_act=TOL_MX, tol_grad=TOL_MX)
    assert_bitwise_equal(outputs(L, False), outputs(run_gpu(inp, persistent=True), False))


def test_mxfp8_local_zipf_full_size_sampled_parity():
    """The full local expert slice in MXFP8 mode (16,384 rows, d=7168, I=2048, one expert over
    40%): the ring's codes and scales bit-exact on sampled positions, the heaviest and the
    lightest expert's dW1 and dW2, and sampled tokens of those two experts, against the MXFP8
    oracle; then a second run bitwise equal to the first."""
    _announce("[mxfp8] local_zipf 16384 rows d=7168 E=8 k=1 I=2048 seed 0, MXFP8")
    inp = workload.make_inputs("local_zipf", seed=0, device=DEV, precision="mxfp8")
    L = run_gpu(inp)
    X, dY = _np(inp["X"]), _np(inp["dY"])
    idx, w = _np(inp["topk_idx"]), _np(inp["topk_w"])
    counts, offsets, row_src, tk_row = oracle.permute(idx, 8)
    for n, want in (("counts", counts), ("offsets", offsets), ("row_src", row_src),
                    ("tk_row", tk_row)):
        np.testing.assert_array_equal(_np(getattr(L, n)), want, err_msg=n)
    pos = np.unique(np.concatenate([[0, len(row_src) - 1],
                                    np.random.default_rng(7).choice(len(row_src), 256)]))
    codes, scales = L.xp()
    q, sc = oracle.mx.quantize(X[row_src[pos]])
    p_dev = torch.from_numpy(pos).to(DEV)
    np.testing.assert_array_equal(_np(codes[p_dev]), q)
    np.testing.assert_array_equal(_np(scales[p_dev]), sc)
    _announce("  permutation and sampled ring codes bit-exact")
    nonempty = np.flatnonzero(counts)
    heavy = int(np.argmax(counts))
    light = int(nonempty[np.argmin(counts[nonempty])])
    W1h, W2h = workload.HostExperts(inp["W1"]), workload.HostExperts(inp["W2"])
    fe = oracle.forward(X, W1h, W2h, topk_idx=idx, topk_w=w, experts=[heavy, light],
                        precision="mxfp8")
    be = oracle.backward(fe, X, W1h, W2h, dY, experts=[heavy, light])
    for i, e in enumerate((heavy, light)):
        assert_grad(f"dW1[{e}] ({counts[e]} rows)", _np(L.dw1[e]), be["dW1"][i], TOL_MX)
        assert_grad(f"dW2[{e}] ({counts[e]} rows)", _np(L.dw2[e]), be["dW2"][i], TOL_MX)
    _announce("  heaviest and lightest experts' weight gradients done")
    rng = np.random.default_rng(8)
    tok = np.unique(np.concatenate([rng.choice(np.flatnonzero(idx[:, 0] == e), 8, replace=False)
                                    for e in (heavy, light)]))
    t_dev = torch.from_numpy(tok).to(DEV)
    rows = tk_row[tok]
    assert_act("Y[tokens]", _np(L.y[t_dev]), fe["Y"][tok], TOL_MX)
    assert_act("dX[tokens]", _np(L.dx[t_dev]), be["dX"][tok], TOL_MX)
    assert_grad("d_topk_w[tokens]", _np(L.d_topk_w[t_dev]), be["dw"][tok], TOL_MX)
    r_dev = torch.from_numpy(rows).to(DEV)
    assert_act("H[rows]", _np(L.H()[r_dev]), fe["H"][rows], TOL_MX)
    assert_act("dH[rows]", _np(L.dH()[r_dev]), be["dH"][rows], TOL_MX)
    ref = outputs(L, False)
    del L
    torch.cuda.empty_cache()
    assert_bitwise_equal(ref, outputs(run_gpu(inp), False, clone=False))
    _announce("  two full-size MXFP8 runs bitwise identical")


# --- MXFP8 weight gradients (MOE_FLAG_MXFP8_WGRAD) ---------------------------------------------

MXW_CASES = {
    "tiny": dict(name="tiny"),
    "ragged": dict(name="tiny", T=300, E=16, k=3, d=512, I=256),
    "zipf_local": dict(name="local_zipf", T=2048, d=256, I=256),
}


@pytest.mark.parametrize("case", list(MXW_CASES))
def test_mxfp8_weight_gradients_match_the_oracle(case):
    """Both weight gradients in MXFP8, their operands quantised along each expert's positions
    (blocks of 32 from the segment start): within 6e-2 of the oracle doing the same, with the
    rest of the layer as in MXFP8 mode; then two runs bitwise equal, and accumulate doubling."""
    spec = dict(MXW_CASES[case])
    name = spec.pop("name")
    _announce(f"[mxfp8 wgrad] case={case} shape={spec} seed=0")
    inp = _mx_inputs(name, seed=0, mx_wgrad=True, **spec)
    L = run_gpu(inp)
    f, b = run_oracle(inp)
    check_parity(L, inp, f, b, tol_act=TOL_MX, tol_grad=TOL_MX)
    routed = "Wr" in inp
    a = outputs(L, routed)
    assert_bitwise_equal(a, outputs(run_gpu(inp), routed, clone=False))
    first = [L.dw1.clone(), L.dw2.clone()]
    L.backward(inp.get("Wr"), inp["W1"], inp["W2"], inp["dY"], accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(L.dw1, 2 * first[0]) and torch.equal(L.dw2, 2 * first[1])


def test_mxfp8_weight_gradients_full_size_local_zipf():
    """MXFP8 weight gradients on the full local expert slice (16,384 rows, d=7168, I=2048, one
    expert of over 8,000 rows): the heaviest and the lightest expert's dW1 and dW2 within 6e-2
    of the oracle quantising the same operands along each expert's positions, then a second
    run bitwise equal to the first."""
    _announce("[mxfp8 wgrad] local_zipf 16384 rows d=7168 E=8 k=1 I=2048 seed 0")
    inp = _mx_inputs("local_zipf", seed=0, mx_wgrad=True)
    L = run_gpu(inp)
    X, dY = _np(inp["X"]), _np(inp["dY"])
    idx, w = _np(inp["topk_idx"]), _np(inp["topk_w"])
    counts = np.bincount(idx[:, 0], minlength=8)
    nonempty = np.flatnonzero(counts)
    heavy = int(np.argmax(counts))
    light = int(nonempty[np.argmin(counts[nonempty])])
    W1h, W2h = workload.HostExperts(inp["W1"]), workload.HostExperts(inp["W2"])
    fe = oracle.forward(X, W1h, W2h, topk_idx=idx, topk_w=w, experts=[heavy, light],
                        precision="mxfp8")
    be = oracle.backward(fe, X, W1h, W2h, dY, experts=[heavy, light], wgrad="mxfp8")
    for i, e in enumerate((heavy, light)):
        assert_grad(f"dW1[{e}] ({counts[e]} rows)", _np(L.dw1[e]), be["dW1"][i], TOL_MX)
        assert_grad(f"dW2[{e}] ({counts[e]} rows)", _np(L.dw2[e]), be["dW2"][i], TOL_MX)
    ref = outputs(L, False)
    del L
    torch.cuda.empty_cache()
    assert_bitwise_equal(ref, outputs(run_gpu(inp), False, clone=False))
    _announce("  two full-size runs with MXFP8 weight gradients bitwise identical")


def test_mxfp8_weight_gradients_with_large_and_empty_experts():
    """Experts of 700, 300, 0 and 24 rows at d=512, I=256: several 128-position K chunks, an
    empty expert (zero blocks) and segments starting off the 32-row grid."""
    counts = [700, 300, 0, 24]
    _announce(f"[mxfp8 wgrad] expert sizes {counts}, d=512 I=256 k=1")
    E, d, I = len(counts), 512, 256
    T = sum(counts)
    inp = workload.make_inputs("local_zipf", seed=15, device=DEV, T=T, d=d, E=E, I=I,
                               precision="mxfp8", mx_wgrad=True)
    idx = np.repeat(np.arange(E, dtype=np.int32), counts)
    np.random.default_rng(15).shuffle(idx)
    inp["topk_idx"] = torch.from_numpy(idx.reshape(T, 1)).to(DEV)
    L = run_gpu(inp)
    f, b = run_oracle(inp)
    assert list(f["counts"]) == counts
    check_parity(L, inp, f, b, tol_act=TOL_MX, tol_grad=TOL_MX)
    assert torch.count_nonzero(L.dw1[2]) == 0 and torch.count_nonzero(L.dw2[2]) == 0
