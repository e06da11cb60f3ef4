"""GPU parity of the MXFP4 mode against the oracle that emulates the same quantisation.

* The quantised weights and the permuted tokens are integer codes (E2M1 nibbles, two a byte,
  and E8M0 scales): they must equal the oracle's quantiser bit for bit, edge values included.
* Routing and the permutation maps are bit-exact, as in BF16 mode.
* Floating outputs and gradients must be within the BF16 mode's bar of the MXFP4-emulating
  oracle: 1e-2 for Y, dX and the saved activations (max-abs and RMS relative error), 2e-2 for
  the weight, router and routing-weight gradients (relative Frobenius error).
* Two runs (one-shot and persistent grids) are bitwise identical, and accumulate doubles the
  weight gradients exactly.

Tolerance. Both sides quantise the same bf16 values with the same rule, and every product of
two E2M1 values times two power-of-two scales is exact, so the GEMM outputs differ only by fp32
summation order (H, O and dXp come out bit-equal to the oracle's at these shapes). What remains
comes from A and dH, which the layer rounds to bf16 and then quantises: where the GPU's bf16
value differs from the oracle's by one ulp (fp32 against fp64 sums), it can cross an E2M1
rounding midpoint, moving one code by up to half its value, or change a block maximum's binade.
Such flips touch few elements, and each moves one term of the next GEMM's sum: measured, Y and
dX stay within 2.1e-3 (max-abs) and the gradients within 1.7e-3, so the BF16 bar holds with a
margin of five.
"""
import numpy as np
import pytest
import torch

import oracle
import workload
from tests._gpu import (DEV, MoeLayer, _announce, _np, assert_bitwise_equal, check_parity,
                        codes_of, m, outputs, run_gpu, run_oracle)
from tests._util import TOL_ACT, TOL_GRAD, assert_act, assert_grad

pytestmark = pytest.mark.gpu


def _up(v):
    return (v + 255) // 256 * 256


def _wq_parts(L):
    """The four MXFP4 weight tensors (element codes unpacked from their nibbles) and their
    scales inside L.wq, in the order the header lists them: W1 along d, W2 along I, W2
    transposed along d, W1 transposed along 2I."""
    E, d, I = L.E, L.d, L.I
    shapes = [(E, 2 * I, d), (E, d, I), (E, I, d), (E, d, 2 * I)]
    out, o = [], 0
    for sh in shapes:
        n = sh[0] * sh[1] * sh[2]
        raw = L.wq[o:o + n // 2].view(sh[0], sh[1], sh[2] // 2)
        o += _up(n // 2)
        sc = L.wq[o:o + n // 32].view(sh[0], sh[1], sh[2] // 32)
        o += _up(n // 32)
        out.append((raw, sc))
    return out


def _check_weights(L, W1, W2, experts=None):
    W1n, W2n = _np(W1), _np(W2)
    refs = [oracle.mx.quantize(W1n, fmt="e2m1"), oracle.mx.quantize(W2n, fmt="e2m1"),
            oracle.mx.quantize(np.swapaxes(W2n, 1, 2), fmt="e2m1"),
            oracle.mx.quantize(np.swapaxes(W1n, 1, 2), fmt="e2m1")]
    for i, ((raw, sc), (q, s)) in enumerate(zip(_wq_parts(L), refs)):
        np.testing.assert_array_equal(_np(sc), s, err_msg=f"scales of part {i}")
        np.testing.assert_array_equal(codes_of(_np(raw), "e2m1"), q, err_msg=f"codes of part {i}")


def _mx4_inputs(name="tiny", seed=0, **over):
    return workload.make_inputs(name, seed=seed, device=DEV, precision="mxfp4", **over)


def test_mxfp4_weight_quantisation_is_bit_exact():
    _announce("[mxfp4] quantised weights, tiny shape")
    inp = _mx4_inputs(seed=0, E=4)
    L = run_gpu(inp)
    _check_weights(L, inp["W1"], inp["W2"])


def _special_blocks(rows, cols, seed):
    """bf16 values [rows, cols] whose 32-blocks along the row exercise the edges of the MXFP4
    quantiser: all +0 and all -0 blocks, bf16 subnormals, the top of the bf16 range, exact
    powers of two, every E2M1 rounding tie at unit scale (block maximum 4), values in (6, 8)
    after scaling (saturation), one large value over tiny ones, and plain normal values."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    nb = cols // 32
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    for r in range(rows):
        for b in range(nb):
            kind = (r * nb + b) % 10
            blk = x[r, 32 * b:32 * b + 32]
            if kind == 0:
                blk[:] = 0.0
            elif kind == 1:
                blk[:] = -0.0
            elif kind == 2:
                blk[:] = rng.choice([-1, 1], 32) * rng.integers(1, 128, 32) * 2.0 ** -133
            elif kind == 3:
                blk[:] = rng.choice([-1, 1], 32) * rng.uniform(1.0, 1.99, 32) * 2.0 ** 127
            elif kind == 4:
                blk[:] = rng.choice([-1, 1], 32) * 2.0 ** rng.integers(-20, 20, 32)
            elif kind == 5:  # amax 4 -> scale 1; every tie, both signs, and a few between
                blk[:] = [4.0] + ties + [-t for t in ties] + [0.5, 1.0, 1.5, 2.0, 3.0, 6.0,
                                                              0.1, 0.3, 0.7, 1.3, 2.2, 3.3,
                                                              -4.4, 4.9, 5.5, -5.1, 0.0]
            elif kind == 6:  # block maximum in (6, 8) after scaling: saturates
                blk[:] = rng.uniform(-1, 1, 32) * 4.0
                blk[0] = 7.0
                blk[1] = -7.5
            elif kind == 7:
                blk[:] = rng.standard_normal(32) * 1e-6
                blk[5] = 3.0e4
    return torch.from_numpy(x).to(torch.bfloat16)


def test_mxfp4_quantiser_edge_values_are_bit_exact():
    """Weights and tokens built from the quantiser's edge cases: the GPU's E2M1 codes and scales
    of W1, W2 (both axes) and of the permuted tokens equal the oracle's quantiser bit for bit."""
    _announce("[mxfp4] quantiser edge values, E=4 d=256 I=256 T=64 k=2")
    T, d, E, k, I = 64, 256, 4, 2, 256
    W1 = _special_blocks(E * 2 * I, d, 1).reshape(E, 2 * I, d).to(DEV)
    W2 = _special_blocks(E * d, I, 2).reshape(E, d, I).to(DEV)
    X = _special_blocks(T, d, 3).to(DEV)
    L = MoeLayer(T, d, E, k, I, device=DEV, precision=m.MOE_PREC_MXFP4)
    L.quantize_weights(W1, W2)
    idx = torch.tensor([[t % E, (t + 1) % E] for t in range(T)], dtype=torch.int32)
    L.set_routing(idx.to(DEV), torch.full((T, k), 0.5, dtype=torch.float32, device=DEV))
    L.permute(X)
    torch.cuda.synchronize()
    _check_weights(L, W1, W2)
    row_src = _np(L.row_src)
    codes, scales = L.xp()
    q, sc = oracle.mx.quantize(_np(X)[row_src // k], fmt="e2m1")
    np.testing.assert_array_equal(_np(scales), sc)
    np.testing.assert_array_equal(codes_of(_np(codes), "e2m1"), q)


MX4_CASES = {
    "tiny": dict(name="tiny"),
    "ragged": dict(name="tiny", T=300, E=16, k=3, d=512, I=256),
    "multi_mtile": dict(name="tiny", T=1024, E=4, k=2, d=512, I=256),
    "zipf_local": dict(name="local_zipf", T=2048, d=256, I=256),
    "d768": dict(name="tiny", T=200, E=4, k=2, d=768, I=256),  # 24 scale bytes a row
}


@pytest.mark.parametrize("case", list(MX4_CASES))
def test_mxfp4_layer_parity(case):
    spec = dict(MX4_CASES[case])
    name = spec.pop("name")
    _announce(f"[mxfp4] case={case} shape={spec} seed=0")
    inp = _mx4_inputs(name, seed=0, **spec)
    L = run_gpu(inp)
    f, b = run_oracle(inp)
    check_parity(L, inp, f, b, tol_act=TOL_ACT, tol_grad=TOL_GRAD)


def test_mxfp4_expert_sizes_at_tile_boundaries_and_determinism():
    """Experts of 0, 1, 127, 128, 129, 255, 256, 257, 384, 511, 512 and 513 rows (full 256-row
    blocks on the direct-to-LDS kernels, 128-row remainder tiles and their ragged last tile; from
    512 rows the weight gradients' big-expert kernel, which reads the expert's Xp rows expanded
    from their E2M1 codes), d = 512 and I = 512 (two K steps of 256 along d and I, several
    column tiles): parity against the MXFP4 oracle, persistent grids bitwise equal to one-shot
    grids, and a second backward with accumulate doubling both weight gradients exactly."""
    counts = [255, 256, 257, 0, 127, 128, 129, 1, 384, 511, 512, 513]
    _announce(f"[mxfp4] expert sizes {counts}, d=512 I=512 k=1")
    E, d, I = len(counts), 512, 512
    T = sum(counts)
    inp = workload.make_inputs("local_zipf", seed=9, device=DEV, T=T, d=d, E=E, I=I,
                               precision="mxfp4")
    idx = np.repeat(np.arange(E, dtype=np.int32), counts)
    np.random.default_rng(9).shuffle(idx)
    inp["topk_idx"] = torch.from_numpy(idx.reshape(T, 1)).to(DEV)
    L = run_gpu(inp)
    f, b = run_oracle(inp)
    assert list(f["counts"]) == counts
    check_parity(L, inp, f, b, tol_act=TOL_ACT, tol_grad=TOL_GRAD)
    assert_bitwise_equal(outputs(L, False), outputs(run_gpu(inp, persistent=True), False))
    first = [g.clone() for g in (L.dw1, L.dw2)]
    L.backward(None, inp["W1"], inp["W2"], inp["dY"], accumulate=True)
    torch.cuda.synchronize()
    for g0, g in zip(first, (L.dw1, L.dw2)):
        assert torch.equal(g, 2 * g0)
    assert torch.count_nonzero(L.dw1[3]) == 0 and torch.count_nonzero(L.dw2[3]) == 0


def test_mxfp4_big_expert_wgrad_with_accumulation():
    """One expert of 700 rows beside small and empty experts (the gate wgrad reads the big
    expert's Xp rows expanded from their E2M1 codes into the dXp buffer, and the others' codes
    directly): parity with the MXFP4 oracle, then a second backward with accumulate=1 doubles
    dW1 and dW2 exactly."""
    counts = [700, 300, 0, 24]
    _announce(f"[mxfp4] big expert {counts}, d=512 I=256 k=1, accumulate")
    E, d, I = len(counts), 512, 256
    T = sum(counts)
    inp = _mx4_inputs("local_zipf", seed=13, T=T, d=d, E=E, I=I)
    idx = np.repeat(np.arange(E, dtype=np.int32), counts)
    np.random.default_rng(13).shuffle(idx)
    inp["topk_idx"] = torch.from_numpy(idx.reshape(T, 1)).to(DEV)
    L = run_gpu(inp)
    f, b = run_oracle(inp)
    assert list(f["counts"]) == counts
    check_parity(L, inp, f, b, tol_act=TOL_ACT, tol_grad=TOL_GRAD)
    first = [g.clone() for g in (L.dw1, L.dw2)]
    L.backward(None, inp["W1"], inp["W2"], inp["dY"], accumulate=True)
    torch.cuda.synchronize()
    for g0, g in zip(first, (L.dw1, L.dw2)):
        assert torch.equal(g, 2 * g0)
    assert torch.count_nonzero(L.dw1[2]) == 0 and torch.count_nonzero(L.dw2[2]) == 0


def test_mxfp4_routed_layer_determinism_and_dwr_accumulation():
    """The routed layer (router, dWr from the E2M1 Xp codes) twice: bitwise equal, and
    dWr doubles exactly under accumulate."""
    _announce("[mxfp4] determinism, routed multi-m-tile shape")
    inp = _mx4_inputs("tiny", seed=2, T=1024, E=8, k=2, d=512, I=256)
    L = run_gpu(inp)
    a = outputs(L, True)
    assert_bitwise_equal(a, outputs(run_gpu(inp, persistent=True), True, clone=False))
    dwr = L.dwr.clone()
    L.backward(inp["Wr"], inp["W1"], inp["W2"], inp["dY"], accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(L.dwr, 2 * dwr)


def test_mxfp4_full_size_sampled_parity_and_determinism():
    """The DeepSeek-V3 shape in MXFP4 mode: routing and permutation bit-exact, ring codes and the
    heaviest expert's quantised weights bit-exact, one sampled token and the heaviest expert's
    weight gradients against the MXFP4 oracle, then a second run bitwise equal."""
    _announce("[mxfp4] dsv3_mxfp4 T=2048 d=7168 E=256 k=8 I=2048 seed 0")
    inp = workload.make_inputs("dsv3_mxfp4", seed=0, device=DEV)
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
    q, sc = oracle.mx.quantize(X[row_src[pos] // k], fmt="e2m1")
    p_dev = torch.from_numpy(pos).to(DEV)
    np.testing.assert_array_equal(codes_of(_np(codes[p_dev]), "e2m1"), q)
    np.testing.assert_array_equal(_np(scales[p_dev]), sc)
    _announce("  ring codes and scales bit-exact on sampled positions")
    heavy = int(np.argmax(counts))
    W1e, W2e = _np(inp["W1"][heavy]), _np(inp["W2"][heavy])
    refs = [oracle.mx.quantize(W1e, fmt="e2m1"), oracle.mx.quantize(W2e, fmt="e2m1"),
            oracle.mx.quantize(W2e.T, fmt="e2m1"), oracle.mx.quantize(W1e.T, fmt="e2m1")]
    for i, ((raw, cs), (rq, rs)) in enumerate(zip(_wq_parts(L), refs)):
        np.testing.assert_array_equal(_np(cs[heavy]), rs, err_msg=f"scales of part {i}")
        np.testing.assert_array_equal(codes_of(_np(raw[heavy]), "e2m1"), rq,
                                      err_msg=f"codes of part {i}")
    _announce(f"  quantised weights of expert {heavy} bit-exact")
    W1h, W2h = workload.HostExperts(inp["W1"]), workload.HostExperts(inp["W2"])
    tok = np.array([int(np.random.default_rng(6).integers(X.shape[0]))])
    f = oracle.forward(X[tok], W1h, W2h, Wr=Wr, k=k, precision="mxfp4")
    bk = oracle.backward(f, X[tok], W1h, W2h, dY[tok], Wr=Wr)
    t_dev = torch.from_numpy(tok).to(DEV)
    assert_act("Y[token]", _np(L.y[t_dev]), f["Y"], TOL_ACT)
    assert_act("dX[token]", _np(L.dx[t_dev]), bk["dX"], TOL_ACT)
    assert_grad("d_topk_w[token]", _np(L.d_topk_w[t_dev]), bk["dw"], TOL_GRAD)
    fe = oracle.forward(X, W1h, W2h, Wr=Wr, k=k, experts=[heavy], precision="mxfp4")
    be = oracle.backward(fe, X, W1h, W2h, dY, Wr=Wr, experts=[heavy])
    assert_grad(f"dW1[{heavy}]", _np(L.dw1[heavy]), be["dW1"][0], TOL_GRAD)
    assert_grad(f"dW2[{heavy}]", _np(L.dw2[heavy]), be["dW2"][0], TOL_GRAD)
    ref = outputs(L, True)
    del L
    torch.cuda.empty_cache()
    assert_bitwise_equal(ref, outputs(run_gpu(inp), True, clone=False))
    _announce("  two full-size MXFP4 runs bitwise identical")


def test_mxfp4_local_zipf_full_size_sampled_parity():
    """The full local expert slice in MXFP4 mode (16,384 rows, d=7168, I=2048, one expert over
    40%: the 256-row MXFP4 kernels and the weight gradients' big-expert kernel on expanded E2M1
    rows): the ring's codes and scales bit-exact on sampled positions, the heaviest and the
    lightest expert's dW1 and dW2, and sampled tokens of those two experts, against the MXFP4
    oracle at the BF16 bar; then a second run bitwise equal to the first."""
    _announce("[mxfp4] local_zipf 16384 rows d=7168 E=8 k=1 I=2048 seed 0, MXFP4")
    inp = _mx4_inputs("local_zipf")
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
    q, sc = oracle.mx.quantize(X[row_src[pos]], fmt="e2m1")
    p_dev = torch.from_numpy(pos).to(DEV)
    np.testing.assert_array_equal(codes_of(_np(codes[p_dev]), "e2m1"), q)
    np.testing.assert_array_equal(_np(scales[p_dev]), sc)
    _announce("  permutation and sampled ring codes bit-exact")
    nonempty = np.flatnonzero(counts)
    heavy = int(np.argmax(counts))
    light = int(nonempty[np.argmin(counts[nonempty])])
    W1h, W2h = workload.HostExperts(inp["W1"]), workload.HostExperts(inp["W2"])
    fe = oracle.forward(X, W1h, W2h, topk_idx=idx, topk_w=w, experts=[heavy, light],
                        precision="mxfp4")
    be = oracle.backward(fe, X, W1h, W2h, dY, experts=[heavy, light])
    for i, e in enumerate((heavy, light)):
        assert_grad(f"dW1[{e}] ({counts[e]} rows)", _np(L.dw1[e]), be["dW1"][i], TOL_GRAD)
        assert_grad(f"dW2[{e}] ({counts[e]} rows)", _np(L.dw2[e]), be["dW2"][i], TOL_GRAD)
    _announce("  heaviest and lightest experts' weight gradients done")
    rng = np.random.default_rng(8)
    tok = np.unique(np.concatenate([rng.choice(np.flatnonzero(idx[:, 0] == e), 8, replace=False)
                                    for e in (heavy, light)]))
    t_dev = torch.from_numpy(tok).to(DEV)
    rows = tk_row[tok]
    assert_act("Y[tokens]", _np(L.y[t_dev]), fe["Y"][tok], TOL_ACT)
    assert_act("dX[tokens]", _np(L.dx[t_dev]), be["dX"][tok], TOL_ACT)
    assert_grad("d_topk_w[tokens]", _np(L.d_topk_w[t_dev]), be["dw"][tok], TOL_GRAD)
    r_dev = torch.from_numpy(rows).to(DEV)
    assert_act("H[rows]", _np(L.H()[r_dev]), fe["H"][rows], TOL_ACT)
    assert_act("dH[rows]", _np(L.dH()[r_dev]), be["dH"][rows], TOL_ACT)
    ref = outputs(L, False)
    del L
    torch.cuda.empty_cache()
    assert_bitwise_equal(ref, outputs(run_gpu(inp), False, clone=False))
    _announce("  two full-size MXFP4 runs bitwise identical")
