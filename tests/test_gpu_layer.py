"""GPU parity of the whole layer against the CPU oracle, through the C ABI.

Integer outputs are compared bit for bit: router logits (fp32 in a stated order), top-k
indices, counts, offsets and both permutation maps, plus the permuted tokens, which are a pure
copy. Floating outputs use the layer's tolerances. The bf16 output Y and the input gradient dX
must be within 1e-2 relative error, both max-abs and RMS. The weight, router and routing-weight
gradients must be within 2e-2 relative Frobenius error. The oracle is the float64 CPU
implementation with bf16 rounding at the same storage points.
"""
import numpy as np
import pytest
import torch

import oracle
import workload
from mixture_experts_layer_deterministic_amd.layer import Macrobatch
from tests._gpu import (DEV, MoeLayer, _announce, _np, assert_bitwise_equal, check_parity, m,
                        outputs, run_gpu, run_oracle)
from tests._util import assert_act, assert_grad

pytestmark = pytest.mark.gpu

# ---------------------------------------------------------------------------------------------

SMALL = {
    "tiny": dict(name="tiny"),
    "ragged": dict(name="tiny", T=300, E=16, k=3, d=512, I=256),
    "multi_mtile": dict(name="tiny", T=1024, E=4, k=2, d=512, I=256),
    "single_token": dict(name="tiny", T=1, E=4, k=2, d=256, I=128),
    "k_equals_E": dict(name="tiny", T=64, E=4, k=4, d=256, I=128),
    "zipf_local": dict(name="local_zipf", T=2048, d=256, I=256),
}


@pytest.mark.parametrize("case", list(SMALL))
def test_layer_parity(case):
    spec = dict(SMALL[case])
    name = spec.pop("name")
    _announce(f"[parity] case={case} shape={spec} seed=0")
    inp = workload.make_inputs(name, seed=0, device=DEV, **spec)
    L = run_gpu(inp)
    f, b = run_oracle(inp)
    check_parity(L, inp, f, b)


def test_persistent_grid_is_bitwise_identical_to_one_shot():
    _announce("[persistent] tiny and zipf_local")
    for name, spec in (("tiny", {}), ("local_zipf", dict(T=2048, d=256, I=256))):
        inp = workload.make_inputs(name, seed=1, device=DEV, **spec)
        a = outputs(run_gpu(inp, persistent=False), "Wr" in inp)
        b = outputs(run_gpu(inp, persistent=True), "Wr" in inp)
        assert_bitwise_equal(a, b)


def test_two_runs_are_bitwise_identical():
    _announce("[determinism] multi_mtile twice")
    inp = workload.make_inputs("tiny", seed=2, device=DEV, T=1024, E=8, k=2, d=512, I=256)
    a = outputs(run_gpu(inp), True)
    # a concurrent kernel on another stream perturbs timing between the runs
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        junk = torch.randn(4096, 4096, device=DEV)
        for _ in range(4):
            junk = junk @ junk.T
            junk = junk / junk.norm()
    b = outputs(run_gpu(inp), True)
    torch.cuda.synchronize()
    assert_bitwise_equal(a, b)


def test_ring_slot_one_matches_slot_zero():
    _announce("[ring] slot 1 of 2")
    inp = workload.make_inputs("tiny", seed=3, device=DEV)
    a = outputs(run_gpu(inp, slot=0, ring_slots=1), True)
    b = outputs(run_gpu(inp, slot=1, ring_slots=2), True)
    assert_bitwise_equal(a, b)


def test_all_rows_to_one_expert_and_empty_experts():
    _announce("[imbalance] every row to expert 2")
    T, d, E, I = 512, 256, 4, 128
    inp = workload.make_inputs("local_zipf", seed=4, device=DEV, T=T, d=d, E=E, I=I)
    inp["topk_idx"] = torch.full((T, 1), 2, dtype=torch.int32, device=DEV)
    L = run_gpu(inp)
    f, b = run_oracle(inp)
    check_parity(L, inp, f, b)
    for e in (0, 1, 3):
        assert torch.count_nonzero(L.dw1[e]) == 0 and torch.count_nonzero(L.dw2[e]) == 0


def test_expert_sizes_at_the_256_row_block_boundaries():
    """Experts of 0, 1, 128, 255, 256, 257, 384, 511, 512 and 513 rows: the forward GEMMs split
    each expert into full 256-row blocks (big-tile kernel) and 128-row remainder tiles. Parity
    against the oracle, and persistent grids bitwise equal to one-shot grids."""
    counts = [255, 256, 257, 0, 511, 512, 513, 1, 128, 384]
    _announce(f"[blocks] expert sizes {counts}, d=256 I=256 k=1")
    E, d, I = len(counts), 256, 256
    T = sum(counts)
    inp = workload.make_inputs("local_zipf", seed=9, device=DEV, T=T, d=d, E=E, I=I)
    idx = np.repeat(np.arange(E, dtype=np.int32), counts)
    np.random.default_rng(9).shuffle(idx)
    inp["topk_idx"] = torch.from_numpy(idx.reshape(T, 1)).to(DEV)
    L = run_gpu(inp)
    f, b = run_oracle(inp)
    assert list(f["counts"]) == counts
    check_parity(L, inp, f, b)
    a = outputs(L, False)
    assert_bitwise_equal(a, outputs(run_gpu(inp, persistent=True), False))


def test_large_experts_on_the_256_tile_kernels_and_accumulation():
    """Experts of 2500, 1000, 596 and 0 rows at d=1024, I=512: the 256 x 256 dgrad kernels
    (several K steps and column tiles, with 128-row remainders on the small kernel) and the
    big-expert wgrad kernel, against the oracle. A second backward with accumulate=1 must then
    double every weight gradient exactly (x + x is exact in fp32), which covers the
    accumulating forms of both wgrad kernels."""
    counts = [2500, 1000, 596, 0]
    _announce(f"[large] expert sizes {counts}, d=1024 I=512 k=1")
    E, d, I = len(counts), 1024, 512
    T = sum(counts)
    inp = workload.make_inputs("local_zipf", seed=11, device=DEV, T=T, d=d, E=E, I=I)
    idx = np.repeat(np.arange(E, dtype=np.int32), counts)
    np.random.default_rng(11).shuffle(idx)
    inp["topk_idx"] = torch.from_numpy(idx.reshape(T, 1)).to(DEV)
    L = run_gpu(inp)
    f, b = run_oracle(inp)
    assert list(f["counts"]) == counts
    check_parity(L, inp, f, b)
    first = [g.clone() for g in (L.dw1, L.dw2)]
    L.backward(None, inp["W1"], inp["W2"], inp["dY"], accumulate=True)
    torch.cuda.synchronize()
    for g0, g in zip(first, (L.dw1, L.dw2)):
        assert torch.equal(g, 2 * g0)


def test_caller_routing_may_repeat_an_expert_within_a_token():
    """Given routing whose rows name one expert twice for a third of the tokens: each row is its
    own position, so the expert receives both rows, and the layer still matches the oracle."""
    T, d, E, k, I = 300, 256, 6, 2, 128
    _announce(f"[repeat] T={T} d={d} E={E} k={k} I={I}, a third of the tokens repeat an expert")
    inp = workload.make_inputs("local_zipf", seed=12, device=DEV, T=T, d=d, E=E, k=k, I=I)
    rng = np.random.default_rng(12)
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    idx[::3, 1] = idx[::3, 0]
    inp["topk_idx"] = torch.from_numpy(idx).to(DEV)
    inp["topk_w"] = torch.from_numpy(rng.random((T, k)).astype(np.float32)).to(DEV)
    L = run_gpu(inp)
    f, b = run_oracle(inp)
    check_parity(L, inp, f, b)


def test_zero_router_and_duplicate_router_rows():
    _announce("[ties] zero router, duplicate rows")
    inp = workload.make_inputs("tiny", seed=5, device=DEV)
    inp["Wr"] = torch.zeros_like(inp["Wr"])
    L = run_gpu(inp)
    k = inp["cfg"]["k"]
    want = torch.arange(k, dtype=torch.int32, device=DEV).expand(inp["cfg"]["T"], k)
    assert torch.equal(L.topk_idx, want)
    assert torch.all(L.topk_w == 1.0 / k)
    inp = workload.make_inputs("tiny", seed=6, device=DEV)
    inp["Wr"][5] = inp["Wr"][1]
    inp["Wr"][6] = inp["Wr"][1]
    L = run_gpu(inp)
    f, b = run_oracle(inp)
    check_parity(L, inp, f, b)


def test_bad_expert_index_sets_the_device_status():
    _announce("[status] out-of-range expert index")
    T, d, E, I = 64, 256, 4, 128
    inp = workload.make_inputs("local_zipf", seed=7, device=DEV, T=T, d=d, E=E, I=I)
    inp["topk_idx"] = inp["topk_idx"] % E
    inp["topk_idx"][10, 0] = E + 3
    L = run_gpu(inp)
    assert L.device_status() == m.MOE_DEVICE_BAD_EXPERT_INDEX
    assert int(L.tk_row[10].item()) == -1
    assert int(L.offsets[E].item()) == T - 1
    assert torch.all(L.dx[10] == 0)
    good = workload.make_inputs("local_zipf", seed=7, device=DEV, T=T, d=d, E=E, I=I)
    good["topk_idx"] = good["topk_idx"] % E
    assert run_gpu(good).device_status() == 0


def test_streaming_microbatches_with_ring_replay():
    """Microbatches 0..n-1 go forward through a 2-slot ring, and backward walks n-1..0. Slots
    overwritten by later microbatches are re-permuted (replayed) before their backward. The
    weight gradients accumulate across microbatches."""
    _announce("[stream] 4 microbatches, 2 slots, reverse walk with replay")
    nmb, S = 4, 2
    inp = workload.make_inputs("stream", seed=8, device=DEV, T=64, d=256, E=16, k=4, I=128,
                               microbatches=nmb)
    cfg = inp["cfg"]
    T, d, E, k, I = cfg["T"], cfg["d"], cfg["E"], cfg["k"], cfg["I"]
    L = MoeLayer(T, d, E, k, I, device=DEV, ring_slots=S)
    saved = [torch.empty_like(L.saved) for _ in range(nmb)]
    routing = []
    ys = []
    for i in range(nmb):
        L.route(inp["X"][i], inp["Wr"])
        L.permute(inp["X"][i], slot=i % S)
        L.forward(inp["W1"], inp["W2"], slot=i % S, saved=saved[i])
        ys.append(L.y.clone())
        routing.append((L.topk_idx.clone(), L.topk_w.clone(), L.counts.clone(),
                        L.offsets.clone(), L.row_src.clone(), L.tk_row.clone()))
    dxs = [None] * nmb
    for i in reversed(range(nmb)):
        for dst, src in zip((L.topk_idx, L.topk_w, L.counts, L.offsets, L.row_src, L.tk_row),
                            routing[i]):
            dst.copy_(src)
        if i < nmb - S:
            L.permute(inp["X"][i], slot=i % S)   # replay: the slot was overwritten
        L.backward(inp["Wr"], inp["W1"], inp["W2"], inp["dY"][i], slot=i % S,
                   accumulate=(i != nmb - 1), saved=saved[i])
        dxs[i] = L.dx.clone()
    torch.cuda.synchronize()
    X, W1, W2, dY, Wr = (_np(inp[n]) for n in ("X", "W1", "W2", "dY", "Wr"))
    dW1 = np.zeros_like(W1, dtype=np.float64)
    dW2 = np.zeros_like(W2, dtype=np.float64)
    dWr = np.zeros_like(Wr, dtype=np.float64)
    for i in range(nmb):
        f = oracle.forward(X[i], W1, W2, Wr=Wr, k=k)
        b = oracle.backward(f, X[i], W1, W2, dY[i], Wr=Wr)
        assert_act(f"Y[{i}]", _np(ys[i]), f["Y"])
        assert_act(f"dX[{i}]", _np(dxs[i]), b["dX"])
        dW1 += b["dW1"]
        dW2 += b["dW2"]
        dWr += b["dWr"]
    assert_grad("dW1 (sum)", _np(L.dw1), dW1)
    assert_grad("dW2 (sum)", _np(L.dw2), dW2)
    assert_grad("dWr (sum)", _np(L.dwr), dWr)


@pytest.mark.parametrize("prec", ["mxfp8", "mxfp4"])
def test_streaming_microbatches_with_ring_replay_in_mx_modes(prec):
    """The reverse ring walk with replay in the MX modes, where a ring slot holds the
    microbatch's MX codes and scales: weights quantised once, 4 microbatches through 2 slots,
    the overwritten slots re-permuted before their backward, the weight gradients accumulated.
    Against the oracle emulating the same quantisation (6e-2 for MXFP8; the BF16 bar for
    MXFP4, which its emulation meets)."""
    _announce(f"[stream {prec}] 4 microbatches, 2 slots, reverse walk with replay")
    nmb, S = 4, 2
    inp = workload.make_inputs("stream", seed=9, device=DEV, T=64, d=256, E=16, k=4, I=256,
                               microbatches=nmb)
    cfg = inp["cfg"]
    T, d, E, k, I = cfg["T"], cfg["d"], cfg["E"], cfg["k"], cfg["I"]
    code = m.MOE_PREC_MXFP8 if prec == "mxfp8" else m.MOE_PREC_MXFP4
    tol_a, tol_g = (6e-2, 6e-2) if prec == "mxfp8" else (1e-2, 2e-2)
    L = MoeLayer(T, d, E, k, I, device=DEV, ring_slots=S, precision=code)
    L.quantize_weights(inp["W1"], inp["W2"])
    saved = [torch.empty_like(L.saved) for _ in range(nmb)]
    routing, ys = [], []
    for i in range(nmb):
        L.route(inp["X"][i], inp["Wr"])
        L.permute(inp["X"][i], slot=i % S)
        L.forward(inp["W1"], inp["W2"], slot=i % S, saved=saved[i])
        ys.append(L.y.clone())
        routing.append((L.topk_idx.clone(), L.topk_w.clone(), L.counts.clone(),
                        L.offsets.clone(), L.row_src.clone(), L.tk_row.clone()))
    dxs = [None] * nmb
    for i in reversed(range(nmb)):
        for dst, src in zip((L.topk_idx, L.topk_w, L.counts, L.offsets, L.row_src, L.tk_row),
                            routing[i]):
            dst.copy_(src)
        if i < nmb - S:
            L.permute(inp["X"][i], slot=i % S)   # replay: the slot was overwritten
        L.backward(inp["Wr"], inp["W1"], inp["W2"], inp["dY"][i], slot=i % S,
                   accumulate=(i != nmb - 1), saved=saved[i])
        dxs[i] = L.dx.clone()
    torch.cuda.synchronize()
    X, W1, W2, dY, Wr = (_np(inp[n]) for n in ("X", "W1", "W2", "dY", "Wr"))
    dW1 = np.zeros_like(W1, dtype=np.float64)
    dW2 = np.zeros_like(W2, dtype=np.float64)
    dWr = np.zeros_like(Wr, dtype=np.float64)
    for i in range(nmb):
        f = oracle.forward(X[i], W1, W2, Wr=Wr, k=k, precision=prec)
        b = oracle.backward(f, X[i], W1, W2, dY[i], Wr=Wr)
        assert_act(f"Y[{i}]", _np(ys[i]), f["Y"], tol_a)
        assert_act(f"dX[{i}]", _np(dxs[i]), b["dX"], tol_a)
        dW1 += b["dW1"]
        dW2 += b["dW2"]
        dWr += b["dWr"]
    assert_grad("dW1 (sum)", _np(L.dw1), dW1, tol_g)
    assert_grad("dW2 (sum)", _np(L.dw2), dW2, tol_g)
    assert_grad("dWr (sum)", _np(L.dwr), dWr, tol_g)


def _macro_outputs(mb):
    outs = []
    for b in mb.mb:
        outs += [b[n].clone() for n in ("topk_idx", "topk_w", "counts", "offsets", "row_src",
                                         "tk_row", "y", "dx", "d_topk_w")]
    return outs + [mb.dw1.clone(), mb.dw2.clone(), mb.dwr.clone()]


def test_macrobatch_overlap_matches_the_serial_walk_and_the_oracle():
    """The macrobatch runner with the next microbatch's routing and permutation (and, in
    backward, the next replay) on a second stream: bitwise equal to the serial ring walk, and
    equal to the oracle per microbatch (Y, dX) and summed (dW1, dW2, dWr)."""
    nmb = 5
    _announce(f"[macrobatch] {nmb} microbatches, 2-slot ring, serial vs two streams")
    inp = workload.make_inputs("stream", seed=14, device=DEV, T=96, d=256, E=16, k=4, I=128,
                               microbatches=nmb)
    c = inp["cfg"]
    T, d, E, k, I = c["T"], c["d"], c["E"], c["k"], c["I"]
    slot = m.moe_query(m.make_cfg(T, d, E, k, I)).ring_slot
    runs = []
    for overlap in (False, True, True):
        mb = Macrobatch(T, d, E, k, I, nmb, 2 * slot, device=DEV, overlap=overlap)
        assert mb.S == 2
        mb.run(inp["X"], inp["Wr"], inp["W1"], inp["W2"], inp["dY"])
        torch.cuda.synchronize()
        runs.append(_macro_outputs(mb))
    assert_bitwise_equal(runs[0], runs[1])
    assert_bitwise_equal(runs[0], runs[2])
    X, W1, W2, dY, Wr = (_np(inp[n]) for n in ("X", "W1", "W2", "dY", "Wr"))
    dW1 = dW2 = dWr = 0
    for i in range(nmb):
        f = oracle.forward(X[i], W1, W2, Wr=Wr, k=k)
        b = oracle.backward(f, X[i], W1, W2, dY[i], Wr=Wr)
        assert_act(f"Y[{i}]", _np(mb.mb[i]["y"]), f["Y"])
        assert_act(f"dX[{i}]", _np(mb.mb[i]["dx"]), b["dX"])
        dW1, dW2, dWr = dW1 + b["dW1"], dW2 + b["dW2"], dWr + b["dWr"]
    assert_grad("dW1 (sum)", _np(mb.dw1), dW1)
    assert_grad("dW2 (sum)", _np(mb.dw2), dW2)
    assert_grad("dWr (sum)", _np(mb.dwr), dWr)
