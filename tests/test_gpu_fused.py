"""The single-launch forward (moe_forward_fused) against the separate calls and the oracle.

moe_forward_fused runs the router, the permutation, both grouped GEMMs and the combine as
phases of one cooperatively launched kernel. Its outputs must equal those of moe_route +
moe_permute + moe_forward bit for bit whenever no expert receives 256 rows (the separate path
gives full 256-row blocks another tile); otherwise they must match the oracle within the
layer's tolerances. Repeated calls reuse the grid barrier's state, so they are run several
times in a row, and the device status word must show no barrier timeout.
"""
import pytest
import torch

import workload
from tests._gpu import DEV, MoeLayer, _announce, assert_bitwise_equal, check_parity, run_oracle

pytestmark = pytest.mark.gpu


def _layer(inp):
    c = inp["cfg"]
    return MoeLayer(c["T"], c["d"], c["E"], c["k"], c["I"], device=DEV)


def _fwd_outputs(L):
    return [L.logits.clone(), L.topk_idx.clone(), L.topk_w.clone(), L.counts.clone(),
            L.offsets.clone(), L.row_src.clone(), L.tk_row.clone(), L.xp().clone(),
            L.H().clone(), L.A().clone(), L.O().clone(), L.y.clone()]


def _separate(inp):
    L = _layer(inp)
    L.route(inp["X"], inp["Wr"])
    L.permute(inp["X"])
    L.forward(inp["W1"], inp["W2"])
    torch.cuda.synchronize()
    return L


def _fused(inp, repeats=1):
    L = _layer(inp)
    outs = []
    for _ in range(repeats):
        L.forward_fused(inp["X"], inp["Wr"], inp["W1"], inp["W2"])
        torch.cuda.synchronize()
        assert L.device_status() == 0
        outs.append(_fwd_outputs(L))
    for o in outs[1:]:
        assert_bitwise_equal(outs[0], o)
    return L


CASES = {
    "tiny": dict(name="tiny"),
    "ragged": dict(name="tiny", T=300, E=16, k=3, d=512, I=256),
    "single_token": dict(name="tiny", T=1, E=4, k=2, d=256, I=128),
    "k_equals_E": dict(name="tiny", T=64, E=4, k=4, d=256, I=128),
    "stream_microbatch": dict(name="stream", T=2368, d=4096, E=512, k=10, I=1024, microbatches=1),
}


@pytest.mark.parametrize("case", list(CASES))
def test_fused_forward_equals_the_separate_calls(case):
    spec = dict(CASES[case])
    name = spec.pop("name")
    _announce(f"[fused] case={case} shape={spec} seed=0, three fused calls in a row")
    inp = workload.make_inputs(name, seed=0, device=DEV, **spec)
    if inp["X"].dim() == 3:
        inp = dict(inp, X=inp["X"][0], dY=inp["dY"][0])
    ref = _separate(inp)
    assert int(ref.counts.max().item()) < 256  # no 256-row block: the tiles are the same
    L = _fused(inp, repeats=3)
    assert_bitwise_equal(_fwd_outputs(ref), _fwd_outputs(L))
    # the backward that follows sees the same inputs, so it matches too
    for layer in (ref, L):
        layer.backward(inp["Wr"], inp["W1"], inp["W2"], inp["dY"])
    torch.cuda.synchronize()
    assert_bitwise_equal([ref.dx, ref.dw1, ref.dw2, ref.dwr, ref.d_topk_w],
                         [L.dx, L.dw1, L.dw2, L.dwr, L.d_topk_w])


def test_fused_forward_with_large_experts_matches_the_oracle():
    """Four experts for 1024 tokens x top-2: every expert has a full 256-row block, which the
    separate path runs on the 256 x 256 kernel. The fused forward runs them on 128 x 128 tiles;
    its outputs match the oracle, and the separate path's routing and H, A bit for bit."""
    _announce("[fused] T=1024 d=512 E=4 k=2 I=256: experts of 256 rows and more")
    inp = workload.make_inputs("tiny", seed=1, device=DEV, T=1024, E=4, k=2, d=512, I=256)
    ref = _separate(inp)
    assert int(ref.counts.max().item()) >= 256
    L = _fused(inp, repeats=2)
    a, b = _fwd_outputs(ref), _fwd_outputs(L)
    assert_bitwise_equal(a[:10], b[:10])  # routing, permutation, ring slot, H and A
    L.backward(inp["Wr"], inp["W1"], inp["W2"], inp["dY"])
    torch.cuda.synchronize()
    f, bk = run_oracle(inp)
    check_parity(L, inp, f, bk)


def test_fused_step_in_a_captured_graph_replays_exactly():
    """The fused forward and the backward captured once into a HIP graph: three replays, with
    eager work and synchronisations between them, each equal to the eager step bit for bit."""
    _announce("[fused] tiny step captured in a HIP graph, three replays")
    inp = workload.make_inputs("tiny", seed=2, device=DEV)
    X, Wr, W1, W2, dY = (inp[n] for n in ("X", "Wr", "W1", "W2", "dY"))
    L = _layer(inp)
    L.step(X, Wr, W1, W2, dY, fused=True)
    torch.cuda.synchronize()
    want = [t.clone() for t in (L.y, L.dx, L.dw1, L.dw2, L.dwr, L.d_topk_w)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        L.step(X, Wr, W1, W2, dY, fused=True)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            L.step(X, Wr, W1, W2, dY, fused=True)
    torch.cuda.synchronize()
    for _ in range(3):
        for t in (L.y, L.dx, L.dw1, L.dw2, L.dwr, L.d_topk_w):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert L.device_status() == 0
        assert_bitwise_equal(want, [L.y, L.dx, L.dw1, L.dw2, L.dwr, L.d_topk_w])
