"""The seeded input generator: reproducible, correctly shaped, with the stated distributions."""
import numpy as np
import torch

import workload


def test_inputs_reproducible_and_shaped():
    a = workload.make_inputs("tiny", seed=0)
    b = workload.make_inputs("tiny", seed=0)
    c = workload.make_inputs("tiny", seed=1)
    for key in ("X", "Wr", "W1", "W2", "dY"):
        assert a[key].dtype == torch.bfloat16
        assert torch.equal(a[key], b[key])
        assert not torch.equal(a[key], c[key])
    assert a["X"].shape == (256, 256)
    assert a["W1"].shape == (8, 1024, 256)
    assert a["W2"].shape == (8, 256, 512)
    assert a["Wr"].shape == (8, 256)
    assert abs(a["X"].float().std().item() - 1.0) < 0.02
    assert abs(a["W1"].float().std().item() - 0.02) < 0.001


def test_zipf_routing_matches_its_description():
    idx, w = workload.zipf_routing(16384, seed=0)
    assert idx.shape == (16384, 1) and w.shape == (16384, 1)
    counts = np.bincount(idx[:, 0], minlength=8)
    assert all(counts[e] == 0 for e in workload.ZIPF_EMPTY)
    assert counts.max() > 0.40 * 16384
    assert counts.argmax() == workload.ZIPF_RANK_TO_EXPERT[0]
    assert np.all((w > 0) & (w < 1))
    assert abs(w.mean() - 1 / 8) < 0.01


def test_stream_inputs_have_microbatch_axis():
    a = workload.make_inputs("stream", seed=0, T=16, d=64, E=8, k=2, I=32)
    assert a["X"].shape == (8, 16, 64)
    assert a["dY"].shape == (8, 16, 64)
