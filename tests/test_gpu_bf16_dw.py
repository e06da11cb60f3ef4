"""bf16 weight gradients (MOE_FLAG_BF16_DW) through the C ABI.

dW1 and dW2 are the same fp32 sums as in the default mode, rounded once to bf16 where they are
stored. So, on the same inputs:
* every other output equals the fp32-dW run's bit for bit, and dW1, dW2 equal that run's fp32
  values cast to bf16 (round to nearest even) bit for bit;
* with accumulate, they equal the stored bf16 value plus the new fp32 sums, rounded once;
* dW1, dW2 are within the layer's gradient tolerance of the oracle's bf16-stored gradients.
The cases cover the task-table wgrad kernel (bf16 and MXFP8 right operands), the 256 x 256
big-expert kernel, the MXFP8 wgrad kernel, MXFP4 mode and empty experts (zero blocks).
"""
import numpy as np
import pytest
import torch

import workload
from tests._gpu import (DEV, _announce, _np, assert_bitwise_equal, check_parity, outputs,
                        run_gpu, run_oracle)

pytestmark = pytest.mark.gpu


def _inputs(case):
    if case == "tiny":
        return workload.make_inputs("tiny", seed=0, device=DEV)
    if case == "zipf_local":  # experts of 512 rows and more, and empty experts
        return workload.make_inputs("local_zipf", seed=0, device=DEV, T=2048, d=256, I=256)
    if case == "large":  # the 256 x 256 wgrad kernel over several K steps and tiles
        counts = [2500, 1000, 596, 0]
        T, E = sum(counts), len(counts)
        inp = workload.make_inputs("local_zipf", seed=11, device=DEV, T=T, d=1024, E=E, I=512)
        idx = np.repeat(np.arange(E, dtype=np.int32), counts)
        np.random.default_rng(11).shuffle(idx)
        inp["topk_idx"] = torch.from_numpy(idx.reshape(T, 1)).to(DEV)
        return inp
    if case == "mxfp8_tiny":
        return workload.make_inputs("tiny", seed=0, device=DEV, precision="mxfp8")
    if case == "mxfp8_zipf_local":
        return workload.make_inputs("local_zipf", seed=0, device=DEV, T=2048, d=256, I=256,
                                    precision="mxfp8")
    if case == "mxfp4_zipf_local":
        return workload.make_inputs("local_zipf", seed=0, device=DEV, T=2048, d=256, I=256,
                                    precision="mxfp4")
    if case == "mxfp8_wgrad_zipf_local":
        return workload.make_inputs("local_zipf", seed=0, device=DEV, T=2048, d=256, I=256,
                                    precision="mxfp8", mx_wgrad=True)
    raise KeyError(case)


CASES = ["tiny", "zipf_local", "large", "mxfp8_tiny", "mxfp8_zipf_local", "mxfp8_wgrad_zipf_local",
         "mxfp4_zipf_local"]


def _backward_again(L, inp, dy, accumulate):
    L.backward(inp.get("Wr"), inp["W1"], inp["W2"], dy, accumulate=accumulate)
    torch.cuda.synchronize()


@pytest.mark.parametrize("case", CASES)
def test_bf16_dw_is_the_fp32_sum_rounded_once(case):
    _announce(f"[bf16 dW] case={case}: against the fp32-dW run, then accumulate")
    inp = _inputs(case)
    routed = "Wr" in inp
    Lf = run_gpu(inp)
    Lb = run_gpu(inp, bf16_dw=True)
    assert Lb.dw1.dtype == torch.bfloat16 and Lb.dw2.dtype == torch.bfloat16
    a, b = outputs(Lf, routed), outputs(Lb, routed)
    # every output but dW1 and dW2 is the same; those are the fp32 values rounded once
    keep = [i for i, t in enumerate(outputs(Lf, routed, clone=False))
            if t.data_ptr() not in (Lf.dw1.data_ptr(), Lf.dw2.data_ptr())]
    assert len(keep) == len(a) - 2
    assert_bitwise_equal([a[i] for i in keep], [b[i] for i in keep])
    for g32, g16 in ((Lf.dw1, Lb.dw1), (Lf.dw2, Lb.dw2)):
        assert torch.equal(g32.to(torch.bfloat16).view(torch.int16), g16.view(torch.int16))
    counts = _np(Lb.counts)
    for e in np.flatnonzero(counts == 0):
        assert torch.count_nonzero(Lb.dw1[e]) == 0 and torch.count_nonzero(Lb.dw2[e]) == 0
    # accumulate: a second batch's gradients added in fp32 to the stored bf16 values
    dy2 = (inp["dY"].float() * -0.5).to(torch.bfloat16)
    first = [Lb.dw1.clone(), Lb.dw2.clone()]
    _backward_again(Lf, inp, dy2, accumulate=False)
    _backward_again(Lb, inp, dy2, accumulate=True)
    for g0, s2, g in zip(first, (Lf.dw1, Lf.dw2), (Lb.dw1, Lb.dw2)):
        want = (g0.float() + s2).to(torch.bfloat16)
        assert torch.equal(want.view(torch.int16), g.view(torch.int16))


@pytest.mark.parametrize("case", ["tiny", "zipf_local", "mxfp8_wgrad_zipf_local",
                                  "mxfp4_zipf_local"])
def test_bf16_dw_matches_the_oracle(case):
    _announce(f"[bf16 dW] case={case}: against the oracle with bf16-stored weight gradients")
    inp = _inputs(case)
    L = run_gpu(inp, bf16_dw=True)
    f, b = run_oracle(inp, dw_dtype="bf16")
    # the MX modes are held to their bar, 6e-2 against the quantisation-emulating oracle
    tol = dict(tol_act=6e-2, tol_grad=6e-2) if inp["cfg"].get("precision") != "bf16" else {}
    check_parity(L, inp, f, b, **tol)
