"""moe_permute_static (no workspace, no allocation) against moe_permute, through the C ABI.

Two calls in a row share the library's fixed scratch: the second one is smaller and must not
see anything the first one left there. Then an MXFP8 and an MXFP4 call. Every output is
compared bit for bit with moe_permute's on the same inputs: counts, offsets, both permutation
maps, the ring slot's contents and the device status word.
"""
import numpy as np
import pytest
import torch

import workload
from tests._gpu import DEV, MoeLayer, _announce, m

pytestmark = pytest.mark.gpu


def _static_call(L, x, slot):
    T, k, E = L.T, L.k, L.E
    out = dict(counts=torch.full((E,), -7, dtype=torch.int32, device=DEV),
               offsets=torch.full((E + 1,), -7, dtype=torch.int32, device=DEV),
               row_src=torch.full((T * k,), -7, dtype=torch.int32, device=DEV),
               tk_row=torch.full((T * k,), -7, dtype=torch.int32, device=DEV),
               status=torch.full((1,), -7, dtype=torch.int32, device=DEV))
    ring = torch.full_like(L.ring, 0xA5)
    m.moe_permute_static(L.cfg, L.topk_idx, x, ring, slot, out["counts"], out["offsets"],
                         out["row_src"], out["tk_row"], out["status"])
    torch.cuda.synchronize()
    out["ring"] = ring
    return out


def _compare(L, x, slot=0):
    # bytes neither call writes (padding, a skipped row's position) then match too
    L.ring.fill_(0xA5)
    for n in ("counts", "offsets", "row_src", "tk_row"):
        getattr(L, n).fill_(-7)
    L.permute(x, slot=slot)
    torch.cuda.synchronize()
    got = _static_call(L, x, slot)
    for n in ("counts", "offsets", "row_src", "tk_row"):
        assert torch.equal(got[n], getattr(L, n)), n
    assert int(got["status"].item()) == L.device_status()
    lo, hi = slot * L.sizes.ring_slot, (slot + 1) * L.sizes.ring_slot
    assert torch.equal(got["ring"][lo:hi], L.ring[lo:hi])


def _layer(T, d, E, k, I, seed, precision=None, ring_slots=1):
    prec = m.MOE_PREC_BF16 if precision is None else precision
    L = MoeLayer(T, d, E, k, I, device=DEV, ring_slots=ring_slots, precision=prec)
    g = torch.Generator(device="cpu").manual_seed(seed)
    idx = torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]).to(torch.int32)
    L.set_routing(idx.to(DEV), torch.full((T, k), 1.0 / k, device=DEV))
    x = workload.make_inputs("tiny", seed=seed, device=DEV, T=T, d=d, E=E, k=k, I=I)["X"]
    return L, x


def test_static_permute_matches_moe_permute_on_two_calls_in_a_row():
    _announce("[no-alloc] T=2048 E=256 k=8 d=256, then T=100 E=16 k=3 d=512 (slot 1 of 2)")
    L, x = _layer(2048, 256, 256, 8, 128, seed=1)
    _compare(L, x)
    L2, x2 = _layer(100, 512, 16, 3, 128, seed=2, ring_slots=2)
    _compare(L2, x2, slot=1)


def test_static_permute_mx_modes_and_bad_index():
    _announce("[no-alloc] MXFP8 T=300 E=8 k=2 d=256; MXFP4 T=200 E=8 k=2 d=512; then a bad "
              "expert index")
    L, x = _layer(300, 256, 8, 2, 128, seed=3, precision=m.MOE_PREC_MXFP8)
    _compare(L, x)
    L4, x4 = _layer(200, 512, 8, 2, 256, seed=5, precision=m.MOE_PREC_MXFP4)
    _compare(L4, x4)
    L2, x2 = _layer(64, 256, 4, 1, 128, seed=4)
    idx = L2.topk_idx.clone()
    idx[10, 0] = 9
    L2.set_routing(idx, L2.topk_w)
    _compare(L2, x2)
    assert L2.device_status() == m.MOE_DEVICE_BAD_EXPERT_INDEX

