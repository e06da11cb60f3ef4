"""Seeded synthetic inputs for the MoE layer, shared by the oracle tests, the GPU tests and the bench.

This module only draws numbers and fixes shapes. It holds none of the layer's arithmetic:
no routing, no permutation and no expert math. The GPU path and the CPU oracle both consume
what it returns, and neither imports the other.

Six workloads are defined, named for what they are:

* ``tiny``: T=256 tokens, d=256, E=8 experts, top-2, SwiGLU intermediate 512.
* ``dsv3``: a DeepSeek-V3-shaped routed layer on one GPU. T=2048, d=7168, E=256, top-8,
  intermediate 2048.
* ``local_zipf``: the expert-parallel local slice of ``dsv3``. 16384 received rows, 8 local
  experts, d=7168, intermediate 2048, one expert per row. Rows follow a Zipf(1.2) expert
  popularity with three experts left empty, and each row carries a given gate weight.
* ``dsv3_mxfp8``: the ``dsv3`` shapes in MXFP8 mode.
* ``dsv3_mxfp4``: the ``dsv3`` shapes in MXFP4 mode.
* ``stream``: 8 microbatches of 2368 tokens through d=4096, E=512, top-10, intermediate 1024,
  sharing one 512 MiB ring buffer.

The values are: activations X ~ N(0, 1); router, gate/up and down weights ~ N(0, 0.02); the
upstream gradient dY ~ N(0, 1). All are rounded to bfloat16 (round to nearest even, by
torch's own cast). Each tensor has its own torch generator, seeded from (seed, workload,
tensor name), so a tensor does not depend on which other tensors were drawn. The values
depend on the device type, because torch's CPU and GPU generators differ, so a test always
hands the oracle host copies of the very tensors the GPU consumed.
"""
from __future__ import annotations

import hashlib

import numpy as np
import torch

WEIGHT_STD = 0.02

CONFIGS = {
    "tiny": dict(T=256, d=256, E=8, k=2, I=512, precision="bf16", routing="router"),
    "dsv3": dict(T=2048, d=7168, E=256, k=8, I=2048, precision="bf16", routing="router"),
    "local_zipf": dict(T=16384, d=7168, E=8, k=1, I=2048, precision="bf16", routing="zipf"),
    "dsv3_mxfp8": dict(T=2048, d=7168, E=256, k=8, I=2048, precision="mxfp8", routing="router"),
    "dsv3_mxfp4": dict(T=2048, d=7168, E=256, k=8, I=2048, precision="mxfp4", routing="router"),
    "stream": dict(T=2368, d=4096, E=512, k=10, I=1024, precision="bf16", routing="router",
                   microbatches=8, ring_bytes=512 * 1024 * 1024),
}

# Zipf(1.2) popularity for the local slice: three of the eight local experts receive nothing,
# and the other five take popularity ranks 1..5 in this id order.
ZIPF_S = 1.2
ZIPF_EMPTY = (0, 3, 7)
ZIPF_RANK_TO_EXPERT = (5, 2, 6, 1, 4)
ZIPF_GLOBAL_TOPK = 8


def config(name: str, **override) -> dict:
    cfg = dict(CONFIGS[name])
    cfg.update(override)
    cfg["name"] = name
    return cfg


def tensor_seed(seed: int, workload: str, tensor: str) -> int:
    """A 63-bit seed derived from (seed, workload, tensor) by SHA-256."""
    h = hashlib.sha256(f"{seed}/{workload}/{tensor}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _normal_bf16(shape, std, seed, device, chunk_dim0=False):
    """N(0, std) drawn in float32, scaled, then cast to bfloat16."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    if not chunk_dim0:
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        return (t * std).to(torch.bfloat16)
    out = torch.empty(shape, device=device, dtype=torch.bfloat16)
    for i in range(shape[0]):
        t = torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32)
        out[i] = (t * std).to(torch.bfloat16)
    return out


def zipf_routing(rows: int, seed: int, workload: str = "local_zipf"):
    """Expert id and gate weight for each received row of the local slice (one expert per row).

    Expert ids: three experts empty, the other five drawn i.i.d. with probability proportional
    to rank**-1.2. Gate weight: u0 / (u0 + ... + u7) with u ~ U(0,1)^8, i.e. this expert's share
    of a renormalised top-8 gate vector. Returns (idx int32 [rows, 1], w float32 [rows, 1]).
    """
    rng = np.random.default_rng(tensor_seed(seed, workload, "routing"))
    ranks = np.arange(1, len(ZIPF_RANK_TO_EXPERT) + 1, dtype=np.float64)
    p = ranks ** (-ZIPF_S)
    p /= p.sum()
    r = rng.choice(len(ranks), size=rows, p=p)
    idx = np.asarray(ZIPF_RANK_TO_EXPERT, dtype=np.int32)[r]
    u = rng.random((rows, ZIPF_GLOBAL_TOPK))
    w = (u[:, 0] / u.sum(axis=1)).astype(np.float32)
    return idx.reshape(rows, 1), w.reshape(rows, 1)


def make_inputs(name: str, seed: int = 0, device="cpu", **override) -> dict:
    """All inputs of one workload as torch tensors on `device`.

    Keys: X [T,d], W1 [E,2I,d] (gate rows 0..I-1, up rows I..2I-1), W2 [E,d,I], dY [T,d]
    (all bfloat16), plus Wr [E,d] bfloat16 when the layer routes for itself, or topk_idx
    [T,k] int32 and topk_w [T,k] float32 when routing is given. For ``stream`` X and dY gain a
    leading microbatch axis.
    """
    cfg = config(name, **override)
    T, d, E, k, I = cfg["T"], cfg["d"], cfg["E"], cfg["k"], cfg["I"]
    mb = cfg.get("microbatches")
    dev = torch.device(device)
    big = E * 2 * I * d > (1 << 26)
    s = lambda t: tensor_seed(seed, name, t)
    out = {"cfg": cfg}
    xshape = (mb, T, d) if mb else (T, d)
    out["X"] = _normal_bf16(xshape, 1.0, s("X"), dev)
    out["W1"] = _normal_bf16((E, 2 * I, d), WEIGHT_STD, s("W1"), dev, chunk_dim0=big)
    out["W2"] = _normal_bf16((E, d, I), WEIGHT_STD, s("W2"), dev, chunk_dim0=big)
    out["dY"] = _normal_bf16(xshape, 1.0, s("dY"), dev)
    if cfg["routing"] == "router":
        out["Wr"] = _normal_bf16((E, d), WEIGHT_STD, s("Wr"), dev)
    else:
        idx, w = zipf_routing(T, seed, name)
        out["topk_idx"] = torch.from_numpy(idx).to(dev)
        out["topk_w"] = torch.from_numpy(w).to(dev)
    return out


def to_numpy(t: torch.Tensor) -> np.ndarray:
    """Host copy of a tensor; bfloat16 is widened to float32 (exact)."""
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


class HostExperts:
    """Per-expert host view of a device weight tensor [E, ...]. Indexing copies one expert's
    block to the host (float32), so a CPU consumer can walk the experts without holding the
    whole tensor in host memory."""

    def __init__(self, t: torch.Tensor):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, e):
        return to_numpy(self.t[e])

    def __len__(self):
        return self.shape[0]
