"""Bitwise determinism across processes: a fresh process, whose buffers sit elsewhere in device
memory (it first takes a 3 GiB spacer allocation), must produce every output of one layer step
bit for bit as this process does, in BF16, MXFP8 and MXFP4, on one-shot and persistent grids,
and at the full sizes: the DeepSeek-V3-shaped layer in all three precisions, the expert slice
and the streaming macrobatch's whole ring walk.

Every output element has one producer and a fixed summation order, so neither buffer placement
nor launch timing may change a bit. The comparison is between two runs of the same library; no
expected value is stored.
"""
import hashlib
import json
import os
import subprocess
import sys

import pytest
import torch

import workload
from tests._gpu import DEV, _announce, outputs, run_gpu
from tests.test_gpu_sizes_full import _stream_run

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (label, workload, shape overrides, options of the layer)
CASES = [
    ("ragged_bf16", "tiny", dict(T=300, E=16, k=3, d=512, I=256), {}),
    ("ragged_mxfp8", "tiny", dict(T=300, E=16, k=3, d=512, I=256, precision="mxfp8"), {}),
    ("ragged_mxfp4", "tiny", dict(T=300, E=16, k=3, d=512, I=256, precision="mxfp4"), {}),
    ("zipf_bf16_persistent", "local_zipf", dict(T=2048, d=256, I=256), dict(persistent=True)),
    ("zipf_mxfp8_wgrad", "local_zipf", dict(T=2048, d=256, I=256, precision="mxfp8",
                                             mx_wgrad=True), {}),
    ("multi_mtile_bf16_dw", "tiny", dict(T=1024, E=4, k=2, d=512, I=256), dict(bf16_dw=True)),
    # the DeepSeek-V3-shaped layer: 2048 tokens, d 7168, 256 experts, top-8, I 2048
    ("dsv3_bf16", "dsv3", {}, {}),
    ("dsv3_mxfp8", "dsv3_mxfp8", {}, {}),
    ("dsv3_mxfp4", "dsv3_mxfp4", {}, {}),
    # one device's expert slice: 16384 rows over 8 experts of d 7168, I 2048, Zipf-skewed
    ("local_zipf_bf16", "local_zipf", {}, {}),
]


def _fingerprint(t):
    """An exact integer fingerprint of a large tensor's bits, on the device: its 16-bit words
    weighted by position (mod 65521, plus one) and summed in int64, 2^26 words per chunk. Each
    product is below 2^31 and each chunk's sum below 2^57, so nothing overflows and the value
    does not depend on the order of the sum."""
    v = t.contiguous().view(-1).view(torch.int16)
    acc, step = 0, 1 << 26
    for i in range(0, v.numel(), step):
        c = v[i:i + step].long()
        w = torch.arange(i, i + c.numel(), device=c.device, dtype=torch.long) % 65521 + 1
        acc += int((c * w).sum())
    return acc


def _digest(tensors):
    h = hashlib.sha1()
    for t in tensors:
        t = t.contiguous()
        if t.dtype == torch.bool:
            t = t.to(torch.uint8)
        h.update(str((t.dtype, tuple(t.shape))).encode())
        if t.numel() * t.element_size() >= (1 << 28) and t.element_size() >= 2:
            h.update(str(_fingerprint(t)).encode())
        else:
            h.update(t.view(torch.uint8).cpu().numpy().tobytes())
    return h.hexdigest()


def digests():
    out = {}
    for label, name, spec, opts in CASES:
        inp = workload.make_inputs(name, seed=7, device=DEV, **spec)
        L = run_gpu(inp, **opts)
        out[label] = _digest(outputs(L, "Wr" in inp, clone=False))
        del L, inp
        torch.cuda.empty_cache()
    # the streaming macrobatch: 8 microbatches of 2368 tokens through a 2-slot ring, forward
    # 0..7, then backward 7..0 with replays and the weight gradients accumulated
    inp = workload.make_inputs("stream", seed=7, device=DEV)
    L, routing, ys, dxs, dtws = _stream_run(inp)
    flat = [t for r in routing for t in r] + ys + dxs + dtws + [L.dw1, L.dw2, L.dwr]
    out["stream_ring_walk"] = _digest(flat)
    del L, inp, routing, ys, dxs, dtws, flat
    torch.cuda.empty_cache()
    return out


def child_main():
    """Entry of the second process: take a spacer allocation first, then print the digests."""
    spacer = torch.empty(3 << 30, dtype=torch.uint8, device=DEV)
    spacer.fill_(1)
    torch.cuda.synchronize()
    print("DIGESTS " + json.dumps(digests()), flush=True)


def test_outputs_are_bitwise_identical_across_processes():
    _announce("[processes] " + ", ".join(c[0] for c in CASES) + ", stream_ring_walk")
    here = digests()
    assert len(set(here.values())) == len(CASES) + 1
    code = "import tests.test_gpu_processes as t; t.child_main()"
    r = subprocess.run([sys.executable, "-u", "-c", code], cwd=ROOT, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    line = [s for s in r.stdout.splitlines() if s.startswith("DIGESTS ")]
    assert line, r.stdout[-2000:]
    there = json.loads(line[-1][len("DIGESTS "):])
    assert there == here
