"""Oracle for the deterministic MoE layer. Test infrastructure only.

This is a plain, slow, CPU-only numpy implementation of what the layer computes. Its only
callers are the test suite, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of
``bench.py``. The GPU library never imports or calls it, and it shares no code with the GPU
library.

The pages describe Mixture-of-Kittens (MoK), a deterministic MoE training megakernel. They name
the layer's steps but never write out its math. The page "Cursor Open-Sources Mixture-of-Kittens
(MoK): A Deterministic MoE Training Megakernel for GB300 NVL72 Racks" (MarkTechPost copy on
ncijnetwork.com) names these steps:

* expert-grouped GEMMs, in section "Three design decisions that matter";
* a SwiGLU backward with the router-weight gradient fused into it, in the closing paragraph of
  that section;
* a ring token buffer that drops no tokens, in the same section and under "Key Takeaways";
* full determinism, in the introduction.

The page "Mixture-of-Kittens: Cursor's Open-Source Kernel Trains AI Up to 2.37x Faster"
(toknow.ai), in its summary, describes an MoE as routing each input to a few experts. Where the
pages are silent, the oracle takes the plainest reading, listed in ``readings`` below.

Numerics: everything is float64, except the router logits. The logits decide integers (which
experts a token visits), so both sides compute them in float32, in one stated order. In
``storage="bf16"`` mode the oracle rounds to bfloat16 at the same storage points as the GPU
path, and downstream steps use the rounded values. ``storage="exact"`` skips that rounding and
gives the mathematical reference.

MXFP8 mode (``precision="mxfp8"``) applies OCP MXFP8 quantisation (``oracle/mx.py``) to the
operands of the forward and dgrad expert GEMMs, along each GEMM's reduction axis.

Pins: tests/test_oracle_*.py check this module against things other than itself:
* brute force over all k-subsets;
* a dense evaluation of every token through every expert, masked;
* central finite differences;
* torch autograd on an independent dense formulation;
* closed forms, special cases and invariants;
* a hand-worked fp32 summation-order example in tests/golden/;
* for MXFP8: torch's float8_e4m3fn decode and cast, brute-force rounding, exact power-of-two
  scale bounds, and quantisation-axis checks on inputs that are exact in MXFP8.
"""
from . import mx  # noqa: F401
from .moe import (  # noqa: F401
    bf16_round,
    router_logits_fp32,
    route_topk,
    permute,
    forward,
    backward,
    layer,
    expert_forward,
    expert_backward,
    gather_sum,
    router_backward,
    readings,
)
