"""Buffer plumbing around the C ABI: allocates the caller-owned device buffers with torch and
calls the entry points in order. It holds no layer arithmetic. Every step runs in the
library's kernels, and torch only provides memory and the stream.
"""
from __future__ import annotations

import torch

from . import (MOE_FLAG_PERSISTENT, MOE_PREC_BF16, MOE_PREC_MXFP8, make_cfg, moe_backward,
               moe_forward, moe_permute, moe_query, moe_quantize_weights, moe_route)


class MoeLayer:
    """Caller-owned buffers for one (T, d, E, k, I) shape on one device.

    ``ring_slots`` slots of T*k permuted rows make up the ring. Forward writes slot ``slot``,
    and backward reads the slot its batch was permuted into. With ``precision=MOE_PREC_MXFP8``
    the layer also owns the quantised-weight buffer ``wq``; ``quantize_weights`` fills it.
    """

    def __init__(self, T, d, E, k, I, device="cuda", ring_slots=1, persistent=False,
                 precision=MOE_PREC_BF16):
        self.T, self.d, self.E, self.k, self.I = T, d, E, k, I
        self.cfg = make_cfg(T, d, E, k, I, precision, MOE_FLAG_PERSISTENT if persistent else 0)
        s = moe_query(self.cfg)
        self.sizes = s
        dev = torch.device(device)
        u8, i32, f32, bf = torch.uint8, torch.int32, torch.float32, torch.bfloat16
        Tk = T * k
        self.ring = torch.empty(s.ring_slot * ring_slots, dtype=u8, device=dev)
        self.workspace = torch.empty(s.workspace, dtype=u8, device=dev)
        self.saved = torch.empty(s.saved, dtype=u8, device=dev)
        self.logits = torch.empty(T, E, dtype=f32, device=dev)
        self.topk_idx = torch.empty(T, k, dtype=i32, device=dev)
        self.topk_w = torch.empty(T, k, dtype=f32, device=dev)
        self.counts = torch.empty(E, dtype=i32, device=dev)
        self.offsets = torch.empty(E + 1, dtype=i32, device=dev)
        self.row_src = torch.empty(Tk, dtype=i32, device=dev)
        self.tk_row = torch.empty(Tk, dtype=i32, device=dev)
        self.y = torch.empty(T, d, dtype=bf, device=dev)
        self.dx = torch.empty(T, d, dtype=bf, device=dev)
        self.d_topk_w = torch.empty(T, k, dtype=f32, device=dev)
        self.dw1 = torch.zeros(E, 2 * I, d, dtype=f32, device=dev)
        self.dw2 = torch.zeros(E, d, I, dtype=f32, device=dev)
        self.dwr = torch.zeros(E, d, dtype=f32, device=dev)
        self.mx = precision == MOE_PREC_MXFP8
        self.wq = torch.empty(s.wq, dtype=u8, device=dev) if self.mx else None

    # views of intermediates -----------------------------------------------------------------
    def _view(self, buf, off, rows, cols):
        n = rows * cols * 2
        return buf[off:off + n].view(torch.bfloat16).view(rows, cols)

    def xp(self, slot=0):
        """The slot's bf16 Xp (BF16 mode), or (E4M3 codes [T*k, d], scale codes [T*k, d/32]) as
        uint8 tensors (MXFP8 mode)."""
        base = slot * self.sizes.ring_slot
        if not self.mx:
            return self._view(self.ring, base, self.T * self.k, self.d)
        Tk, d = self.T * self.k, self.d
        codes = self.ring[base:base + Tk * d].view(Tk, d)
        sc0 = base + (Tk * d + 255) // 256 * 256
        return codes, self.ring[sc0:sc0 + Tk * d // 32].view(Tk, d // 32)

    def H(self):
        return self._view(self.saved, self.sizes.saved_H, self.T * self.k, 2 * self.I)

    def A(self):
        return self._view(self.saved, self.sizes.saved_A, self.T * self.k, self.I)

    def O(self):
        return self._view(self.workspace, self.sizes.ws_O, self.T * self.k, self.d)

    def dH(self):
        return self._view(self.workspace, self.sizes.ws_dH, self.T * self.k, 2 * self.I)

    def dXp(self):
        return self._view(self.workspace, self.sizes.ws_dXp, self.T * self.k, self.d)

    def device_status(self):
        return int(self.workspace[:4].view(torch.int32).item())

    # steps ----------------------------------------------------------------------------------
    def route(self, x, w_router, stream=None):
        moe_route(self.cfg, x, w_router, self.logits, self.topk_idx, self.topk_w, self.workspace,
                  stream)

    def set_routing(self, topk_idx, topk_w):
        self.topk_idx.copy_(topk_idx)
        self.topk_w.copy_(topk_w)

    def permute(self, x, slot=0, stream=None):
        moe_permute(self.cfg, self.topk_idx, x, self.ring, slot, self.counts, self.offsets,
                    self.row_src, self.tk_row, self.workspace, stream)

    def quantize_weights(self, w1, w2, stream=None):
        moe_quantize_weights(self.cfg, w1, w2, self.wq, stream)

    def forward(self, w1, w2, slot=0, saved=None, stream=None):
        moe_forward(self.cfg, self.ring, slot, self.offsets, self.tk_row, self.topk_w, w1, w2,
                    self.wq, self.y, self.saved if saved is None else saved, self.workspace,
                    stream)

    def backward(self, w_router, w1, w2, dy, slot=0, accumulate=False, saved=None, stream=None):
        moe_backward(self.cfg, self.ring, slot, self.offsets, self.row_src, self.tk_row,
                     self.topk_idx, self.topk_w, w_router, w1, w2, self.wq,
                     self.saved if saved is None else saved, dy, self.dx, self.dw1, self.dw2,
                     self.dwr if w_router is not None else None, self.d_topk_w, accumulate,
                     self.workspace, stream)

    def step(self, x, w_router, w1, w2, dy, slot=0, stream=None):
        """One fwd+bwd pass: route (when w_router is given), permute, forward, backward."""
        if w_router is not None:
            self.route(x, w_router, stream)
        self.permute(x, slot, stream)
        self.forward(w1, w2, slot, stream=stream)
        self.backward(w_router, w1, w2, dy, slot, stream=stream)
