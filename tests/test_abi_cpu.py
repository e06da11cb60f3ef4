"""The C-ABI library loads without a GPU, exports every function include/moe.h declares, sizes
buffers and rejects bad arguments on the host before touching the device."""
import ctypes

import pytest

from tests._util import ensure_built

m = ensure_built()


def test_every_declared_function_is_exported():
    names = m.header_functions()
    assert set(names) >= {"moe_query", "moe_route", "moe_permute", "moe_forward",
                          "moe_backward", "moe_status_string"}
    L = m.lib()
    for n in names:
        assert hasattr(L, n), n


def test_query_sizes_follow_the_shapes():
    T, d, E, k, I = 2048, 7168, 256, 8, 2048
    s = m.moe_query(m.make_cfg(T, d, E, k, I))
    Tk = T * k
    assert s.ring_slot == Tk * d * 2
    assert s.saved >= Tk * (2 * I + I) * 2
    assert s.saved_A >= s.saved_H + Tk * 2 * I * 2
    assert s.workspace >= s.ws_dXp + Tk * d * 2
    for off in (s.saved_H, s.saved_A, s.ws_O, s.ws_dH, s.ws_dXp):
        assert off % 256 == 0
    # disjoint intermediates in the workspace
    spans = sorted([(s.ws_O, Tk * d * 2), (s.ws_dH, Tk * 2 * I * 2), (s.ws_dXp, Tk * d * 2)])
    for (a, n), (b, _) in zip(spans, spans[1:]):
        assert a + n <= b


@pytest.mark.parametrize("shape", [
    (0, 256, 8, 2, 128),      # no tokens
    (16, 200, 8, 2, 128),     # d not a multiple of 256
    (16, 256, 8, 2, 100),     # I not a multiple of 128
    (16, 256, 8, 9, 128),     # k > E
    (16, 256, 2000, 2, 128),  # E > 1024
    (16, 256, 128, 65, 128),  # k > 64
    (300000, 7168, 8, 1, 128),  # T * d >= 2^31 (32-bit row offsets)
    (600000, 256, 8, 1, 2048),  # T * 2I >= 2^31 (32-bit byte offsets into an expert's dH)
    (16, 65536, 8, 2, 65536),   # one expert's W1 bytes (4 I d) >= 2^31
    (16, 32768, 8, 2, 16384),   # 4 I d = 2^31 exactly
    (150000, 7168, 8, 2, 128),  # T*k*d >= 2^31 (all rows may go to one expert)
    (300000, 256, 8, 2, 2048),  # T*k*2I >= 2^31
])
def test_query_rejects_bad_shapes(shape):
    with pytest.raises(m.MoeError) as ei:
        m.moe_query(m.make_cfg(*shape))
    assert ei.value.status == -1


def test_query_accepts_the_largest_expert_weights_below_the_limit():
    # 4 I d = 2^31 - 2^22 < 2^31: accepted (host only; nothing is allocated or launched)
    s = m.moe_query(m.make_cfg(16, 32768 - 256, 8, 2, 16384 + 128))
    assert s.ring_slot > 0


def _fake(addr=1 << 20):
    return ctypes.c_void_p(addr)


def test_entry_points_reject_bad_arguments_before_launching():
    L = m.lib()
    cfg = m.make_cfg(64, 256, 8, 2, 128)
    s = m.moe_query(cfg)
    p = _fake()
    null = None
    # null pointer
    assert L.moe_route(ctypes.byref(cfg), null, p, p, p, p, p, s.workspace, None) == -1
    # misaligned bf16 matrix
    assert L.moe_route(ctypes.byref(cfg), _fake((1 << 20) + 2), p, p, p, p, p, s.workspace,
                       None) == -1
    assert L.moe_route(ctypes.byref(cfg), p, p, p, p, p, p, s.workspace - 1, None) == -5
    # ring too small for the slot, and negative slot
    assert L.moe_permute(ctypes.byref(cfg), p, p, p, s.ring_slot - 1, 0, p, p, p, p, p,
                         s.workspace, None) == -2
    assert L.moe_permute(ctypes.byref(cfg), p, p, p, 2 * s.ring_slot, 2, p, p, p, p, p,
                         s.workspace, None) == -2
    assert L.moe_permute(ctypes.byref(cfg), p, p, p, 2 * s.ring_slot, -1, p, p, p, p, p,
                         s.workspace, None) == -2
    # workspace too small
    assert L.moe_permute(ctypes.byref(cfg), p, p, p, s.ring_slot, 0, p, p, p, p, p,
                         s.workspace - 1, None) == -5
    assert L.moe_forward(ctypes.byref(cfg), p, s.ring_slot, 0, p, p, p, p, p, None, 0, p, p,
                         s.saved - 1, p, s.workspace, None) == -5
    # an unknown precision is not provided by the library
    cfgx = m.make_cfg(64, 256, 8, 2, 128, 3)
    assert L.moe_route(ctypes.byref(cfgx), p, p, p, p, p, p, s.workspace, None) == -3
    # MXFP8: the quantised weights are required, and sized
    cfg8 = m.make_cfg(64, 256, 8, 2, 128, m.MOE_PREC_MXFP8)
    s8 = m.moe_query(cfg8)
    assert L.moe_forward(ctypes.byref(cfg8), p, s8.ring_slot, 0, p, p, p, p, p, None, 0, p, p,
                         s8.saved, p, s8.workspace, None) == -1
    assert L.moe_forward(ctypes.byref(cfg8), p, s8.ring_slot, 0, p, p, p, p, p, p, s8.wq - 1, p,
                         p, s8.saved, p, s8.workspace, None) == -5
    assert L.moe_quantize_weights(ctypes.byref(cfg), p, p, p, 1 << 30, None) == -1
    assert L.moe_quantize_weights(ctypes.byref(cfg8), p, p, p, s8.wq - 1, None) == -5
    # unknown flag bits
    cfgf = m.make_cfg(64, 256, 8, 2, 128, 0, 8)
    assert L.moe_route(ctypes.byref(cfgf), p, p, p, p, p, p, s.workspace, None) == -1
    # backward: bad dwr when the router weight is given
    assert L.moe_backward(ctypes.byref(cfg), p, s.ring_slot, 0, p, p, p, p, p, p, p, p, None, 0,
                          p, s.saved, p, p, p, p, null, p, 0, p, s.workspace, None) == -1


def test_static_permute_checks_its_fixed_scratch_before_launching():
    L = m.lib()
    p = _fake()
    # 4 (nb E + nb + T k) bytes beyond the 4 MiB fixed scratch: refused on the host
    big = m.make_cfg(300000, 256, 1024, 4, 128)
    sb = m.moe_query(big)
    assert L.moe_permute_static(ctypes.byref(big), p, p, p, sb.ring_slot, 0, p, p, p, p, p,
                                None) == -5
    cfg = m.make_cfg(64, 256, 8, 2, 128)
    s = m.moe_query(cfg)
    # a null status word, and a ring too small for the slot
    assert L.moe_permute_static(ctypes.byref(cfg), p, p, p, s.ring_slot, 0, p, p, p, p, None,
                                None) == -1
    assert L.moe_permute_static(ctypes.byref(cfg), p, p, p, s.ring_slot, 1, p, p, p, p, p,
                                None) == -2
    assert m.MOE_STATIC_SCRATCH_BYTES == 4 << 20


def test_mxfp8_sizes():
    T, d, E, k, I = 2048, 7168, 256, 8, 2048
    s = m.moe_query(m.make_cfg(T, d, E, k, I, m.MOE_PREC_MXFP8))
    Tk = T * k
    up = lambda v: (v + 255) // 256 * 256
    assert s.ring_slot == up(Tk * d) + up(Tk * d // 32)
    wq = 2 * (up(E * 2 * I * d) + up(E * 2 * I * d // 32)) + 2 * (up(E * d * I) + up(E * d * I // 32))
    assert s.wq == wq
    assert m.moe_query(m.make_cfg(T, d, E, k, I)).wq == 0


def test_mxfp4_sizes_and_mode_checks():
    """MXFP4 codes take half a byte: the ring slot, the quantised weights and the quantised
    activations shrink accordingly; I must be a multiple of 256 and the MXFP8 wgrad flag is
    refused; the fused forward does not provide the mode."""
    T, d, E, k, I = 2048, 7168, 256, 8, 2048
    s4 = m.moe_query(m.make_cfg(T, d, E, k, I, m.MOE_PREC_MXFP4))
    s8 = m.moe_query(m.make_cfg(T, d, E, k, I, m.MOE_PREC_MXFP8))
    Tk = T * k
    up = lambda v: (v + 255) // 256 * 256
    assert s4.ring_slot == up(Tk * d // 2) + up(Tk * d // 32)
    wq = (2 * (up(E * 2 * I * d // 2) + up(E * 2 * I * d // 32)) +
          2 * (up(E * d * I // 2) + up(E * d * I // 32)))
    assert s4.wq == wq
    # dY, A and dH codes: half of MXFP8's
    assert s8.workspace - s4.workspace == up(T * d) - up(T * d // 2) + up(Tk * I) - \
        up(Tk * I // 2) + up(Tk * 2 * I) - up(Tk * 2 * I // 2)
    assert s4.saved == s8.saved
    for cfg in (m.make_cfg(64, 256, 8, 2, 128, m.MOE_PREC_MXFP4),
                m.make_cfg(64, 256, 8, 2, 256, m.MOE_PREC_MXFP4, m.MOE_FLAG_MXFP8_WGRAD)):
        with pytest.raises(m.MoeError) as ei:
            m.moe_query(cfg)
        assert ei.value.status == -1
    got = m.moe_query(m.make_cfg(300, 512, 16, 3, 256, m.MOE_PREC_MXFP4, m.MOE_FLAG_BF16_DW))
    base = m.moe_query(m.make_cfg(300, 512, 16, 3, 256, m.MOE_PREC_MXFP4))
    assert (got.ring_slot, got.workspace, got.wq) == (base.ring_slot, base.workspace, base.wq)
    L = m.lib()
    p = _fake()
    cfg4 = m.make_cfg(64, 256, 8, 2, 256, m.MOE_PREC_MXFP4)
    q = m.moe_query(cfg4)
    assert L.moe_forward_fused(ctypes.byref(cfg4), p, p, p, p, p, p, q.ring_slot, 0, p, p, p, p,
                               p, p, p, p, q.saved, p, q.workspace, None) == -3


def test_status_strings():
    assert m.status_string(0) == "ok"
    assert "ring" in m.status_string(-2)
    assert m.status_string(-99) == "unknown status"


@pytest.mark.skipif(__import__("torch").cuda.device_count() != 0,
                    reason="checks the no-device path; on a GPU host the call would launch")
def test_entry_points_report_a_missing_device_instead_of_launching():
    """With valid arguments an entry point reaches its device check; with no HIP device it
    returns MOE_ERR_HIP and enqueues nothing (on a non-gfx950 device: MOE_ERR_UNSUPPORTED)."""
    L = m.lib()
    cfg = m.make_cfg(64, 256, 8, 2, 128)
    s = m.moe_query(cfg)
    p = _fake()
    assert L.moe_route(ctypes.byref(cfg), p, p, p, p, p, p, s.workspace, None) == -4
    assert L.moe_permute(ctypes.byref(cfg), p, p, p, s.ring_slot, 0, p, p, p, p, p,
                         s.workspace, None) == -4


def test_fused_forward_checks_arguments_before_launching():
    L = m.lib()
    cfg = m.make_cfg(64, 256, 8, 2, 128)
    s = m.moe_query(cfg)
    p = _fake()
    args = lambda c, ring_bytes, slot, saved, ws: (ctypes.byref(c), p, p, p, p, p, p, ring_bytes,
                                                   slot, p, p, p, p, p, p, p, p, saved, p, ws, None)
    # MXFP8 mode is not provided by the single-launch forward
    cfg8 = m.make_cfg(64, 256, 8, 2, 128, m.MOE_PREC_MXFP8)
    s8 = m.moe_query(cfg8)
    assert L.moe_forward_fused(*args(cfg8, s8.ring_slot, 0, s8.saved, s8.workspace)) == -3
    assert L.moe_forward_fused(*args(cfg, s.ring_slot - 1, 0, s.saved, s.workspace)) == -2
    assert L.moe_forward_fused(*args(cfg, s.ring_slot, 0, s.saved - 1, s.workspace)) == -5
    assert L.moe_forward_fused(*args(cfg, s.ring_slot, 0, s.saved, s.workspace - 1)) == -5
    bad = list(args(cfg, s.ring_slot, 0, s.saved, s.workspace))
    bad[2] = None  # no router weight
    assert L.moe_forward_fused(*bad) == -1


def test_mxfp8_wgrad_flag_needs_mxfp8_mode_and_sizes_its_workspace():
    L = m.lib()
    p = _fake()
    bad = m.make_cfg(64, 256, 8, 2, 128, m.MOE_PREC_BF16, m.MOE_FLAG_MXFP8_WGRAD)
    with pytest.raises(m.MoeError) as ei:
        m.moe_query(bad)
    assert ei.value.status == -1
    assert L.moe_route(ctypes.byref(bad), p, p, p, p, p, p, 1 << 30, None) == -1
    plain = m.moe_query(m.make_cfg(2048, 7168, 256, 8, 2048, m.MOE_PREC_MXFP8))
    mxw = m.moe_query(m.make_cfg(2048, 7168, 256, 8, 2048, m.MOE_PREC_MXFP8,
                                 m.MOE_FLAG_MXFP8_WGRAD))
    P = (2048 * 8 + 256 * 127 + 127) // 128 * 128  # padded positions of all expert segments
    assert mxw.workspace - plain.workspace >= (2 * 4096 * P + 2 * 4096 * P // 32) // 2


def test_bf16_dw_flag_is_accepted_in_both_precisions_and_changes_no_size():
    for prec, extra in ((m.MOE_PREC_BF16, 0), (m.MOE_PREC_MXFP8, 0),
                        (m.MOE_PREC_MXFP8, m.MOE_FLAG_MXFP8_WGRAD)):
        base = m.moe_query(m.make_cfg(300, 512, 16, 3, 256, prec, extra))
        got = m.moe_query(m.make_cfg(300, 512, 16, 3, 256, prec, extra | m.MOE_FLAG_BF16_DW))
        for f in ("ring_slot", "saved", "workspace", "wq"):
            assert getattr(got, f) == getattr(base, f), (prec, extra, f)
    with pytest.raises(m.MoeError) as ei:
        m.moe_query(m.make_cfg(64, 256, 8, 2, 128, m.MOE_PREC_BF16, 8))  # an unknown flag bit
    assert ei.value.status == -1
