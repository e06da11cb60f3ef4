"""Pins of the oracle's MXFP8 quantisation and of its MXFP8 layer mode.

* E4M3 decode: all 256 codes against torch's float8_e4m3fn, an independent library.
* E4M3 encode: against torch's cast (round to nearest even) for in-range values, including
  exact ties and subnormals, and against brute force over the 127 finite magnitudes; saturation
  to 448.
* E8M0 scale: the scaled block maximum lies in [256, 512), checked with exact power-of-two
  bounds; all-zero blocks; blocks are independent.
* The MX GEMM: qdq(A) qdq(B)^T equals the float64 product of operands dequantised through torch.
* Quantisation axes of the layer: inputs built to be exact in MXFP8 along the axis the mode
  reading names leave the forward H and the backward dH unchanged between MXFP8 and BF16 modes.
  A wrong axis, or a transposed operand, would change them.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import mx


def _torch_e4m3_to_f64(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8).copy())
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_encode(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = mx.e4m3_value(codes)
    ref = _torch_e4m3_to_f64(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.isnan(ours).sum() == 2  # 0x7F and 0xFF
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])
    assert np.nanmax(ours) == 448.0 and mx.e4m3_value(1) == 2.0 ** -9


def test_e4m3_encode_matches_torch_rne_including_ties_and_subnormals():
    rng = np.random.default_rng(0)
    pos = mx.e4m3_value(np.arange(127))  # the non-negative finite values, ascending
    mids = (pos[:-1] + pos[1:]) / 2  # exact ties, representable in float32
    vals = np.concatenate([
        rng.uniform(-448, 448, 20000), rng.uniform(-2 ** -6, 2 ** -6, 5000),
        mids, -mids, pos, -pos[1:], rng.uniform(-1, 1, 5000) * 2.0 ** rng.integers(-12, 8, 5000),
    ]).astype(np.float32).astype(np.float64)
    ours = mx.e4m3_encode(vals)
    ref = _torch_encode(vals)
    # compare values (torch and this oracle may differ only in the sign of a zero)
    np.testing.assert_array_equal(mx.e4m3_value(ours), _torch_e4m3_to_f64(ref))


def test_e4m3_encode_brute_force_nearest_even():
    rng = np.random.default_rng(1)
    pos = mx.e4m3_value(np.arange(127))  # the non-negative finite values, ascending
    vals = np.concatenate([rng.uniform(0, 450, 3000), (pos[:-1] + pos[1:]) / 2])
    got = mx.e4m3_encode(vals)
    for v, c in zip(vals, got):
        a = min(v, 448.0)
        dist = np.abs(pos - a)
        best = np.flatnonzero(dist == dist.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert c == want, (v, c, want)


def test_e4m3_encode_saturates_to_448():
    v = np.array([448.0, 449.0, 479.9, 480.0, 1e6, -500.0, -1e30])
    got = mx.e4m3_encode(v)
    np.testing.assert_array_equal(got, [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE])


def test_every_value_times_every_scale_round_trips():
    codes = np.arange(127, dtype=np.uint8)
    for s in (100, 127, 140):
        blk = np.tile(codes, 2)[:96].astype(np.uint8)
        blk[0] = 0x7E  # a block maximum in [256, 448] fixes the scale at s
        blk[32] = 0x78
        blk[64] = 0x7A
        sc = np.full(3, s, np.uint8)
        x = mx.dequantize(blk, sc)
        q, sc2 = mx.quantize(x)
        np.testing.assert_array_equal(sc2, sc)
        np.testing.assert_array_equal(mx.e4m3_value(q), mx.e4m3_value(blk))


def test_scale_puts_block_max_in_256_to_512_and_zero_blocks_get_code_0():
    rng = np.random.default_rng(2)
    amax = np.concatenate([2.0 ** rng.uniform(-100, 100, 5000), 2.0 ** np.arange(-100, 101)])
    code = mx.e8m0_code(amax).astype(np.float64)
    scaled = amax / 2.0 ** (code - 127)
    assert np.all((scaled >= 256) & (scaled < 512))
    assert mx.e8m0_code(0.0) == 0
    assert mx.e8m0_code(448.0) == 127 and mx.e8m0_code(1.0) == 119
    assert mx.e8m0_code(2.0 ** 200) == 254 and mx.e8m0_code(2.0 ** -200) == 0


def test_blocks_are_independent_and_error_is_bounded():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((8, 128)) * 2.0 ** rng.integers(-6, 6, (8, 1))
    q, sc = mx.quantize(x)
    y = x.copy()
    y[:, 32:64] *= 1000.0
    q2, sc2 = mx.quantize(y)
    keep = np.r_[0:32, 64:128]
    np.testing.assert_array_equal(q[:, keep], q2[:, keep])
    np.testing.assert_array_equal(sc[:, [0, 2, 3]], sc2[:, [0, 2, 3]])
    d = mx.dequantize(q, sc)
    scale = np.repeat(2.0 ** (sc.astype(np.float64) - 127), 32, axis=1)
    # half an ulp of E4M3 (2^-4 relative for normals, 2^-10 absolute in scaled units below)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, scale * 2.0 ** -10)
    sat = np.abs(x) / scale > 448
    assert np.all((np.abs(d - x) <= bound) | sat)
    assert np.all(np.abs(d[sat]) == 448 * scale[sat])


def test_mx_gemm_equals_float64_product_of_torch_dequantised_operands():
    rng = np.random.default_rng(4)
    A = rng.standard_normal((24, 128))
    B = rng.standard_normal((40, 128)) * 0.02
    qa, sa = mx.quantize(A)
    qb, sb = mx.quantize(B)
    ta = _torch_e4m3_to_f64(qa) * np.repeat(2.0 ** (sa.astype(np.float64) - 127), 32, axis=1)
    tb = _torch_e4m3_to_f64(qb) * np.repeat(2.0 ** (sb.astype(np.float64) - 127), 32, axis=1)
    np.testing.assert_array_equal(mx.qdq(A) @ mx.qdq(B).T, ta @ tb.T)


def _mx_exact(shape, rng, scale_lo=110, scale_hi=125):
    """Values exactly representable in MXFP8 along the last axis: random finite codes with one
    block maximum in [256, 448] per block, times a random scale per block."""
    *lead, n = shape
    codes = rng.integers(0, 127, size=shape).astype(np.uint8)
    codes |= (rng.integers(0, 2, size=shape) << 7).astype(np.uint8)
    codes[..., ::32] = rng.integers(0x78, 0x7F, size=(*lead, n // 32)).astype(np.uint8)
    sc = rng.integers(scale_lo, scale_hi, size=(*lead, n // 32)).astype(np.uint8)
    x = mx.dequantize(codes, sc)
    assert np.array_equal(mx.qdq(x), x)
    assert np.array_equal(oracle.bf16_round(x), x)
    return x


def test_forward_quantises_x_and_w1_along_d():
    rng = np.random.default_rng(5)
    T, d, E, k, I = 24, 64, 4, 2, 32
    X = _mx_exact((T, d), rng, 118, 126)
    W1 = _mx_exact((E, 2 * I, d), rng, 108, 114)
    W2 = oracle.bf16_round(rng.standard_normal((E, d, I)) * 0.05)
    Wr = oracle.bf16_round(rng.standard_normal((E, d)) * 0.1)
    fb = oracle.forward(X, W1, W2, Wr=Wr, k=k)
    fm = oracle.forward(X, W1, W2, Wr=Wr, k=k, precision="mxfp8")
    np.testing.assert_array_equal(fm["H"], fb["H"])
    np.testing.assert_array_equal(fm["A"], fb["A"])
    assert not np.array_equal(fm["O"], fb["O"])  # A is not MX-exact, so GEMM2 does quantise
    # the same W1 made exact along 2I instead of d no longer leaves H unchanged
    W1t = np.swapaxes(_mx_exact((E, d, 2 * I), rng, 108, 114), 1, 2).copy()
    fb2 = oracle.forward(X, W1t, W2, Wr=Wr, k=k)
    fm2 = oracle.forward(X, W1t, W2, Wr=Wr, k=k, precision="mxfp8")
    assert not np.array_equal(fm2["H"], fb2["H"])


def test_backward_quantises_dy_and_w2_along_d():
    rng = np.random.default_rng(6)
    T, d, E, k, I = 24, 64, 4, 2, 32
    X = oracle.bf16_round(rng.standard_normal((T, d)))
    W1 = oracle.bf16_round(rng.standard_normal((E, 2 * I, d)) * 0.1)
    W2 = np.swapaxes(_mx_exact((E, I, d), rng, 108, 114), 1, 2).copy()  # exact along d
    dY = _mx_exact((T, d), rng, 118, 126)
    Wr = oracle.bf16_round(rng.standard_normal((E, d)) * 0.1)
    fb = oracle.forward(X, W1, W2, Wr=Wr, k=k)
    fm = oracle.forward(X, W1, W2, Wr=Wr, k=k, precision="mxfp8")
    fm_h = dict(fm, H=fb["H"], A=fb["A"])  # isolate the backward: same saved H and A
    bb = oracle.backward(fb, X, W1, W2, dY, Wr=Wr)
    bm = oracle.backward(fm_h, X, W1, W2, dY, Wr=Wr)
    np.testing.assert_array_equal(bm["dH"], bb["dH"])
    # and the fused router-weight gradient equals <dY, A W2^T> in exact arithmetic
    np.testing.assert_allclose(bm["dw"], bb["dw"], rtol=1e-2, atol=1e-3)
    # W2 exact along I instead: dgrad requantisation changes dH
    W2i = _mx_exact((E, d, I), rng, 108, 114)
    bb2 = oracle.backward(oracle.forward(X, W1, W2i, Wr=Wr, k=k), X, W1, W2i, dY, Wr=Wr)
    fm2 = oracle.forward(X, W1, W2i, Wr=Wr, k=k, precision="mxfp8")
    f2 = oracle.forward(X, W1, W2i, Wr=Wr, k=k)
    bm2 = oracle.backward(dict(fm2, H=f2["H"], A=f2["A"]), X, W1, W2i, dY, Wr=Wr)
    assert not np.array_equal(bm2["dH"], bb2["dH"])


@pytest.mark.parametrize("seed", [7, 8])
def test_mxfp8_layer_stays_within_its_error_bound_of_the_exact_layer(seed):
    rng = np.random.default_rng(seed)
    T, d, E, k, I = 48, 128, 6, 2, 64
    X = oracle.bf16_round(rng.standard_normal((T, d)))
    W1 = oracle.bf16_round(rng.standard_normal((E, 2 * I, d)) * 0.05)
    W2 = oracle.bf16_round(rng.standard_normal((E, d, I)) * 0.05)
    Wr = oracle.bf16_round(rng.standard_normal((E, d)) * 0.05)
    dY = oracle.bf16_round(rng.standard_normal((T, d)))
    fe = oracle.forward(X, W1, W2, Wr=Wr, k=k, storage="exact")
    be = oracle.backward(fe, X, W1, W2, dY, Wr=Wr)
    fm = oracle.forward(X, W1, W2, Wr=Wr, k=k, precision="mxfp8")
    bm = oracle.backward(fm, X, W1, W2, dY, Wr=Wr)
    np.testing.assert_array_equal(fm["idx"], fe["idx"])

    def rel(a, b):
        return np.linalg.norm(a - b) / np.linalg.norm(b)

    # E4M3 keeps 3 mantissa bits: each quantised operand carries a relative rounding error of
    # at most 2^-4, about 2^-4 / sqrt(3) = 0.036 RMS; a sum of such products keeps that relative
    # size. Y passes through 4 quantised operands (Xp, W1, A, W2), dX through up to 6, and the
    # weight gradients through 2-4, so their root-sum-square is 0.07-0.09. The bound allows
    # 0.12, and the floor shows that quantisation did happen.
    for name, a, b in (("Y", fm["Y"], fe["Y"]), ("dX", bm["dX"], be["dX"]),
                       ("dW1", bm["dW1"], be["dW1"]), ("dW2", bm["dW2"], be["dW2"]),
                       ("dWr", bm["dWr"], be["dWr"])):
        r = rel(a, b)
        assert 1e-3 < r < 0.12, (name, r)


# --- MXFP8 weight gradients: quantisation along the positions of each expert segment ----------

def test_segment_quantisation_matches_a_block_by_block_brute_force():
    """qdq_segment: blocks of 32 rows from row 0, the last one short (45 = 32 + 13 rows). Each
    block and column: scale from the block's largest magnitude (frexp), elements by brute-force
    nearest E4M3 value (ties to the even code), saturated to 448."""
    import math
    rng = np.random.default_rng(9)
    x = rng.standard_normal((45, 6)) * 2.0 ** rng.integers(-5, 5, (45, 6))
    got = mx.qdq_segment(x)
    pos = mx.e4m3_value(np.arange(127))  # non-negative finite E4M3 values, ascending
    want = np.zeros_like(x)
    for r0 in range(0, 45, 32):
        blk = x[r0:r0 + 32]
        for c in range(6):
            amax = max(abs(v) for v in blk[:, c])
            e = math.frexp(amax)[1] - 1 if amax > 0 else None
            code = 0 if e is None else min(max(e - 8 + 127, 0), 254)
            scale = 2.0 ** (code - 127)
            for i, v in enumerate(blk[:, c]):
                a = min(abs(v) / scale, 448.0)
                dist = np.abs(pos - a)
                best = np.flatnonzero(dist == dist.min())
                q = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
                want[r0 + i, c] = math.copysign(pos[q] * scale, v)
    np.testing.assert_array_equal(got, want)


def _segment_exact(counts, cols, rng):
    """Rows exact in MXFP8 along the rows within each segment of `counts` rows (blocks of 32
    from each segment's first row), and the same rows made exact along the columns instead."""
    parts_r, parts_c = [], []
    for c in counts:
        n32 = (c + 31) // 32 * 32
        codes = rng.integers(0, 127, size=(n32, cols)).astype(np.uint8)
        codes[::32] = 0x7A
        sc = rng.integers(115, 125, size=(n32 // 32, cols)).astype(np.uint8)
        parts_r.append(mx.dequantize(codes, sc, axis=0)[:c])
        parts_c.append(mx.qdq(rng.standard_normal((c, cols)) * 0.5, axis=1) if cols % 32 == 0
                       else None)
    return parts_r, parts_c


def test_mxfp8_wgrad_quantises_along_each_expert_segment():
    """Given routing with segments of 45, 20 and 40 positions (none a multiple of 32, so blocks
    of later experts start off the 32-row grid of the whole position axis). With w = 1, dY rows
    and the saved A made exact in MXFP8 along each segment's positions, the MXFP8 dW2 equals the
    BF16 dW2 bit for bit; made exact along the columns instead, it differs."""
    rng = np.random.default_rng(10)
    counts = [45, 20, 40]
    E, d, I = 3, 64, 32
    T = sum(counts)
    idx = np.repeat(np.arange(E, dtype=np.int32), counts)
    rng.shuffle(idx)
    idx = idx.reshape(T, 1)
    w = np.ones((T, 1))
    X = oracle.bf16_round(rng.standard_normal((T, d)))
    W1 = oracle.bf16_round(rng.standard_normal((E, 2 * I, d)) * 0.1)
    W2 = oracle.bf16_round(rng.standard_normal((E, d, I)) * 0.1)
    f = oracle.forward(X, W1, W2, topk_idx=idx, topk_w=w, precision="mxfp8")
    rows_dy, _ = _segment_exact(counts, d, rng)
    rows_a, cols_a = _segment_exact(counts, I, rng)
    dY = np.zeros((T, d))
    dY[f["row_src"]] = np.concatenate(rows_dy)  # position p holds token row_src[p] (k = 1)
    fa = dict(f, A=np.concatenate(rows_a))
    bb = oracle.backward(fa, X, W1, W2, dY)
    bm = oracle.backward(fa, X, W1, W2, dY, wgrad="mxfp8")
    np.testing.assert_array_equal(bm["dW2"], bb["dW2"])
    assert not np.array_equal(bm["dW1"], bb["dW1"])  # dH and Xp are not exact: dW1 quantises
    fc = dict(f, A=np.concatenate(cols_a))
    assert not np.array_equal(oracle.backward(fc, X, W1, W2, dY, wgrad="mxfp8")["dW2"],
                              oracle.backward(fc, X, W1, W2, dY)["dW2"])


@pytest.mark.parametrize("seed", [11, 12])
def test_mxfp8_wgrad_stays_within_its_error_bound(seed):
    """Two more quantised operands per weight gradient than the MXFP8 layer's: dW1 and dW2 stay
    within the same 0.12 relative error of the exact layer (and above 1e-3: they quantise)."""
    rng = np.random.default_rng(seed)
    T, d, E, k, I = 80, 128, 5, 2, 64
    X = oracle.bf16_round(rng.standard_normal((T, d)))
    W1 = oracle.bf16_round(rng.standard_normal((E, 2 * I, d)) * 0.05)
    W2 = oracle.bf16_round(rng.standard_normal((E, d, I)) * 0.05)
    Wr = oracle.bf16_round(rng.standard_normal((E, d)) * 0.05)
    dY = oracle.bf16_round(rng.standard_normal((T, d)))
    fe = oracle.forward(X, W1, W2, Wr=Wr, k=k, storage="exact")
    be = oracle.backward(fe, X, W1, W2, dY, Wr=Wr)
    fm = oracle.forward(X, W1, W2, Wr=Wr, k=k, precision="mxfp8")
    bm = oracle.backward(fm, X, W1, W2, dY, Wr=Wr, wgrad="mxfp8")
    for name in ("dW1", "dW2"):
        r = np.linalg.norm(bm[name] - be[name]) / np.linalg.norm(be[name])
        assert 1e-3 < r < 0.12, (name, r)
    with pytest.raises(AssertionError):
        oracle.backward(fe, X, W1, W2, dY, Wr=Wr, wgrad="mxfp8")  # MXFP8 mode only
