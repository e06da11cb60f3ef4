"""Pins of the oracle's MXFP4 quantiser and its MXFP4 layer mode (CPU).

* E2M1 decode: the 16 codes against the format's table of values (sign, then the magnitudes
  0, 0.5, 1, 1.5, 2, 3, 4, 6, as OCP MX v1.0 lists them).
* E2M1 encode: against a brute-force nearest-value search with ties to the even code and
  saturation at 6, on a fine grid that holds every tie, and on random values.
* The E8M0 scale puts each block's largest magnitude in [4, 8) after scaling; only values in
  (6, 8) times the scale saturate; the error of every element is at most half the E2M1 spacing
  of its binade (times the scale), or the saturation gap.
* The layer: inputs exact in MXFP4 along the stated axes leave the forward H and the backward
  dH unchanged between BF16 and MXFP4 modes (and exact along the other axis they do not), and
  the whole MXFP4 layer stays within its derived error bound of the exact layer.
"""
import numpy as np
import pytest

import oracle
from oracle import mx

# OCP MX v1.0, FP4 (E2M1): the magnitudes of codes 0..7; codes 8..15 are their negatives
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_matches_the_format_table():
    want = np.array(E2M1_TABLE + [-v for v in E2M1_TABLE])
    got = mx.e2m1_value(np.arange(16))
    np.testing.assert_array_equal(got, want)
    assert np.signbit(got[8]) and not np.signbit(got[0])  # code 8 is -0


def _brute_encode(v):
    """Nearest E2M1 magnitude by search; ties to the even code; beyond 6 saturates."""
    a = min(abs(v), 6.0)
    best = None
    for c, m in enumerate(E2M1_TABLE):
        d = abs(a - m)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1] | (8 if np.signbit(v) else 0)


def test_e2m1_encode_against_brute_force():
    grid = np.arange(-8 * 64, 8 * 64 + 1) / 64.0  # every tie (multiples of 1/4) is on the grid
    rng = np.random.default_rng(1)
    vals = np.concatenate([grid, rng.standard_normal(4000) * 3, [-0.0, 1e-30, -7.99, 100.0]])
    got = mx.e2m1_encode(vals)
    want = np.array([_brute_encode(v) for v in vals], dtype=np.uint8)
    np.testing.assert_array_equal(got, want)


def test_e2m1_ties_go_to_the_even_code():
    ties = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for v, want in ties.items():
        for s in (1, -1):
            assert mx.e2m1_value(mx.e2m1_encode(s * v)) == s * want, (s * v)


def test_mxfp4_scale_and_saturation():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 256)) * np.exp2(rng.integers(-20, 20, size=(64, 1)))
    q, sc = mx.quantize(x, fmt="e2m1")
    b = x.reshape(64, 8, 32)
    scale = np.exp2(sc.astype(np.float64) - 127.0)[..., None]
    amax = np.max(np.abs(b), axis=-1, keepdims=True) / scale
    assert np.all((amax >= 4.0) & (amax < 8.0))
    v = mx.dequantize(q, sc, fmt="e2m1").reshape(64, 8, 32)
    a = np.abs(b) / scale
    sat = a > 6.0
    np.testing.assert_array_equal(np.abs(v[sat]) / scale.repeat(32, -1)[sat], 6.0)
    # every other element within half the spacing of its binade: 0.25 below 2, 0.5 in [2, 4),
    # 1 in [4, 8)
    half = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0))
    err = np.abs(np.abs(v) / scale - a)
    assert np.all(err[~sat] <= half[~sat])
    assert np.all(err[sat] < 2.0)
    # all-zero blocks: scale code 0, zero codes
    qz, sz = mx.quantize(np.zeros((2, 64)), fmt="e2m1")
    assert not qz.any() and not sz.any()


def _mx4_exact(shape, rng, scale_lo=115, scale_hi=125):
    """Values exactly representable in MXFP4 along the last axis: random codes with one block
    maximum of magnitude 4 or 6 per block, times a random scale per block."""
    *lead, n = shape
    codes = rng.integers(0, 16, size=shape).astype(np.uint8)
    codes[..., ::32] = rng.integers(6, 8, size=(*lead, n // 32)).astype(np.uint8)
    sc = rng.integers(scale_lo, scale_hi, size=(*lead, n // 32)).astype(np.uint8)
    x = mx.dequantize(codes, sc, fmt="e2m1")
    assert np.array_equal(mx.qdq4(x), x)
    assert np.array_equal(oracle.bf16_round(x), x)
    return x


def test_mxfp4_forward_quantises_x_and_w1_along_d():
    rng = np.random.default_rng(5)
    T, d, E, k, I = 24, 64, 4, 2, 32
    X = _mx4_exact((T, d), rng, 120, 126)
    W1 = _mx4_exact((E, 2 * I, d), rng, 110, 116)
    W2 = oracle.bf16_round(rng.standard_normal((E, d, I)) * 0.05)
    Wr = oracle.bf16_round(rng.standard_normal((E, d)) * 0.1)
    fb = oracle.forward(X, W1, W2, Wr=Wr, k=k)
    fm = oracle.forward(X, W1, W2, Wr=Wr, k=k, precision="mxfp4")
    np.testing.assert_array_equal(fm["H"], fb["H"])
    np.testing.assert_array_equal(fm["A"], fb["A"])
    assert not np.array_equal(fm["O"], fb["O"])  # A is not MXFP4-exact: GEMM2 quantises
    W1t = np.swapaxes(_mx4_exact((E, d, 2 * I), rng, 110, 116), 1, 2).copy()
    fb2 = oracle.forward(X, W1t, W2, Wr=Wr, k=k)
    fm2 = oracle.forward(X, W1t, W2, Wr=Wr, k=k, precision="mxfp4")
    assert not np.array_equal(fm2["H"], fb2["H"])


def test_mxfp4_backward_quantises_dy_and_w2_along_d():
    rng = np.random.default_rng(6)
    T, d, E, k, I = 24, 64, 4, 2, 32
    X = oracle.bf16_round(rng.standard_normal((T, d)))
    W1 = oracle.bf16_round(rng.standard_normal((E, 2 * I, d)) * 0.1)
    W2 = np.swapaxes(_mx4_exact((E, I, d), rng, 110, 116), 1, 2).copy()  # exact along d
    dY = _mx4_exact((T, d), rng, 120, 126)
    Wr = oracle.bf16_round(rng.standard_normal((E, d)) * 0.1)
    fb = oracle.forward(X, W1, W2, Wr=Wr, k=k)
    fm = oracle.forward(X, W1, W2, Wr=Wr, k=k, precision="mxfp4")
    fm_h = dict(fm, H=fb["H"], A=fb["A"])  # isolate the backward: same saved H and A
    bb = oracle.backward(fb, X, W1, W2, dY, Wr=Wr)
    bm = oracle.backward(fm_h, X, W1, W2, dY, Wr=Wr)
    np.testing.assert_array_equal(bm["dH"], bb["dH"])
    W2i = _mx4_exact((E, d, I), rng, 110, 116)  # exact along I instead
    f2 = oracle.forward(X, W1, W2i, Wr=Wr, k=k)
    fm2 = oracle.forward(X, W1, W2i, Wr=Wr, k=k, precision="mxfp4")
    bb2 = oracle.backward(f2, X, W1, W2i, dY, Wr=Wr)
    bm2 = oracle.backward(dict(fm2, H=f2["H"], A=f2["A"]), X, W1, W2i, dY, Wr=Wr)
    assert not np.array_equal(bm2["dH"], bb2["dH"])


@pytest.mark.parametrize("seed", [7, 8])
def test_mxfp4_layer_stays_within_its_error_bound_of_the_exact_layer(seed):
    rng = np.random.default_rng(seed)
    T, d, E, k, I = 48, 128, 6, 2, 64
    X = oracle.bf16_round(rng.standard_normal((T, d)))
    W1 = oracle.bf16_round(rng.standard_normal((E, 2 * I, d)) * 0.05)
    W2 = oracle.bf16_round(rng.standard_normal((E, d, I)) * 0.05)
    Wr = oracle.bf16_round(rng.standard_normal((E, d)) * 0.05)
    dY = oracle.bf16_round(rng.standard_normal((T, d)))
    fe = oracle.forward(X, W1, W2, Wr=Wr, k=k, storage="exact")
    be = oracle.backward(fe, X, W1, W2, dY, Wr=Wr)
    fm = oracle.forward(X, W1, W2, Wr=Wr, k=k, precision="mxfp4")
    bm = oracle.backward(fm, X, W1, W2, dY, Wr=Wr)
    np.testing.assert_array_equal(fm["idx"], fe["idx"])

    def rel(a, b):
        return np.linalg.norm(a - b) / np.linalg.norm(b)

    # E2M1 keeps 1 mantissa bit. With the block maximum scaled into [4, 8), a Gaussian block's
    # elements spread over the binades below it, where the spacing relative to the value is
    # 1/4 to 1/2 (and values under half the scale round to 0 or 0.5): the RMS relative error of
    # one MXFP4 image of Gaussian data is about 0.11 (checked here on X). A product of two such
    # images carries about sqrt(2) of it; Y passes through two GEMMs (four images, about 0.22),
    # dX through up to six (about 0.27), and the requantised A and dH add to both (0.22-0.32
    # measured at these seeds). The bound allows 0.5, and the floor (0.05) shows that the
    # quantisation happened; MXFP8 with 3 mantissa bits stays under 0.12.
    eps = rel(mx.qdq4(X), X)
    assert 0.08 < eps < 0.16, eps
    for name, a, b in (("Y", fm["Y"], fe["Y"]), ("dX", bm["dX"], be["dX"]),
                       ("dW1", bm["dW1"], be["dW1"]), ("dW2", bm["dW2"], be["dW2"]),
                       ("dWr", bm["dWr"], be["dWr"])):
        r = rel(a, b)
        assert 0.05 < r < 0.5, (name, r)


@pytest.mark.parametrize("precision, qdq, bound", [("mxfp8", mx.qdq, 0.05), ("mxfp4", mx.qdq4, 0.2)])
def test_mx_dwr_reads_the_ring_image_of_x_and_its_distance_from_the_exact_product(precision, qdq,
                                                                                   bound):
    """In the MX modes dWr = dlogits^T Xq, Xq being the MX image of X that the ring holds (the
    readings "mxfp8", "mxfp4"), not dlogits^T X. This pins that it is exactly that product (on
    the oracle's own dlogits) and states how far it is from the exact one: the relative
    Frobenius distance is the MX quantisation error of X carried through one product, about
    0.02 (E4M3) and 0.11 (E2M1) on Gaussian tokens."""
    rng = np.random.default_rng(11)
    T, d, E, k, I = 64, 256, 8, 2, 64
    X = oracle.bf16_round(rng.standard_normal((T, d)))
    W1 = oracle.bf16_round(rng.standard_normal((E, 2 * I, d)) * 0.05)
    W2 = oracle.bf16_round(rng.standard_normal((E, d, I)) * 0.05)
    Wr = oracle.bf16_round(rng.standard_normal((E, d)) * 0.05)
    dY = oracle.bf16_round(rng.standard_normal((T, d)))
    f = oracle.forward(X, W1, W2, Wr=Wr, k=k, precision=precision)
    b = oracle.backward(f, X, W1, W2, dY, Wr=Wr)
    dl = b["dlogits"]
    np.testing.assert_allclose(b["dWr"], dl.T @ qdq(X), rtol=1e-12, atol=1e-15)
    exact = dl.T @ X
    dist = np.linalg.norm(b["dWr"] - exact) / np.linalg.norm(exact)
    eps_x = np.linalg.norm(qdq(X) - X) / np.linalg.norm(X)
    print(f"  {precision}: dWr vs dlogits^T X: rel fro {dist:.3e} (X's MX error {eps_x:.3e})")
    assert 0.3 * eps_x < dist < bound, (dist, eps_x)
