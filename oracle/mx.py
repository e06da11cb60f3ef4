"""MXFP8 and MXFP4 quantisation for the oracle. Test infrastructure only: the GPU library never
uses it.

The pages name an MXFP8 precision mode next to BF16 (MarkTechPost, "Cursor Open-Sources
Mixture-of-Kittens (MoK)", closing paragraph of "Three design decisions that matter") and give
no recipe. The format is the OCP Microscaling (MX) v1.0 MXFP8 format:
* the element is E4M3: sign, 4 exponent bits with bias 7, 3 mantissa bits. Exponent field 0
  encodes subnormals m/8 * 2^-6. There is no infinity. S.1111.111 is NaN, so the largest
  finite magnitude is 1.75 * 2^8 = 448;
* every block of 32 consecutive elements along the reduction axis shares one E8M0 scale, a bare
  power of two 2^(code - 127) with code 0..254 (255 is NaN).

Readings (the pages are silent):
* The scale exponent is floor(log2(amax)) - 8, with 8 the largest normal exponent of E4M3,
  clamped to the E8M0 range. An all-zero block gets code 0.
* Each element v becomes E4M3(v / scale), rounded to nearest with ties to the even code.
  Magnitudes beyond 448 saturate to 448. After scaling the block maximum lies in [256, 512), so
  only values in (448, 512) saturate.

MXFP4, the 4-bit analogue (the pages name NVFP4 training kernels beside the MXFP8 ones; OCP MX
v1.0 defines MXFP4 with the same E8M0 block scale):
* the element is E2M1: sign, 2 exponent bits with bias 1, 1 mantissa bit. Exponent field 0
  encodes the subnormal 0.5; the magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6. There is no infinity
  or NaN;
* the scale exponent is floor(log2(amax)) - 2, with 2 the largest exponent of E2M1, so after
  scaling the block maximum lies in [4, 8) and values in (6, 8) saturate to 6; elements round to
  nearest with ties to the even code, as in MXFP8.
Codes are returned one per element (the GPU packs two per byte).
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E4M3_MAX = 448.0
E4M3_EMAX = 8  # exponent of the largest normal E4M3 value


def _e4m3_formula(codes) -> np.ndarray:
    """float64 value of each E4M3 code by the format's definition; NaN for S.1111.111."""
    c = np.asarray(codes, dtype=np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


_VALUES = _e4m3_formula(np.arange(256))  # value of every code


def e4m3_value(codes) -> np.ndarray:
    """float64 value of each E4M3 code (uint8); NaN for S.1111.111."""
    return _VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v) -> np.ndarray:
    """E4M3 codes of float64 values: round to nearest, ties to the even code, and saturate to
    +-448. The sign bit is the sign of v.

    A magnitude a <= 448 lies in the binade [2^e, 2^(e+1)), where E4M3 values are spaced
    2^(e-3); the subnormals below 2^-6 share the spacing 2^-9. The nearest value is
    n * 2^(e-3) with n = a / 2^(e-3) rounded half-to-even. n's parity is the code's last bit,
    so ties go to the even code. n = 16 carries into the next binade."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    _, x = np.frexp(a)                       # a = f 2^x, f in [0.5, 1): floor(log2 a) = x - 1
    e = np.maximum(x - 1, -6)
    n = np.rint(a / np.exp2(e - 3.0))        # 0..16; round half to even
    carry = n == 16
    e = np.where(carry, e + 1, e)
    n = np.where(carry, 8, n)
    code = np.where(n < 8, n, (e + 7) * 8 + (n - 8)).astype(np.uint8)
    return code | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)


E2M1_MAX = 6.0
E2M1_EMAX = 2  # exponent of the largest E2M1 value


def _e2m1_formula(codes) -> np.ndarray:
    """float64 value of each E2M1 code (0..15) by the format's definition."""
    c = np.asarray(codes, dtype=np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m / 2.0, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return np.where(s == 1, -mag, mag)


_VALUES4 = _e2m1_formula(np.arange(16))


def e2m1_value(codes) -> np.ndarray:
    """float64 value of each E2M1 code (0..15)."""
    return _VALUES4[np.asarray(codes, dtype=np.uint8) & 15]


def e2m1_encode(v) -> np.ndarray:
    """E2M1 codes (0..15) of float64 values: round to nearest, ties to the even code, and
    saturate to +-6. The sign bit (8) is the sign of v.

    A magnitude a <= 6 lies in the binade [2^e, 2^(e+1)) (e = 0 for the subnormal range below
    1), where E2M1 values are spaced 2^(e-1). The nearest value is n 2^(e-1) with n = a / 2^(e-1)
    rounded half-to-even; n's parity is the code's last bit, so ties go to the even code. n = 4
    carries into the next binade (never past 6, since a <= 6)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E2M1_MAX)
    _, x = np.frexp(a)
    e = np.maximum(x - 1, 0)
    n = np.rint(a / np.exp2(e - 1.0))        # 0..4; round half to even
    carry = n == 4
    e = np.where(carry, e + 1, e)
    n = np.where(carry, 2, n)
    code = np.where(n < 2, n, (e + 1) * 2 + (n - 2)).astype(np.uint8)
    return code | np.where(np.signbit(v), 8, 0).astype(np.uint8)


# element format -> (encode, decode, exponent of the largest element)
FORMATS = {"e4m3": (e4m3_encode, e4m3_value, E4M3_EMAX),
           "e2m1": (e2m1_encode, e2m1_value, E2M1_EMAX)}


def e8m0_code(amax, emax=E4M3_EMAX) -> np.ndarray:
    """Shared-scale code of blocks with the given max magnitudes: floor(log2 amax) - emax + 127,
    clamped to 0..254, and 0 for an all-zero block; emax is the element format's largest
    exponent (8 for E4M3, 2 for E2M1). frexp gives amax = f 2^x with f in [0.5, 1), so
    floor(log2 amax) = x - 1 exactly."""
    amax = np.asarray(amax, dtype=np.float64)
    _, x = np.frexp(amax)
    code = np.clip(x - 1 - emax + 127, 0, 254)
    return np.where(amax > 0, code, 0).astype(np.uint8)


def quantize(x, axis=-1, fmt="e4m3"):
    """MX quantisation along `axis` (its length a multiple of 32) with element format `fmt`
    ("e4m3": MXFP8, "e2m1": MXFP4). Returns (codes uint8 with the shape of x, one per element,
    scale codes uint8 with that axis divided by 32)."""
    enc, _, emax = FORMATS[fmt]
    x = np.moveaxis(np.asarray(x, dtype=np.float64), axis, -1)
    n = x.shape[-1]
    assert n % BLOCK == 0, "the quantised axis must be a multiple of 32"
    b = x.reshape(*x.shape[:-1], n // BLOCK, BLOCK)
    sc = e8m0_code(np.max(np.abs(b), axis=-1), emax)
    q = enc(b / np.exp2(sc.astype(np.float64) - 127.0)[..., None])
    q = q.reshape(x.shape)
    return np.moveaxis(q, -1, axis), np.moveaxis(sc, -1, axis)


def dequantize(q, sc, axis=-1, fmt="e4m3") -> np.ndarray:
    """float64 values of MX codes with their block scales along `axis`."""
    _, dec, _ = FORMATS[fmt]
    q = np.moveaxis(np.asarray(q), axis, -1)
    sc = np.moveaxis(np.asarray(sc), axis, -1)
    v = dec(q).reshape(*q.shape[:-1], q.shape[-1] // BLOCK, BLOCK)
    v = v * np.exp2(sc.astype(np.float64) - 127.0)[..., None]
    return np.moveaxis(v.reshape(q.shape), -1, axis)


def qdq(x, axis=-1, fmt="e4m3") -> np.ndarray:
    """The float64 image of x after MX quantisation along `axis` (MXFP8 by default)."""
    q, sc = quantize(x, axis, fmt)
    return dequantize(q, sc, axis, fmt)


def qdq4(x, axis=-1) -> np.ndarray:
    """The float64 image of x after MXFP4 quantisation along `axis`."""
    return qdq(x, axis, "e2m1")


def qdq_segment(x) -> np.ndarray:
    """The float64 image of x [rows, cols] after MXFP8 quantisation along its ROWS in blocks of
    32 consecutive rows starting at row 0, the last block holding what is left (fewer than 32
    rows when rows is not a multiple of 32). Rows are the positions of one expert segment, the
    reduction axis of a weight-gradient product. The short last block is quantised as if padded
    with zero rows: zeros change neither its largest magnitude nor any product."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    pad = (-n) % BLOCK
    xp = np.concatenate([x, np.zeros((pad,) + x.shape[1:])], axis=0) if pad else x
    return qdq(xp, axis=0)[:n]
