"""float64 oracle of the fp8 input step: incoherent processing and per-tensor
e4m3 quantisation.  Test infrastructure only (see ``oracle/__init__.py``).

[Comparison] "Notes", FA-3 entry, and [Evolution] §4: FlashAttention-3 runs
both products in fp8 and applies incoherent processing first: Q and K are
multiplied along the head dimension by the same random orthogonal matrix
(a Hadamard matrix with random signs), which leaves Q Kᵀ unchanged and
spreads a channel's outliers over all channels, so that a per-tensor scale
wastes fewer code values.  The pages name the transform and its purpose but
print no formula; the plain reading written out here:

    R        = diag(signs) · H_d / sqrt(d)      H_d the Sylvester Hadamard
                                                matrix, H[i][j] = (-1)^popcount(i & j)
    y        = x · R                            per row of d values
    descale  = max |y| / 448                    one factor per tensor (448 is
                                                the largest finite e4m3 value)
    code     = e4m3(y / descale)                round to nearest, ties to even
                                                mantissa, saturating at ±448

so that code · descale ≈ x · R and (x R)(z R)ᵀ = x zᵀ for any rows x, z.
Without signs (V, which is not rotated) y = x.

The e4m3 format (OCP "E4M3FN"): sign, 4 exponent bits (bias 7), 3 mantissa
bits, subnormals at exponent field 0, code 0x7F/0xFF is NaN and there is no
infinity.  The rounding here picks, among all finite code values, the nearest
one by value, which is a different construction from a bit-manipulating
encoder.
"""

import numpy as np

E4M3_MAX = 448.0


def hadamard_ref(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d (a power of two), entries ±1:
    H[i][j] = (-1)^popcount(i & j)."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    i = np.arange(d)
    bits = np.bitwise_and.outer(i, i)
    pop = np.zeros_like(bits)
    while bits.any():
        pop += bits & 1
        bits = bits >> 1
    return np.where(pop % 2 == 0, 1.0, -1.0)


def rotation_ref(signs) -> np.ndarray:
    """R = diag(signs) · H_d / sqrt(d) for a ±1 sign vector of length d."""
    s = np.asarray(signs, dtype=np.float64)
    d = s.shape[0]
    return (s[:, None] * hadamard_ref(d)) / np.sqrt(d)


def rotate_ref(x, signs) -> np.ndarray:
    """y = x · R over the last axis, in float64."""
    x = np.asarray(x, dtype=np.float64)
    return x @ rotation_ref(signs)


def e4m3_values() -> np.ndarray:
    """Value of every non-negative finite e4m3 code 0x00..0x7E, by code."""
    c = np.arange(0x7F)
    e = c >> 3
    m = c & 7
    return np.where(e == 0, m * 2.0 ** -9, (8 + m) * 2.0 ** (e.astype(np.float64) - 10))


def e4m3_round_ref(v) -> np.ndarray:
    """Codes of the e4m3 values nearest to v (ties to the even code, i.e. the
    even mantissa), saturating at ±448, keeping the sign of v also when the
    magnitude rounds to zero (0x80 = -0).  v must be finite."""
    v = np.asarray(v, dtype=np.float64)
    table = e4m3_values()
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.clip(np.searchsorted(table, a, side="left"), 0, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - table[lo]
    d_hi = table[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)


def e4m3_decode_ref(codes) -> np.ndarray:
    """float64 values of finite e4m3 codes."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = e4m3_values()[np.minimum(c & 0x7F, 0x7E)]
    return np.where(c & 0x80, -mag, mag)


def rotate_quantize_ref(x, signs=None):
    """(codes uint8, descale float) of one tensor x [..., d]: rotated by R
    when signs are given, then quantised per tensor.  The codes decode to
    y / descale rounded to e4m3."""
    x = np.asarray(x, dtype=np.float64)
    y = rotate_ref(x, signs) if signs is not None else x
    amax = float(np.abs(y).max()) if y.size else 0.0
    descale = amax / E4M3_MAX if amax > 0 else 1.0
    return e4m3_round_ref(y / descale), descale
