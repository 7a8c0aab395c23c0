"""OCP FP8 E4M3FN codec, written from the format definition (fp64, NumPy).

Test infrastructure only (see the package docstring).

Format ("FP8 E4M3FN" is the Q/K/V data type in the constraint table of
"Quant Block Sparse Attention", section "Operator introduction"):
  1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits.
  exponent field 1..15 -> normal   (-1)^s * 2^(e-7) * (1 + m/8)
  exponent field 0     -> subnormal (-1)^s * 2^(-6) * (m/8)
  S.1111.111 is NaN; there is no infinity; the largest finite value is
  0b0.1111.110 = 2^8 * 1.75 = 448.

Encoding rounds to nearest, ties to even, and saturates finite values of
magnitude above 448 to +-448 (the saturating variant); NaN maps to 0x7F.
"""
import numpy as np

MAX_E4M3 = 448.0
MIN_NORMAL_EXP = -6          # smallest normal exponent, 2^-6
MANT_BITS = 3


def _decode_code(c: int) -> float:
    s = -1.0 if (c >> 7) & 1 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (2.0 ** MIN_NORMAL_EXP) * (m / 8.0)
    return s * (2.0 ** (e - 7)) * (1.0 + m / 8.0)


# Table of all 256 codes, built from the definition above.
DECODE_TABLE = np.array([_decode_code(c) for c in range(256)], dtype=np.float64)


def decode(codes) -> np.ndarray:
    """uint8 codes (any shape) -> float64 values."""
    return DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


def round_to_grid(x) -> np.ndarray:
    """Round float64 values to the nearest E4M3FN value (RNE, saturating), as float64.

    For |x| >= 2^-6 the grid spacing at exponent e = floor(log2|x|) is 2^(e-3);
    below 2^-6 (subnormals) it is 2^-9.  Division by a power of two is exact in
    fp64 and np.rint rounds half to even, so the result is the correctly rounded
    value.  A value that rounds up past 448 saturates to 448.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    with np.errstate(divide="ignore", invalid="ignore"):
        _, E = np.frexp(a)                       # a = f * 2^E, f in [0.5, 1)
    e = np.maximum(E - 1, MIN_NORMAL_EXP)        # exponent of the binade (clamped to subnormal range)
    q = np.ldexp(1.0, e - MANT_BITS)             # grid spacing
    r = np.rint(a / q) * q
    r = np.minimum(r, MAX_E4M3)
    r = np.where(np.isnan(x), np.nan, r)
    return np.copysign(r, x)


def encode(x) -> np.ndarray:
    """float64 values -> uint8 E4M3FN codes (RNE, saturating; NaN -> 0x7F)."""
    v = round_to_grid(x)
    out = np.empty(v.shape, dtype=np.uint8)
    flat_v = v.reshape(-1)
    flat_o = out.reshape(-1)
    # Positive codes 0x00..0x7E are strictly increasing in value, so a sorted
    # search over that half of the table maps each grid value to its code.
    pos_vals = DECODE_TABLE[:0x7F]
    mag = np.abs(flat_v)
    nan = np.isnan(flat_v)
    idx = np.searchsorted(pos_vals, np.where(nan, 0.0, mag))
    sign = np.signbit(flat_v) & ~nan
    flat_o[:] = idx.astype(np.uint8) | (sign.astype(np.uint8) << 7)
    flat_o[nan] = 0x7F
    return out
