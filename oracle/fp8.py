"""8-bit floating-point (E4M3) KV storage -- TEST INFRASTRUCTURE ONLY.

Part of the CPU oracle: only tests/, the smoke check and the CPU-baseline leg
of the benchmark use it.  It shares nothing with the HIP library.

Why an 8-bit cache at all: the KV-cache article (intelliparadigm) lists a
low-bit (fp8) loading option among its fixes in §4.2 and names a deeper
combination of paging with quantisation as a direction in §5.  The pages
fix no format, so the format is the OCP 8-bit floating point
specification's E4M3 encoding (the one gfx950's conversion instructions
implement):

* bit 7 sign, bits 6..3 exponent e (bias 7), bits 2..0 mantissa m;
* e > 0: value (-1)^s * 2^(e-7) * (1 + m/8);  e = 0: (-1)^s * 2^-6 * (m/8);
* e = 15 with m = 7 is NaN; there is no infinity, so 448 (e = 15, m = 6) is
  the largest finite magnitude.

Storing a real value x with a per-tensor scale s (reading of this library:
one scale for every K element, one for every V element):
  1. y = x / s, one correctly rounded float32 division of float32 operands;
  2. the code is the finite E4M3 value nearest to y; a tie goes to the code
     with an even mantissa; magnitudes above 448 saturate to 448 (the OCP
     specification's saturating conversion), signs are kept (-0 -> 0x80).
Reading a code back gives e4m3_value(code) * s.

Parity pins: tests/test_oracle_fp8.py checks the value table against values
the specification fixes by hand, against torch's float8_e4m3fn decoding, and
the encoder against brute-force nearest search, exact ties, saturation and
torch's round-to-nearest-even cast.
"""

import numpy as np

E4M3_MAX = 448.0


def e4m3_value(code):
    """Value of one E4M3 code (int 0..255) as a Python float, from its fields."""
    code = int(code)
    if not 0 <= code <= 255:
        raise ValueError("code must be a byte")
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (2.0 ** -6) * (m / 8.0)
    return sign * (2.0 ** (e - 7)) * (1.0 + m / 8.0)


def e4m3_table():
    """float64 array of the 256 code values (NaN at 0x7F and 0xFF)."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def _positive_codes():
    """Non-negative finite codes 0x00..0x7E and their values, ascending."""
    codes = np.arange(0x7F, dtype=np.int64)
    vals = np.array([e4m3_value(c) for c in codes], dtype=np.float64)
    assert np.all(np.diff(vals) > 0)
    return codes, vals


def float_to_e4m3(y):
    """Round float32 values to E4M3 codes: nearest, ties to even, saturating.

    `y` is converted to float32 first; the comparison itself is exact in
    float64 (every float32 and every midpoint of two codes is a float64).
    For each |y| the two neighbouring code values lo <= |y| < hi are found
    in the ascending table; the nearer wins, an exact tie goes to the code
    whose mantissa (code bit 0) is even.
    """
    y = np.asarray(y, dtype=np.float32)
    flat = y.reshape(-1).astype(np.float64)
    codes, vals = _positive_codes()
    a = np.abs(flat)
    nan = np.isnan(flat)
    sign = np.where(np.signbit(flat), 0x80, 0x00).astype(np.int64)
    j = np.clip(np.searchsorted(vals, np.where(nan, 0.0, a), side="right"), 1, len(vals) - 1)
    lo, hi = j - 1, j
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick = np.where(d_lo < d_hi, lo,
                    np.where(d_hi < d_lo, hi, np.where(codes[lo] % 2 == 0, lo, hi)))
    out = codes[pick]
    out = np.where(a >= E4M3_MAX, 0x7E, out)
    out = np.where(nan, 0x7F, out) | sign
    return out.astype(np.uint8).reshape(y.shape)


def quantize(x, scale):
    """Codes for real values x with per-tensor scale s: float_to_e4m3(x / s),
    the division done once in float32 (IEEE, correctly rounded)."""
    x32 = np.asarray(x, dtype=np.float32)
    s32 = np.float32(scale)
    if not (np.isfinite(s32) and s32 > 0):
        raise ValueError("scale must be a positive finite float32")
    with np.errstate(over="ignore"):
        y = np.divide(x32, s32, dtype=np.float32)
    return float_to_e4m3(y)


def dequantize(codes, scale):
    """float64 values code_value * s of a uint8 code array."""
    codes = np.asarray(codes, dtype=np.uint8)
    return e4m3_table()[codes.astype(np.int64)] * float(np.float32(scale))
