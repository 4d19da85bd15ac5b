"""OCP 8-bit floating point, E4M3 variant ("e4m3fn"), written from the format's definition.

Test infrastructure only (see ``oracle/__init__``).

Encoding of a byte ``b``: sign ``b >> 7``, exponent field ``(b >> 3) & 15``
with bias 7, mantissa field ``b & 7``.

* exponent field 0: subnormal, value = m/8 * 2**(1-7)
* exponent field 1..15: value = (1 + m/8) * 2**(e-7)
* exponent 15 with mantissa 7 (0x7F, 0xFF) is NaN; there is no infinity.

Largest finite magnitude 448 (0x7E), smallest normal 2**-6, smallest
subnormal 2**-9.

The encoder rounds a float32 value to the nearest representable magnitude,
ties to the code with an even mantissa (round-to-nearest-even), saturating at
448; the sign of the input is kept (a negative value that rounds to zero
gives 0x80).  NaN inputs are outside its domain.
"""

from __future__ import annotations

import numpy as np

MAX = 448.0


def _decode_formula(codes) -> np.ndarray:
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    sub = m / 8.0 * 2.0 ** -6
    nrm = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    val = np.where(e == 0, sub, nrm) * sign
    return np.where((e == 15) & ((c & 7) == 7), np.nan, val)


# The value of every code, from the formula above; decoding is a table lookup.
_TABLE = _decode_formula(np.arange(256))


def decode(codes) -> np.ndarray:
    """uint8 codes -> float64 values (NaN for 0x7F / 0xFF)."""
    return _TABLE[np.asarray(codes).astype(np.uint8)]


# Non-negative finite codes 0x00..0x7E in order; their values increase with the code.
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALS = decode(_POS_CODES)


def encode(values) -> np.ndarray:
    """float32 values -> uint8 codes, round-to-nearest-even, saturating at +-448."""
    v = np.asarray(values, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    hi = np.searchsorted(_POS_VALS, a, side="left")          # first value >= a
    hi = np.clip(hi, 0, len(_POS_VALS) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALS) - 1)
    v_hi, v_lo = _POS_VALS[hi], _POS_VALS[lo]
    d_hi, d_lo = v_hi - a, a - v_lo
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((_POS_CODES[hi] & 1) == 0))
    code = np.where(a >= v_hi, hi, np.where(pick_hi, hi, lo))
    code = np.where(a >= MAX, 0x7E, code)
    code = code | np.where(np.signbit(v), 0x80, 0)
    return code.astype(np.uint8)
