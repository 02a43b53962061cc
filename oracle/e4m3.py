"""OCP FP8 E4M3 ("e4m3fn") codec written from the format's definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Format: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits. No infinities;
the codes S.1111.111 are NaN, so the largest finite magnitude is
2^8 * 1.75 = 448. Exponent field 0 encodes subnormals m/8 * 2^-6.

The Step-3 summary page (§5 Model-System Co-design) speaks of an 8-bit KV
cache and of KV quantisation; the 8-bit float format itself is not named
there. OCP e4m3 is the reading taken here.
"""
from __future__ import annotations

import numpy as np

MAX_FINITE = 448.0
NAN_CODES = (0x7F, 0xFF)


def decode_code(code: int) -> float:
    """Value of one code, from the closed form (NaN for 0x7F / 0xFF)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# Table of all 256 decoded values (fp64, exact).
DECODE_TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)

# Non-negative finite values in increasing order: codes 0x00 .. 0x7E.
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = DECODE_TABLE[:0x7F]


def decode(codes: np.ndarray) -> np.ndarray:
    """Decode an array of uint8 codes to fp64."""
    return DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


def encode_rne(x: np.ndarray) -> np.ndarray:
    """Encode float values to e4m3 codes: nearest value, ties to the even code.

    Magnitudes beyond the largest finite value saturate to +-448 (the values
    this oracle quantises never get there: see ``oracle.mfa.quantize_tokens``).
    The sign bit of the input is kept, so negative values that round to zero
    give the negative-zero code 0x80. NaN inputs are rejected.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN input to e4m3 encoder")
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), MAX_FINITE)
    # index of the first table value >= a
    hi = np.searchsorted(_POS_VALUES, a, side="left")
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    v_hi = _POS_VALUES[hi]
    v_lo = _POS_VALUES[lo]
    d_hi = v_hi - a
    d_lo = a - v_lo
    pick_hi = d_hi < d_lo
    tie = d_hi == d_lo
    # ties: take the even code (codes of adjacent values differ by one)
    pick_hi = np.where(tie, (_POS_CODES[hi] % 2) == 0, pick_hi)
    # exact hits: a == v_hi gives d_hi == 0 < d_lo, or a == v_lo == v_hi at 0
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    return np.where(neg, code | 0x80, code).astype(np.uint8)
