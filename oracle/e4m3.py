"""OCP FP8 E4M3 ("fn" variant) codec for the CPU oracle -- test infrastructure only.

Only tests, the smoke check and the benchmark's CPU-baseline leg import this.

Format (OCP 8-bit floating point specification, E4M3): 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits; exponent field 0 holds subnormals
(m/8 * 2^-6); exponent field 15 with mantissa 7 is NaN and there are no
infinities, so the largest finite magnitude is 1.75 * 2^8 = 448.

The encoder rounds to nearest, ties to even, and saturates magnitudes at or
above 448 to 448 (the fp8 workload's activation quantiser never produces NaN).
The sign of the input is kept, also when the result is zero.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def _decode_one(code: int) -> float:
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        v = (m / 8.0) * 2.0 ** -6
    else:
        v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


#: value of every code 0..255 (float64; NaN at 0x7F and 0xFF)
E4M3_VALUES = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)
#: the 127 finite non-negative values, codes 0x00..0x7E, ascending
_POS = E4M3_VALUES[:127].copy()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64 values."""
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """float32 values -> uint8 codes: round to nearest even, saturate at 448, keep the sign."""
    v = np.asarray(v, dtype=np.float32)
    if not np.all(np.isfinite(v)):
        raise ValueError("e4m3_encode expects finite inputs")
    a = np.abs(v).astype(np.float64)
    i = np.searchsorted(_POS, a, side="right") - 1          # _POS[i] <= a
    i = np.clip(i, 0, 125)
    lo = _POS[i]
    hi = _POS[i + 1]
    d_lo = a - lo
    d_hi = hi - a
    up = (d_hi < d_lo) | ((d_hi == d_lo) & (((i + 1) & 1) == 0))
    code = np.where(up, i + 1, i)
    code = np.where(a >= E4M3_MAX, 126, code)
    code = code.astype(np.uint8)
    code |= np.where(np.signbit(v), np.uint8(0x80), np.uint8(0))
    return code
