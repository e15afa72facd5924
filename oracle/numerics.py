"""Number formats the oracle needs: bfloat16 and OCP FP8 E4M3 (e4m3fn).

Test infrastructure (see the package docstring).

* bfloat16 = the top 16 bits of an IEEE binary32; widening is exact.  Rounding
  an fp32 value to bf16 is round-to-nearest, ties to even, written here as
  arithmetic on the significand so that it is checkable against the format's
  definition rather than against another bit trick.
* E4M3 (OCP 8-bit floating point specification, "E4M3" with no infinities):
  1 sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 encodes
  subnormals ``m * 2**-9``; exponent 15 with mantissa 7 is NaN; the largest
  finite magnitude is 448.  Encoding rounds to nearest, ties to even, and
  saturates magnitudes above 448 to 448 (the FP8 chain's ``FP8_MAX`` scale
  convention, flashrt-structures ``prefill_tower/fp8_chain.py`` ``_quantize``,
  only works if nothing maps past the largest finite value).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64 exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) * np.uint32(65536)
    return b.view(np.float32).astype(np.float64)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) * np.uint32(65536)
    return b.view(np.float32).copy()


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 bit patterns: nearest, ties to even.

    The low 16 bits of the binary32 pattern are the part of the significand that
    bf16 drops.  Keep the high half, then add one unit in its last place when the
    dropped part exceeds half a unit, or equals half a unit and the kept part is
    odd.  Finite inputs only.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    hi = u // 65536
    lo = u % 65536
    up = (lo > 32768) | ((lo == 32768) & (hi % 2 == 1))
    return (hi + up.astype(np.uint64)).astype(np.uint16)


def _e4m3_table() -> np.ndarray:
    """Value of each of the 256 codes (NaN for 0x7F / 0xFF)."""
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 15 and m == 7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = s * m * 2.0 ** -9
        else:
            vals[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_VALUES = _e4m3_table()
# non-negative finite codes sorted by value (codes 0..126 are already increasing)
_POS_CODES = np.arange(0, 127, dtype=np.int64)
_POS_VALS = E4M3_VALUES[:127]


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code (ties to the even code), saturating at +-448. Finite x."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS_VALS, a, side="left")          # first value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS_VALS[lo]
    dhi = _POS_VALS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(a == _POS_VALS[hi], _POS_CODES[hi], code)
    neg = np.signbit(x) & (code != 0)
    return (code + np.where(neg, 128, 0)).astype(np.uint8)


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """x rounded to the nearest E4M3 value (saturating), as float64."""
    return e4m3_decode(e4m3_encode(x))
