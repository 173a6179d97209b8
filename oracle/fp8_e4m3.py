"""OCP FP8 E4M3FN codec, from the format definition.  Oracle (test infrastructure).

Why FP8 at all: the dpshk.com PagedAttention article ("企业官网建设流程全解析"),
section 3.2, lists FP8 quantised storage of KV blocks as a memory optimisation.
The pages do not say which FP8 format; this library reads it as OCP E4M3FN, the
native FP8 of the target GPU (the OCP 8-bit floating point specification,
format E4M3):

* 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
* exponent field 0 encodes subnormals  m/8 * 2**-6;
* otherwise the value is (1 + m/8) * 2**(e - 7);
* S.1111.111 (0x7F, 0xFF) is NaN; there is no infinity; the largest finite
  magnitude is S.1111.110 = 448.

Encoding rounds to the nearest representable value, ties to the code whose
mantissa LSB is 0 (round-half-to-even), saturates every magnitude above 448
(including infinity) to 448, and maps NaN to 0x7F.  The encoder is a nearest
search over the 127 non-negative finite values, so it is correct by
construction rather than by bit tricks.
"""

import numpy as np

FP8_MAX = 448.0


def fp8_finite_values() -> np.ndarray:
    """The 127 non-negative finite E4M3FN values, indexed by code 0x00..0x7E."""
    vals = np.empty(0x7F, dtype=np.float64)
    for code in range(0x7F):
        e = code >> 3
        m = code & 0x7
        if e == 0:
            vals[code] = (m / 8.0) * 2.0 ** -6
        else:
            vals[code] = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_VALS = fp8_finite_values()


def fp8_decode(codes) -> np.ndarray:
    """uint8 codes -> float64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = (c & 0x7F).astype(np.int64)
    out = np.where(mag == 0x7F, np.nan, _VALS[np.minimum(mag, 0x7E)])
    return np.where((c & 0x80) != 0, -out, out)


def fp8_encode(x) -> np.ndarray:
    """float32 values -> uint8 E4M3FN codes (RNE, saturating, NaN -> 0x7F).

    The input is taken as float32; every float32 is exactly representable in
    float64, and the neighbour/midpoint comparisons below are exact in float64
    (the midpoint of two adjacent E4M3 values has at most 5 significant bits).
    """
    x32 = np.asarray(x, dtype=np.float32)
    a = np.abs(x32).astype(np.float64)
    nan = np.isnan(a)
    a_safe = np.where(nan, 0.0, a)

    code = np.empty(a.shape, dtype=np.int64)
    sat = a_safe >= FP8_MAX
    # Index of the first finite value >= a; a is then in (VALS[i-1], VALS[i]].
    i = np.searchsorted(_VALS, np.minimum(a_safe, FP8_MAX), side="left")
    i = np.clip(i, 0, 0x7E)
    hi = i
    lo = np.maximum(i - 1, 0)
    exact = _VALS[hi] == a_safe
    mid = (_VALS[lo] + _VALS[hi]) / 2.0
    below = a_safe < mid
    above = a_safe > mid
    tie_pick = np.where(lo % 2 == 0, lo, hi)  # even mantissa LSB == even code
    pick = np.where(below, lo, np.where(above, hi, tie_pick))
    code[...] = np.where(exact, hi, pick)
    code = np.where(sat, 0x7E, code)
    code = np.where(np.signbit(x32), code | 0x80, code)
    code = np.where(nan, 0x7F, code)
    return code.astype(np.uint8)
