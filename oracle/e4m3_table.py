"""Independent E4M3 (and E5M2) value tables written from the formats' bit fields.

TEST INFRASTRUCTURE (part of the oracle): used only by the tests to pin the C
oracle's decoder and encoder from a second, separately written source.

E4M3 per "FP8量化与长上下文推理" section 1 (4 exponent bits, 3 mantissa bits,
largest value about 448) and "cooking-agi: FP8 and the KV cache", section "how
to enable it in the engine" (smallest subnormal 2^-9). Exponent bias 7, no
infinities and NaN = S.1111.111 are the OCP definition that page cites.
"""

import math

import numpy as np

BIAS = 7
MAX_FINITE = 448.0
MIN_SUBNORMAL = 2.0 ** -9


def value_of(code: int) -> float:
    """Real value of one 8-bit code, computed from its fields in Python floats."""
    sign = -1.0 if code & 0x80 else 1.0
    exp_field = (code >> 3) & 0xF
    man_field = code & 0x7
    if exp_field == 0xF and man_field == 0x7:
        return math.nan
    if exp_field == 0:
        # subnormal: 0.mmm * 2^(1 - bias)
        return sign * (man_field / 8.0) * 2.0 ** (1 - BIAS)
    return sign * (1.0 + man_field / 8.0) * 2.0 ** (exp_field - BIAS)


def table() -> np.ndarray:
    """float64[256] of every code's value (NaN for the two NaN codes)."""
    return np.array([value_of(c) for c in range(256)], dtype=np.float64)


def nearest_code(y: float) -> int:
    """Saturating round-to-nearest-even encode of one value, by brute force
    over the 127 non-negative finite values (small inputs only)."""
    sign = 0x80 if math.copysign(1.0, y) < 0 else 0
    if math.isnan(y):
        return 0x7F | sign
    a = min(abs(y), MAX_FINITE)
    vals = [value_of(c) for c in range(127)]
    dist = [abs(a - v) for v in vals]
    best = min(dist)
    cands = [c for c in range(127) if dist[c] == best]
    even = [c for c in cands if c % 2 == 0]
    return (even[0] if even else cands[0]) | sign


# ---------------------------------------------------------------------------
# E5M2, from its bit fields the same way: "FP8量化与长上下文推理" section 1
# (5 exponent bits, 2 mantissa bits, range about +-57344). Exponent bias 15,
# S.11111.00 = infinity and S.11111.xx (xx != 0) = NaN are the OCP
# definition.
# ---------------------------------------------------------------------------
E5M2_BIAS = 15
E5M2_MAX_FINITE = 57344.0
E5M2_MIN_SUBNORMAL = 2.0 ** -16


def e5m2_value_of(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    exp_field = (code >> 2) & 0x1F
    man_field = code & 0x3
    if exp_field == 0x1F:
        return math.nan if man_field else sign * math.inf
    if exp_field == 0:
        return sign * (man_field / 4.0) * 2.0 ** (1 - E5M2_BIAS)
    return sign * (1.0 + man_field / 4.0) * 2.0 ** (exp_field - E5M2_BIAS)


def e5m2_table() -> np.ndarray:
    return np.array([e5m2_value_of(c) for c in range(256)], dtype=np.float64)


def e5m2_nearest_code(y: float) -> int:
    """Saturating round-to-nearest-even e5m2 encode of one value, by brute
    force over the 124 non-negative finite values (small inputs only)."""
    sign = 0x80 if math.copysign(1.0, y) < 0 else 0
    if math.isnan(y):
        return 0x7F | sign
    a = min(abs(y), E5M2_MAX_FINITE)
    vals = [e5m2_value_of(c) for c in range(124)]
    dist = [abs(a - v) for v in vals]
    best = min(dist)
    cands = [c for c in range(124) if dist[c] == best]
    even = [c for c in cands if c % 2 == 0]
    return (even[0] if even else cands[0]) | sign
