"""Element and scale formats of NVFP4, decoded from their bit definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

E2M1 (OCP Microscaling Formats v1.0, FP4 element type): 1 sign bit, 2 exponent
bits, 1 mantissa bit, exponent bias 1, no Inf/NaN.  The pages fix only its
largest magnitude, 6, through the divisor 6*448 of the activation global scale
(DSV4 audit page, section P0).

E4M3 "FN" (OCP 8-bit Floating Point Specification): 1 sign bit, 4 exponent
bits, 3 mantissa bits, bias 7, no infinities, S.1111.111 is NaN, largest finite
value 448.  The 448 in the same divisor pins this variant (the FNUZ variant
used by older AMD parts tops out at 240).
"""
import numpy as np


def e2m1_value(code):
    """Real value of a 4-bit E2M1 code (0..15), from the bit fields."""
    code = int(code)
    if not 0 <= code <= 15:
        raise ValueError("E2M1 code out of range")
    sign = -1.0 if code & 0x8 else 1.0
    exp = (code >> 1) & 0x3
    man = code & 0x1
    if exp == 0:                       # subnormal: 0.m * 2^(1 - bias)
        mag = (man / 2.0) * 2.0 ** (1 - 1)
    else:                              # normal: 1.m * 2^(exp - bias)
        mag = (1.0 + man / 2.0) * 2.0 ** (exp - 1)
    return sign * mag


def e4m3_value(code):
    """Real value of an 8-bit E4M3 (FN) code (0..255); NaN for S.1111.111."""
    code = int(code)
    if not 0 <= code <= 255:
        raise ValueError("E4M3 code out of range")
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:                       # subnormal: 0.mmm * 2^(1 - bias)
        mag = (man / 8.0) * 2.0 ** (1 - 7)
    else:
        mag = (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return sign * mag


# Decode tables (float64).  Every entry is exact in float64.
E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)

# Non-negative magnitudes in increasing order: E2M1 codes 0..7, E4M3 codes 0..0x7E.
E2M1_MAGS = E2M1_TABLE[:8].copy()
E4M3_MAX_CODE = 0x7E
E4M3_MAGS = E4M3_TABLE[:E4M3_MAX_CODE + 1].copy()

E2M1_MAX = float(E2M1_MAGS[-1])        # 6
E4M3_MAX = float(E4M3_MAGS[-1])        # 448

# Midpoints between neighbouring magnitudes.  The round-to-nearest decision
# between codes c and c+1 is taken against mids[c]; on an exact tie the code
# with an even mantissa (even code index) wins.
E2M1_MIDS = (E2M1_MAGS[:-1] + E2M1_MAGS[1:]) / 2.0      # 0.25 0.75 1.25 1.75 2.5 3.5 5
E4M3_MIDS = (E4M3_MAGS[:-1] + E4M3_MAGS[1:]) / 2.0
