"""Exact rational reference used to pin the oracle on tiny inputs.

Independent of `oracle/`: values come from torch's float8 decoding and the
golden E2M1 table, rounding is brute-force nearest-with-ties-to-even over
Python Fractions, and the float32 rounding is written here from scratch.
"""
import math
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_table(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if not line:
            continue
        code, val = line.split()
        out[int(code, 16)] = float(val)
    return out


E2M1 = load_table("e2m1_ocp_mx.txt")
E2M1_MAGS = [Fraction(E2M1[c]) for c in range(8)]
# E4M3 magnitudes of codes 0..126 via torch's float8_e4m3fn decoding.
E4M3_MAGS = [Fraction(float(v)) for v in
             torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).tolist()]


def f32_rne(q):
    """Round a Fraction to the nearest float32 (ties to even); returns a Fraction."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                       # subnormals share the min-normal quantum
    quantum = Fraction(2) ** (e - 23)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * quantum


def nearest_even(value, grid):
    """Index of the grid point nearest to `value`; exact ties go to the even index."""
    best = None
    for i, g in enumerate(grid):
        d = abs(g - value)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0 and best[1] % 2 == 1):
            best = (d, i)
    return best[1]


def global_scale(x):
    amax = max((abs(Fraction(float(v))) for v in np.asarray(x, dtype=np.float32).ravel()), default=Fraction(0))
    amax = max(amax, Fraction(float(np.float32(1e-8))))
    return f32_rne(amax / 2688)


def quantize(x, gs=None):
    """Brute-force NVFP4: returns (codes [rows, cols] 4-bit, scales [rows, cols/16], gs Fraction)."""
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    gs = global_scale(x) if gs is None else Fraction(float(np.float32(gs)))
    codes = np.zeros((rows, cols), dtype=np.uint8)
    scales = np.zeros((rows, cols // 16), dtype=np.uint8)
    for r in range(rows):
        for b in range(cols // 16):
            blk = [Fraction(float(v)) for v in x[r, 16 * b:16 * b + 16]]
            amax_b = max(abs(v) for v in blk)
            s = nearest_even(amax_b / (6 * gs), E4M3_MAGS)
            scales[r, b] = s
            d = E4M3_MAGS[s]
            for j, v in enumerate(blk):
                mag = 0 if d == 0 else nearest_even(abs(v) / (d * gs), E2M1_MAGS)
                neg = np.signbit(x[r, 16 * b + j])
                codes[r, 16 * b + j] = (8 if neg else 0) | mag
    return codes, scales, gs


def code_value(c):
    return Fraction(E2M1[int(c)]) if int(c) not in (0x8,) else Fraction(0)


def dequant(codes, scales, gs):
    """Exact rational dequantised matrix (list of lists of Fractions)."""
    rows, cols = codes.shape
    return [[code_value(codes[r, k]) * E4M3_MAGS[int(scales[r, k // 16])] * gs for k in range(cols)]
            for r in range(rows)]


def gemm(a_rows, b_rows):
    """Exact C = A . B^T for lists of lists of Fractions."""
    return [[sum((x * y for x, y in zip(ar, br)), Fraction(0)) for br in b_rows] for ar in a_rows]
