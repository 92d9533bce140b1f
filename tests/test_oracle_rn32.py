"""Pins of the float32 rounding (RN32) that precedes every quantisation of a
contraction's output in the oracle.

The device holds the GLU output H, and the down projection's output Y, in
float32 registers; the oracle's readings are that H is quantised as RN32(H)
(requantisation straight into the down projection's NVFP4 input: llama.cpp
discussion, "What the patch does"), that a quantising down projection
quantises RN32(Y) (DSV4 audit page, section P8 item 1), and that a chained
layer's input is bf16(RN32(Y)).

Each case below is built from hand-placed NVFP4 codes and scales so that a
float64 value sits a sub-ulp distance from a rounding decision: rounding it to
float32 first lands exactly on the decision point (where ties-to-even
decides), while the float64 value itself lies strictly on one side.  The
expected codes are derived by hand in the comments; a brute-force check on
exact rationals confirms that quantising the float64 value directly would give
different codes, so a version of the oracle that skipped the RN32 step fails
here.
"""
from fractions import Fraction

import numpy as np

from oracle import mlp as omlp
from oracle import quant
from tests import exact_ref

# E4M3 codes used below: 0x01 = 2^-9, 0x08 = 2^-6, 0x20 = 0.125, 0x38 = 1.0,
# 0x40 = 2.0, 0x42 = 2.5, 0x7E = 448.  E2M1 codes: 0x1 = 0.5, 0x2 = 1.0,
# 0x3 = 1.5, 0x4 = 2.0, 0x6 = 4.0, 0x7 = 6.0, 0x9 = -0.5.
E4M3 = {0x01: 2.0 ** -9, 0x08: 2.0 ** -6, 0x20: 0.125, 0x38: 1.0, 0x40: 2.0, 0x42: 2.5, 0x7E: 448.0}
E2M1 = {0x1: 0.5, 0x2: 1.0, 0x3: 1.5, 0x4: 2.0, 0x6: 4.0, 0x7: 6.0, 0x9: -0.5}


def nvfp4(rows, cols, entries, gs=1.0):
    """NVFP4 matrix whose only non-zero elements are entries {(r, k): (e2m1 code, e4m3 scale code)};
    entries of one 16-element block must name the same scale."""
    codes = np.zeros((rows, cols), np.uint8)
    scales = np.zeros((rows, cols // 16), np.uint8)
    for (r, k), (c, s) in entries.items():
        assert scales[r, k // 16] in (0, s)
        codes[r, k] = c
        scales[r, k // 16] = s
    return quant.NVFP4(quant.pack_codes(codes), scales, np.float32(gs), rows, cols)


# x (one token, K = 48): 2688 at k=0, 224 at k=1 (block scale 448), 2^-10 at
# k=16 (block scale 2^-9), 1 and 6 at k=32, 33 (block scale 1).
X = nvfp4(1, 48, {(0, 0): (0x7, 0x7E), (0, 1): (0x1, 0x7E), (0, 16): (0x1, 0x01),
                  (0, 32): (0x2, 0x38), (0, 33): (0x7, 0x38)})
# gate rows (I = 32):
#   row 0:  2688 * 1                          = 2688            (sets amax, so gs = 1)
#   row 1:  224 * 5 + 2^-10 * 2^-10           = 1120 + 2^-20
#   row 2:  224 * 1.5 + 2^-10 * (-2^-10)      = 336 - 2^-20
#   row 16: 6 * 8 + 1 * 3 + 2^-10 * 2^-10     = 51 + 2^-20
WG = nvfp4(32, 48, {(0, 0): (0x2, 0x38),
                    (1, 1): (0x4, 0x42), (1, 16): (0x1, 0x01),
                    (2, 1): (0x3, 0x38), (2, 16): (0x9, 0x01),
                    (16, 33): (0x6, 0x40), (16, 32): (0x3, 0x40), (16, 16): (0x1, 0x01)})
# up rows: 1 for rows 0-2, 0.125 for row 16, 0 elsewhere
WU = nvfp4(32, 48, {(0, 32): (0x2, 0x38), (1, 32): (0x2, 0x38), (2, 32): (0x2, 0x38),
                    (16, 32): (0x2, 0x20)})

# For g >= 37, e^-g < 2^-53, so SiLU(g) = g / (1 + e^-g) is g exactly in float64 and
# H = SiLU(G) * U is exact:
#   H[0] = 2688, H[1] = 1120 + 2^-20, H[2] = 336 - 2^-20, H[16] = 6.375 + 2^-23.
# gs_h = RN32(2688 / 2688) = 1.
# Block 0: amax 2688 -> 2688 / 6 = 448 -> scale 0x7E.
#   RN32(H[1]) = 1120 (float32 spacing 2^-13 there); 1120 / 448 = 2.5 is the tie
#   between E2M1 2 (index 4) and 3 (index 5): the even index wins -> 2 (code 0x4).
#   In float64 the quotient exceeds 2.5 -> 3 (code 0x5).
#   RN32(H[2]) = 336; 336 / 448 = 0.75 is the tie between 0.5 (index 1) and 1 (index
#   2): the even index wins -> 1 (code 0x2).  In float64 it is below -> 0.5 (0x1).
# Block 1: RN32(H[16]) = 6.375 (float32 spacing 2^-21); 6.375 / 6 = 1.0625 is the tie
#   between E4M3 1.0 (0x38) and 1.125 (0x39): the even code wins -> 0x38.  In float64
#   it is above -> 0x39.  H[16] / 1.0 = 6.375 > 6 saturates to 6 (0x7) either way.
EXPECT_H_SCALES = [0x7E, 0x38]
EXPECT_H_CODES = {0: 0x7, 1: 0x4, 2: 0x2, 16: 0x7}


def _expected(codes_at, scales):
    c = np.zeros((1, 32), np.uint8)
    for k, v in codes_at.items():
        c[0, k] = v
    return c, np.array([scales], np.uint8)


def _f64_direct_bruteforce(v, gs):
    """NVFP4 decisions taken on the float64 values themselves (no float32 step), on exact rationals."""
    v = np.asarray(v, np.float64).reshape(1, -1)
    gs = Fraction(float(gs))
    codes = np.zeros(v.shape, np.uint8)
    scales = np.zeros((1, v.shape[1] // 16), np.uint8)
    for b in range(v.shape[1] // 16):
        blk = [Fraction(float(a)) for a in v[0, 16 * b:16 * b + 16]]
        s = exact_ref.nearest_even(max(abs(a) for a in blk) / (6 * gs), exact_ref.E4M3_MAGS)
        scales[0, b] = s
        d = exact_ref.E4M3_MAGS[s]
        for j, a in enumerate(blk):
            mag = 0 if d == 0 else exact_ref.nearest_even(abs(a) / (d * gs), exact_ref.E2M1_MAGS)
            codes[0, 16 * b + j] = (8 if a < 0 else 0) | mag
    return codes, scales


def _check(q, codes, scales):
    assert np.array_equal(q.scales, scales), (q.scales, scales)
    assert np.array_equal(quant.unpack_codes(q.codes), codes), quant.unpack_codes(q.codes)


def test_constructed_h_is_exact():
    h, _ = omlp.mlp_gu_act(X, WG, WU)
    want = np.zeros((1, 32))
    want[0, 0], want[0, 1], want[0, 2], want[0, 16] = 2688, 1120 + 2.0 ** -20, 336 - 2.0 ** -20, 6.375 + 2.0 ** -23
    assert np.array_equal(h, want)


def test_requantisation_rounds_h_to_float32_first():
    h, hq = omlp.mlp_gu_act(X, WG, WU)
    assert hq.gs == np.float32(1.0)
    codes, scales = _expected(EXPECT_H_CODES, EXPECT_H_SCALES)
    _check(hq, codes, scales)
    _check(omlp.requantize(h), codes, scales)
    # the same decisions taken on the float64 H differ at all three constructed places
    c64, s64 = _f64_direct_bruteforce(h, 1.0)
    assert s64[0, 1] == 0x39 and c64[0, 1] == 0x5 and c64[0, 2] == 0x1
    assert not np.array_equal(c64, codes) and not np.array_equal(s64, scales)


def test_static_scale_gate_up_rounds_h_to_float32_first():
    _, hq = omlp.mlp_gu_act_static(X, WG, WU, np.float32(1.0))
    codes, scales = _expected(EXPECT_H_CODES, EXPECT_H_SCALES)
    _check(hq, codes, scales)


def test_quantising_down_projection_rounds_y_to_float32_first():
    # Y = X~ . Wg~^T: Y[0] = 2688, Y[1] = 1120 + 2^-20, Y[2] = 336 - 2^-20, Y[16] = 51 + 2^-20.
    # With gs_y = 1: block 0 as for H above.  Block 1: RN32(Y[16]) = 51 (float32
    # spacing 2^-18); 51 / 6 = 8.5 is the tie between E4M3 8 (0x50) and 9 (0x51):
    # the even code wins -> 0x50, and 51 / 8 = 6.375 saturates to 6.  In float64 the
    # scale would be 0x51 and 51.000001 / 9 = 5.67 rounds to 6 as well.
    yq = omlp.mlp_down_quant(X, WG, np.float32(1.0))
    codes, scales = _expected(EXPECT_H_CODES, [0x7E, 0x50])
    _check(yq, codes, scales)
    c64, s64 = _f64_direct_bruteforce(omlp.mlp_down(X, WG), 1.0)
    assert s64[0, 1] == 0x51 and c64[0, 1] == 0x5 and c64[0, 2] == 0x1


def test_grouped_requantisation_rounds_h_to_float32_first():
    g = omlp.grouped_mlp(X, np.array([0]), [0, 1], [WG], [WU], [nvfp4(16, 32, {})])
    codes, scales = _expected(EXPECT_H_CODES, EXPECT_H_SCALES)
    _check(g["hq"], codes, scales)


def test_chained_input_is_bf16_of_float32_y():
    # y = 1 + 2^-8 + 2^-30: RN32 drops 2^-30 (below half the float32 spacing 2^-23 at 1),
    # leaving 1 + 2^-8, the exact midpoint between the bf16 neighbours 1 and 1 + 2^-7;
    # ties go to the even mantissa, 1.  Rounded directly from float64 it would be 1 + 2^-7.
    y = np.array([1.0 + 2.0 ** -8 + 2.0 ** -30])
    assert omlp.bf16_round(y)[0] == np.float32(1.0)
    direct = Fraction(1) + Fraction(1, 2 ** 7)          # nearest bf16 of the float64 value
    assert abs(Fraction(float(y[0])) - direct) < abs(Fraction(float(y[0])) - 1)
