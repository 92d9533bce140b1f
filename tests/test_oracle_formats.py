"""Pins of the oracle's format tables against the published format definitions."""
import math

import numpy as np
import torch

from oracle import formats
from tests import exact_ref


def test_e2m1_table_matches_ocp_mx_golden():
    golden = exact_ref.load_table("e2m1_ocp_mx.txt")
    assert sorted(golden) == list(range(16))
    for code, val in golden.items():
        got = formats.E2M1_TABLE[code]
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code


def test_e4m3_table_matches_ocp_ofp8_golden():
    for code, val in exact_ref.load_table("e4m3_ocp_ofp8.txt").items():
        got = formats.E4M3_TABLE[code]
        if math.isnan(val):
            assert math.isnan(got), code
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), code


def test_e4m3_table_matches_torch_float8_e4m3fn_all_codes():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = formats.E4M3_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))
    assert nan.sum() == 2                        # 0x7F and 0xFF


def test_magnitude_grids_strictly_increasing_and_sized():
    assert len(formats.E2M1_MAGS) == 8 and np.all(np.diff(formats.E2M1_MAGS) > 0)
    assert len(formats.E4M3_MAGS) == 127 and np.all(np.diff(formats.E4M3_MAGS) > 0)
    assert formats.E2M1_MAX * formats.E4M3_MAX == 2688.0
    assert list(formats.E2M1_MIDS) == [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]


def test_sign_symmetry():
    for c in range(8):
        assert formats.E2M1_TABLE[c | 8] == -formats.E2M1_TABLE[c] or (c == 0)
    for c in range(0x7F):
        assert formats.E4M3_TABLE[c | 0x80] == -formats.E4M3_TABLE[c] or c == 0


def test_midpoints_have_few_significant_bits():
    # the exactness argument of the quantiser needs <= 5 significant bits per midpoint
    def sig_bits(v):
        m, e = math.frexp(v)
        bits = 0
        while m != int(m):
            m *= 2
            bits += 1
        return bits
    assert max(sig_bits(v) for v in formats.E4M3_MIDS) <= 5
    assert max(sig_bits(v) for v in formats.E2M1_MIDS) <= 3
