"""Pins of the oracle's NVFP4 quantiser: closed forms, brute force, ties, invariants."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats, quant
from synthetic import bf16_bits_to_f32, bf16_normal
from tests import exact_ref


def _golden_gs_cases():
    out = []
    for line in open(f"{exact_ref.GOLDEN}/global_scale_cases.txt"):
        line = line.split("#")[0].strip()
        if line:
            a, g = line.split()
            out.append((float(a), float(g)))
    return out


@pytest.mark.parametrize("amax,gs", _golden_gs_cases())
def test_global_scale_golden(amax, gs):
    x = np.zeros((2, 32), dtype=np.float32)
    x[1, 7] = -amax
    assert quant.global_scale(x) == np.float32(gs)


def test_global_scale_matches_exact_rounding_random():
    rng = np.random.default_rng(11)
    amaxes = np.concatenate([rng.uniform(0, 10, 300), 10.0 ** rng.uniform(-12, 6, 300), [1e-9, 1e-8, 2e-8]])
    for a in amaxes.astype(np.float32):
        x = np.array([[a] + [0.0] * 15], dtype=np.float32)
        expect = exact_ref.global_scale(x)
        assert Fraction(float(quant.global_scale(x))) == expect, a


def test_global_scale_floor_for_zero_tensor():
    expect = exact_ref.f32_rne(Fraction(float(np.float32(1e-8))) / 2688)
    assert Fraction(float(quant.global_scale(np.zeros((3, 16), np.float32)))) == expect
    assert Fraction(float(quant.global_scale(np.zeros((0, 16), np.float32)))) == expect


def _check_against_bruteforce(x, gs=None):
    q = quant.quantize(x, gs)
    codes, scales, g = exact_ref.quantize(x, gs)
    assert Fraction(float(q.gs)) == g
    assert np.array_equal(q.scales, scales)
    assert np.array_equal(quant.unpack_codes(q.codes), codes)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_quantize_matches_bruteforce_normal_bf16(seed):
    x = bf16_bits_to_f32(bf16_normal(seed, (3, 48)))
    _check_against_bruteforce(x)


def test_quantize_matches_bruteforce_wide_dynamic_range():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((4, 64)) * 10.0 ** rng.uniform(-7, 2, (4, 64))).astype(np.float32)
    x[0, :16] = 0.0
    x[1, 3] = -0.0
    x[2, 16:32] *= 1e-6          # tiny block: subnormal or zero E4M3 scale
    _check_against_bruteforce(x)


def test_quantize_matches_bruteforce_given_gs_saturating():
    x = bf16_bits_to_f32(bf16_normal(9, (2, 32)))
    _check_against_bruteforce(x, gs=np.float32(1e-4))    # forces S = 448 and |codes| = 6
    q = quant.quantize(x, gs=np.float32(1e-4))
    assert np.all(q.scales == 0x7E)


def _gs_one_tensor(blocks):
    """Rows of 16-blocks plus a first block holding 2688, so gs == 1 exactly."""
    x = np.zeros((1, 16 * (len(blocks) + 1)), dtype=np.float32)
    x[0, 0] = 2688.0
    for i, b in enumerate(blocks):
        x[0, 16 * (i + 1):16 * (i + 2)] = b
    return x


def test_block_scale_ties_round_to_even():
    # amax_b / 6 exactly halfway between neighbouring E4M3 values
    b1 = np.zeros(16, np.float32); b1[0] = 6 * 1.0625      # 1.0 (0x38) | 1.125 (0x39) -> 0x38
    b2 = np.zeros(16, np.float32); b2[0] = 6 * 1.1875      # 1.125 (0x39) | 1.25 (0x3A) -> 0x3A
    b3 = np.zeros(16, np.float32); b3[0] = 6 * 1.0625 * 2 ** -3
    q = quant.quantize(_gs_one_tensor([b1, b2, b3]))
    assert q.gs == np.float32(1.0)
    assert list(q.scales[0]) == [0x7E, 0x38, 0x3A, 0x20]


def test_element_ties_round_to_even():
    # gs = 1 and a block scale of exactly 1.0 (block amax 6): thresholds are the midpoints themselves
    blk = np.array([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0,
                    -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0, 0.0], dtype=np.float32)
    q = quant.quantize(_gs_one_tensor([blk]))
    assert q.scales[0, 1] == 0x38
    mags = [0, 2, 2, 4, 4, 6, 6]            # even code index wins on each midpoint
    expect = [7] + mags + [8 | m for m in mags] + [0]
    assert list(quant.unpack_codes(q.codes)[0, 16:32]) == expect
    _check_against_bruteforce(_gs_one_tensor([blk]))


def test_just_off_ties_round_to_nearest():
    eps = np.float32(2.0 ** -20)
    blk = np.array([6.0, 0.25 + eps, 0.75 - eps, 1.25 + eps, 1.75 - eps, 2.5 + eps, 3.5 - eps, 5.0 + eps]
                   + [0.0] * 8, dtype=np.float32)
    q = quant.quantize(_gs_one_tensor([blk]))
    assert list(quant.unpack_codes(q.codes)[0, 16:24]) == [7, 1, 1, 3, 3, 5, 5, 7]


def test_invariants_random_bf16():
    x = bf16_bits_to_f32(bf16_normal(21, (64, 256)))
    q = quant.quantize(x)
    codes = quant.unpack_codes(q.codes)
    d = formats.E4M3_TABLE[q.scales.astype(int)]
    # block holding the tensor amax gets the largest scale code
    r, c = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert q.scales[r, c // 16] == 0x7E
    # in every block with a normal scale, the block's largest element codes to +-6
    xb = np.abs(x).reshape(64, 16, 16)
    arg = np.argmax(xb, axis=-1)
    top_codes = np.take_along_axis(codes.reshape(64, 16, 16), arg[..., None], -1)[..., 0]
    normal = d >= 2.0 ** -6
    assert np.all((top_codes[normal] & 7) == 7)
    # dequantised values lie on the scaled grid and within half a grid step of x
    xh = quant.dequantize(q)
    step = np.array([0.5, 0.5, 0.5, 0.5, 1.0, 1.0, 2.0, 2.0])[codes & 7]
    dd = np.repeat(d, 16, axis=1) * np.float64(q.gs)
    nrm = np.repeat(normal, 16, axis=1)
    assert np.all((np.abs(x - xh) <= step / 2 * dd)[nrm])
    assert np.all(np.signbit(xh[xh != 0]) == np.signbit(x[xh != 0]))


def test_all_zero_and_constant_tensors():
    z = np.zeros((2, 32), np.float32)
    z[1, 5] = -0.0
    q = quant.quantize(z)
    assert np.all(q.scales == 0)
    codes = quant.unpack_codes(q.codes)
    assert codes[1, 5] == 8 and np.sum(codes) == 8
    for c in (1.5, -3.0, 1e-3):
        q = quant.quantize(np.full((2, 48), c, np.float32))
        assert np.all(q.scales == 0x7E)
        assert np.all(quant.unpack_codes(q.codes) == (0xF if c < 0 else 0x7))


def test_pack_unpack_roundtrip_and_nibble_order():
    rng = np.random.default_rng(3)
    c = rng.integers(0, 16, (5, 64), dtype=np.uint8)
    p = quant.pack_codes(c)
    assert p.shape == (5, 32)
    assert np.array_equal(quant.unpack_codes(p), c)
    assert p[0, 0] == (c[0, 0] | (c[0, 1] << 4))       # element 0 in the low nibble


def test_rejects_bad_shapes_and_nonfinite():
    with pytest.raises(ValueError):
        quant.quantize(np.zeros((2, 17), np.float32))
    with pytest.raises(ValueError):
        quant.quantize(np.array([[np.inf] + [0.0] * 15], np.float32))


def test_empty_tensor():
    q = quant.quantize(np.zeros((0, 64), np.float32))
    assert q.codes.shape == (0, 32) and q.scales.shape == (0, 4)
