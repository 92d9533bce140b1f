"""Pins of the oracle's static-global-scale MLP and its NVFP4-emitting down
projection (DSV4 audit page, section P0 fix 1 and section P8 item 1)."""
import math

import numpy as np

from oracle import mlp as omlp
from oracle import quant
from synthetic import bf16_bits_to_f32, bf16_normal
from tests import exact_ref


def _w(seed, shape):
    return quant.quantize(bf16_bits_to_f32(bf16_normal(seed, shape, 0.02)))


def _codes_scales_equal(q, ref_codes, ref_scales):
    assert np.array_equal(quant.unpack_codes(q.codes), ref_codes)
    assert np.array_equal(q.scales, ref_scales)


def test_static_with_the_dynamic_scales_is_the_dynamic_mlp():
    t, k, i = 4, 64, 48
    x = bf16_bits_to_f32(bf16_normal(71, (t, k)))
    wg, wu, wd = _w(72, (i, k)), _w(73, (i, k)), _w(74, (k, i))
    dyn = omlp.mlp(x, wg, wu, wd)
    gs_x, gs_h = omlp.warmup_scales(x, wg, wu)      # warm-up on the same batch
    st = omlp.mlp_static(x, wg, wu, wd, gs_x, gs_h)
    for key in ("xq", "hq"):
        assert np.array_equal(st[key].codes, dyn[key].codes)
        assert np.array_equal(st[key].scales, dyn[key].scales)
        assert st[key].gs == dyn[key].gs
    assert np.array_equal(st["y"], dyn["y"])


def test_static_mlp_matches_scalar_bruteforce_with_given_scales():
    """Fractions + nearest-representable search, with scales that differ from
    the batch's own (a warm-up on another batch), including saturated blocks."""
    t, k, i = 3, 32, 32
    x = bf16_bits_to_f32(bf16_normal(81, (t, k)))
    xw = bf16_bits_to_f32(bf16_normal(82, (t, k))) * np.float32(0.25)   # a quieter warm-up batch
    wg_f = bf16_bits_to_f32(bf16_normal(83, (i, k), 0.02))
    wu_f = bf16_bits_to_f32(bf16_normal(84, (i, k), 0.02))
    wd_f = bf16_bits_to_f32(bf16_normal(85, (k, i), 0.02))
    wg, wu, wd = quant.quantize(wg_f), quant.quantize(wu_f), quant.quantize(wd_f)
    gs_x, gs_h = omlp.warmup_scales(xw, wg, wu)
    out = omlp.mlp_static(x, wg, wu, wd, gs_x, gs_h)

    cx, sx, _ = exact_ref.quantize(x, gs=gs_x)
    assert (sx == 0x7E).any()                       # the quieter warm-up makes some blocks saturate
    _codes_scales_equal(out["xq"], cx, sx)
    X = exact_ref.dequant(cx, sx, exact_ref.Fraction(float(gs_x)))
    Wg = exact_ref.dequant(*exact_ref.quantize(wg_f))
    Wu = exact_ref.dequant(*exact_ref.quantize(wu_f))
    G, U = exact_ref.gemm(X, Wg), exact_ref.gemm(X, Wu)
    H = np.array([[float(g) / (1.0 + math.exp(-float(g))) * float(u) for g, u in zip(gr, ur)]
                  for gr, ur in zip(G, U)])
    np.testing.assert_allclose(out["h"], H, rtol=1e-14, atol=0)
    ch, sh, gh = exact_ref.quantize(H.astype(np.float32), gs=gs_h)
    _codes_scales_equal(out["hq"], ch, sh)
    Y = exact_ref.gemm(exact_ref.dequant(ch, sh, gh), exact_ref.dequant(*exact_ref.quantize(wd_f)))
    np.testing.assert_allclose(out["y"], np.array([[float(v) for v in r] for r in Y]), rtol=1e-15, atol=0)


def test_saturation_closed_form():
    # every |h| far above 6 * 448 * gs: block scales 448 (0x7E) and codes +-6
    h = np.array([[1.0, -2.0, 3.0, -4.0] * 4, [5.0] * 16], dtype=np.float32)
    q = quant.quantize(h, gs=np.float32(2.0 ** -20))
    assert np.all(q.scales == 0x7E)
    c = quant.unpack_codes(q.codes)
    assert np.all((c & 7) == 7)
    assert np.array_equal(c >> 3, (h < 0).astype(np.uint8))


def test_down_quant_of_a_block_permutation_reproduces_the_input():
    """An NVFP4 tensor whose every block holds a +-6 code is exactly
    re-encoded by quantising its own values with its own global scale; a down
    weight that permutes whole 16-column blocks therefore gives back the
    block-permuted input, bit for bit (a transposed weight would apply the
    inverse permutation, which differs)."""
    rng = np.random.default_rng(5)
    t, n = 4, 64
    nb = n // 16
    codes = rng.integers(0, 16, size=(t, n), dtype=np.uint8)
    codes[codes == 0x8] = 0x0     # -0 comes back as +0 (a sum of signed zeros is +0)
    for b in range(nb):
        codes[:, 16 * b + rng.integers(0, 16)] = 0x7 | (8 * rng.integers(0, 2))   # a +-6 in every block
    scales = rng.integers(0x30, 0x50, size=(t, nb), dtype=np.uint8)
    hq = quant.NVFP4(quant.pack_codes(codes), scales, np.float32(0.375), t, n)
    perm = np.array([2, 0, 3, 1])                       # output block j takes input block perm[j]
    assert not np.array_equal(np.argsort(perm), perm)   # not its own inverse
    w = np.zeros((n, n), dtype=np.float64)
    wc = np.zeros((n, n), dtype=np.uint8)
    for j, pj in enumerate(perm):
        for e in range(16):
            w[16 * j + e, 16 * pj + e] = 1.0
            wc[16 * j + e, 16 * pj + e] = 0x2                      # E2M1 code of 1.0
    wq = quant.NVFP4(quant.pack_codes(wc), np.full((n, nb), 0x38, np.uint8), np.float32(1.0), n, n)  # scale 1.0
    assert np.array_equal(quant.dequantize(wq), w)
    yq = omlp.mlp_down_quant(hq, wq, hq.gs)
    assert np.array_equal(quant.unpack_codes(yq.codes), codes.reshape(t, nb, 16)[:, perm].reshape(t, n))
    assert np.array_equal(yq.scales, scales[:, perm])
