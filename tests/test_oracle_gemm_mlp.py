"""Pins of the oracle's contraction, GLU, MLP, stacked and grouped paths."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy.special import expit

from oracle import gemm as ogemm
from oracle import mlp as omlp
from oracle import quant
from synthetic import bf16_bits_to_f32, bf16_normal
from tests import exact_ref


def _q(seed, shape, sigma=1.0):
    return quant.quantize(bf16_bits_to_f32(bf16_normal(seed, shape, sigma)))


@pytest.mark.parametrize("m,k,n", [(1, 16, 1), (3, 32, 5), (4, 64, 8), (2, 48, 3)])
def test_gemm_matches_fraction_bruteforce(m, k, n):
    xa = bf16_bits_to_f32(bf16_normal(100 + m, (m, k)))
    xb = bf16_bits_to_f32(bf16_normal(200 + n, (n, k), 0.02))
    a, b = quant.quantize(xa), quant.quantize(xb)
    ca, sa, ga = exact_ref.quantize(xa)
    cb, sb, gb = exact_ref.quantize(xb)
    exact = exact_ref.gemm(exact_ref.dequant(ca, sa, ga), exact_ref.dequant(cb, sb, gb))
    got = ogemm.gemm(a, b)
    assert got.shape == (m, n)
    for i in range(m):
        for j in range(n):
            # one float64 rounding of the exact value
            assert got[i, j] == float(exact[i][j]), (i, j)
    # the accumulation itself is exact
    acc = ogemm.gemm_acc(a, b)
    for i in range(m):
        for j in range(n):
            assert Fraction(acc[i, j]) == exact[i][j] / (ga * gb)


def test_gemm_integer_path_equals_float_path():
    a = _q(7, (5, 256))
    b = _q(8, (6, 256), 0.02)
    ea, eb = quant.expand(a), quant.expand(b)
    ai = np.rint(ea * 1024).astype(np.int64)
    bi = np.rint(eb * 1024).astype(np.int64)
    ref = (ai @ bi.T).astype(np.float64) / 2 ** 20
    assert np.array_equal(ogemm.gemm_acc(a, b), ref)
    # force the large-magnitude branch: expanded values near the top of the range
    big = quant.NVFP4(np.full((2, 4096), 0x77, np.uint8), np.full((2, 512), 0x7E, np.uint8),
                      np.float32(1.0), 2, 8192)
    acc = ogemm.gemm_acc(big, big)
    assert acc[0, 0] == 8192 * 2688.0 ** 2


def test_gemm_identity_weight_returns_dequantised_input():
    k = 64
    x = bf16_bits_to_f32(bf16_normal(31, (3, k)))
    xq = quant.quantize(x)
    wq = quant.quantize(np.eye(k, dtype=np.float32))
    # each weight row holds a single 1.0, quantised to code 6 with scale 448 and gs = RN32(1/2688)
    c = 6.0 * 448.0 * np.float64(wq.gs)
    assert np.array_equal(ogemm.gemm(xq, wq), quant.dequantize(xq) * c)


def test_gemm_operand_orientation():
    # C = A . B^T with A [M,K], B [N,K]: a rank-one check catches a transposed operand
    k = 32
    a = np.zeros((2, k), np.float32); a[0, 3] = 1.0; a[1, 17] = 1.0
    b = np.zeros((3, k), np.float32); b[2, 17] = 1.0; b[0, 3] = 1.0
    c = ogemm.gemm(quant.quantize(a), quant.quantize(b))
    nz = np.argwhere(c != 0).tolist()
    assert nz == [[0, 0], [1, 2]]


def test_silu_identities_and_library_agreement():
    g = np.linspace(-30, 30, 2001)
    s = omlp.silu(g)
    assert omlp.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(s - omlp.silu(-g), g, rtol=1e-13, atol=1e-13)   # g*sig(g) + g*sig(-g) = g
    np.testing.assert_allclose(s, g * expit(g), rtol=1e-14, atol=1e-300)
    assert omlp.silu(np.array([-1e4]))[0] == 0.0
    assert omlp.silu(np.array([1e4]))[0] == 1e4


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(100000) * 10.0 ** rng.uniform(-5, 5, 100000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(omlp.bf16_round(x), ref)


def _bruteforce_mlp(x, wg, wu, wd):
    """Scalar Python MLP on Fractions (quantise, exact GEMMs), math.exp for SiLU."""
    cx, sx, gx = exact_ref.quantize(x)
    X = exact_ref.dequant(cx, sx, gx)
    Wg = exact_ref.dequant(*exact_ref.quantize(wg))
    Wu = exact_ref.dequant(*exact_ref.quantize(wu))
    G = exact_ref.gemm(X, Wg)
    U = exact_ref.gemm(X, Wu)
    H = np.array([[float(g) / (1.0 + math.exp(-float(g))) * float(u) for g, u in zip(gr, ur)]
                  for gr, ur in zip(G, U)])
    h32 = H.astype(np.float32)
    ch, sh, gh = exact_ref.quantize(h32)
    Hq = exact_ref.dequant(ch, sh, gh)
    Wd = exact_ref.dequant(*exact_ref.quantize(wd))
    Y = exact_ref.gemm(Hq, Wd)
    return H, (ch, sh, gh), np.array([[float(v) for v in r] for r in Y])


def test_mlp_matches_scalar_bruteforce():
    t, k, i = 3, 32, 48
    x = bf16_bits_to_f32(bf16_normal(41, (t, k)))
    wg = bf16_bits_to_f32(bf16_normal(42, (i, k), 0.02))
    wu = bf16_bits_to_f32(bf16_normal(43, (i, k), 0.02))
    wd = bf16_bits_to_f32(bf16_normal(44, (k, i), 0.02))
    out = omlp.mlp(x, quant.quantize(wg), quant.quantize(wu), quant.quantize(wd))
    H, (ch, sh, gh), Y = _bruteforce_mlp(x, wg, wu, wd)
    np.testing.assert_allclose(out["h"], H, rtol=1e-14, atol=0)
    assert Fraction(float(out["hq"].gs)) == gh
    assert np.array_equal(out["hq"].scales, sh)
    assert np.array_equal(quant.unpack_codes(out["hq"].codes), ch)
    np.testing.assert_allclose(out["y"], Y, rtol=1e-15, atol=0)


def test_gate_and_up_are_not_interchangeable():
    # SiLU applies to the gate projection only: swapping the two changes H
    t, k, i = 2, 32, 16
    x = bf16_bits_to_f32(bf16_normal(51, (t, k)))
    wg = quant.quantize(bf16_bits_to_f32(bf16_normal(52, (i, k), 0.02)))
    wu = quant.quantize(bf16_bits_to_f32(bf16_normal(53, (i, k), 0.02)))
    xq = quant.quantize(x)
    h1, _ = omlp.mlp_gu_act(xq, wg, wu)
    h2, _ = omlp.mlp_gu_act(xq, wu, wg)
    assert not np.allclose(h1, h2)
    g = ogemm.gemm(xq, wg)
    u = ogemm.gemm(xq, wu)
    np.testing.assert_allclose(h1, g * expit(g) * u, rtol=1e-13)


def test_stacked_layers_chain_bf16_and_ubatches_are_independent():
    k, i = 32, 48
    x = bf16_bits_to_f32(bf16_normal(61, (8, k)))
    layers = [tuple(quant.quantize(bf16_bits_to_f32(bf16_normal(62 + 3 * l + j, shp, 0.02)))
                    for j, shp in enumerate([(i, k), (i, k), (k, i)])) for l in range(2)]
    y, chained = omlp.stacked_mlp(x, layers, ubatch=4)
    for u0 in (0, 4):
        cur = x[u0:u0 + 4]
        for li, (wg, wu, wd) in enumerate(layers):
            yl = omlp.mlp(cur, wg, wu, wd)["y"]
            cur = torch.from_numpy(yl.astype(np.float32)).to(torch.bfloat16).float().numpy()
            assert np.array_equal(chained[li][u0:u0 + 4], cur)
        assert np.array_equal(y[u0:u0 + 4], yl)
    # a different ubatch split changes the per-call global scales, hence (generally) the result
    y_one, _ = omlp.stacked_mlp(x, layers, ubatch=8)
    assert y_one.shape == y.shape


def test_grouped_single_expert_equals_dense_and_permutes():
    t, k, i = 6, 32, 16
    x = bf16_bits_to_f32(bf16_normal(71, (t, k)))
    xq = quant.quantize(x)
    w = [quant.quantize(bf16_bits_to_f32(bf16_normal(72 + j, s, 0.02))) for j, s in
         enumerate([(i, k), (i, k), (k, i)])]
    dense = omlp.mlp(x, *w)
    g = omlp.grouped_mlp(xq, np.arange(t), [0, t], [w[0]], [w[1]], [w[2]])
    assert np.array_equal(g["y"], dense["y"])
    perm = np.array([3, 0, 5, 1, 4, 2])
    gp = omlp.grouped_mlp(xq, perm, [0, t], [w[0]], [w[1]], [w[2]])
    assert np.array_equal(gp["y"], dense["y"][perm])


def test_grouped_experts_use_their_own_weights():
    t, k, i, e = 10, 32, 16, 3
    x = bf16_bits_to_f32(bf16_normal(81, (t, k)))
    xq = quant.quantize(x)
    W = [[quant.quantize(bf16_bits_to_f32(bf16_normal(90 + 3 * ex + j, s, 0.02))) for j, s in
          enumerate([(i, k), (i, k), (k, i)])] for ex in range(e)]
    a_rows = np.array([0, 2, 4, 6, 8, 1, 3, 5, 7, 9])
    offsets = [0, 4, 4, 10]              # expert 1 is empty
    g = omlp.grouped_mlp(xq, a_rows, offsets, [w[0] for w in W], [w[1] for w in W], [w[2] for w in W])
    # gate/up of each expert on its own slots
    for ex, (s0, s1) in enumerate(zip(offsets[:-1], offsets[1:])):
        if s1 > s0:
            hh, _ = omlp.mlp_gu_act(xq.take_rows(a_rows[s0:s1]), W[ex][0], W[ex][1])
            assert np.array_equal(g["h"][s0:s1], hh)
            assert np.array_equal(g["y"][s0:s1], ogemm.gemm(g["hq"].take_rows(np.arange(s0, s1)), W[ex][2]))
    # one requantisation over all slots
    assert g["hq"].gs == quant.global_scale(g["h"].astype(np.float32))
