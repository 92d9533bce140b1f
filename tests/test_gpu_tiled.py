"""Tile-contiguous weight copies (nvfp4_tile_weight).

- The copy is the permutation the header defines, bit for bit: blocks of 128
  rows x 128 K, the block's 16-byte code units in the order the large-batch
  contraction stages them in LDS (unit u of row r at r*4 + (u ^ ((r/4) % 4))),
  then its rows' 8 scale bytes; rows past N zero.  The expected bytes are
  built here with numpy from the row-major codes and scales.
- Every contraction call gives bit-identical outputs with and without the copy
  (the copy changes where the weights are staged from, not the arithmetic or
  its order): dense store and split-K store, gate/up with requantisation, the
  whole-MLP call, the static-scale pair, the expert-grouped GEMMs, and the
  decode sizes (whose weight streams ignore the copy).
- One MLP with tiled weights staged against the oracle directly.
"""
import dataclasses

import numpy as np
import pytest
import torch

from synthetic import bf16_normal
from tests.gpu_util import announce, dev_bf16, dev_quantize, require_gpu
from tests.test_gpu_mlp import _weights, check_mlp

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


def _tiled(w):
    """The same weight (shared codes and scales) with its tiled copy written."""
    t = dataclasses.replace(w, tiled=None)
    t.tile()
    return t


def _expected_tiles(codes, scales, e, n, k):
    """The tiled layout of [E][N][K] codes/scales (numpy uint8), per the header."""
    g, cn = (n + 127) // 128, k // 128
    c = np.zeros((e, g * 128, k // 2), np.uint8)
    s = np.zeros((e, g * 128, k // 16), np.uint8)
    c[:, :n] = codes.reshape(e, n, k // 2)
    s[:, :n] = scales.reshape(e, n, k // 16)
    c = c.reshape(e, g, 128, cn, 4, 16).transpose(0, 1, 3, 2, 4, 5)          # [e, g, chunk, row, unit, 16]
    r = np.arange(128)[:, None]
    src_unit = np.arange(4)[None, :] ^ ((r >> 2) & 3)                        # position p holds unit p ^ swz(r)
    c = np.take_along_axis(c, np.broadcast_to(src_unit[None, None, None, :, :, None], c.shape), axis=4)
    s = s.reshape(e, g, 128, cn, 8).transpose(0, 1, 3, 2, 4)                 # [e, g, chunk, row, 8]
    blocks = np.concatenate([c.reshape(e, g, cn, 8192), s.reshape(e, g, cn, 1024)], axis=3)
    return blocks.reshape(-1)


LAYOUTS = [(1, 200, 384), (3, 256, 256), (1, 17408, 5120)]


@pytest.mark.parametrize("e,n,k", LAYOUTS, ids=[f"E{e}_N{n}_K{k}" for e, n, k in LAYOUTS])
def test_tile_layout_bit_exact(e, n, k):
    import mlp_prefill_amd as m
    announce(f"tile layout E={e} N={n} K={k}")
    ws = [dev_quantize(bf16_normal(910 + x, (n, k), sigma=0.02)) for x in range(e)]
    w = m.NVFP4.stack(ws) if e > 1 else ws[0]
    t = _tiled(w)
    torch.cuda.synchronize()
    got = t.tiled.cpu().numpy()
    want = _expected_tiles(w.codes.cpu().numpy(), w.scales.cpu().numpy(), e, n, k)
    assert got.size == want.size == m.tile_weight_bytes(n, k, e)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:5].tolist()}"


def _same(a, b, what):
    assert torch.equal(a, b), f"{what}: outputs differ with the tiled weights"


# large batches (unsplit, split K, the 1024-token down projection) and the
# 3-16 token stream (ragged N, 8 and 16 staged token rows, split K)
GEMMS = [(96, 200, 1024), (64, 512, 8192), (1024, 5120, 17408), (5, 100, 4352), (12, 200, 5120), (16, 96, 17408),
         (3, 5120, 17408),
         # a 256-wide store tile whose second 128-row group does not exist (clamped, never stored)
         (96, 100, 1024)]


@pytest.mark.parametrize("mm,n,k", GEMMS, ids=[f"{mm}x{n}x{k}" for mm, n, k in GEMMS])
def test_gemm_tiled_bit_identical(mm, n, k):
    """Dense store contraction: unsplit, split K (64 x 512 x 8192), the
    1024-token down-projection shape (4 splits), and the 3-16 token stream;
    float32 and bf16 outputs."""
    import mlp_prefill_amd as m
    announce(f"gemm tiled vs row-major {mm}x{n}x{k}")
    a = dev_quantize(bf16_normal(920, (mm, k)))
    b = dev_quantize(bf16_normal(921, (n, k), sigma=0.02))
    bt = _tiled(b)
    for dt in (torch.float32, torch.bfloat16):
        if dt == torch.bfloat16 and n % 8:
            continue
        c0 = torch.empty((mm, n), dtype=dt, device="cuda")
        c1 = torch.empty((mm, n), dtype=dt, device="cuda")
        m.nvfp4_gemm(a, b, c0)
        m.nvfp4_gemm(a, bt, c1)
        torch.cuda.synchronize()
        _same(c0, c1, f"gemm {dt}")


def _nvfp4_same(x, y, what):
    torch.cuda.synchronize()
    for f in ("codes", "scales", "gscale"):
        _same(getattr(x, f), getattr(y, f), f"{what} {f}")


MLPS = [(64, 256, 384), (300, 512, 640), (1024, 5120, 17408), (1, 5120, 17408), (5, 5120, 17408),
        (8, 3072, 1024), (12, 5120, 640), (16, 2304, 384), (3, 1024, 256)]


@pytest.mark.parametrize("t,k,i", MLPS, ids=[f"T{t}_K{k}_I{i}" for t, k, i in MLPS])
def test_mlp_tiled_bit_identical(t, k, i):
    """The separate calls (gate/up with its float32 H, requantisation, down)
    and the whole-MLP call give the same bits with the tiled weights."""
    import mlp_prefill_amd as m
    announce(f"mlp tiled vs row-major T={t} K={k} I={i}")
    wdev, _ = _weights(k, i, (930, 931, 932)) if k < 5120 else (None, None)
    if wdev is None:
        wdev = [dev_quantize(bf16_normal(930 + j, shp, sigma=0.02)) for j, shp in enumerate([(i, k), (i, k), (k, i)])]
    wt = [_tiled(w) for w in wdev]
    x = dev_bf16(bf16_normal(933, (t, k)))
    outs = []
    for w in (wdev, wt):
        xq, hq = m.NVFP4.empty(t, k), m.NVFP4.empty(t, i)
        m.nvfp4_quantize_act(x, xq)
        ws = m.nvfp4_mlp_gu_act(xq, w[0], w[1], hq)
        y = torch.empty((t, k), dtype=torch.float32, device="cuda")
        m.nvfp4_mlp_down(hq, w[2], y)
        xq2, hq2 = m.NVFP4.empty(t, k), m.NVFP4.empty(t, i)
        y2 = torch.empty((t, k), dtype=torch.bfloat16, device="cuda")
        m.nvfp4_mlp(x, w[0], w[1], w[2], xq2, hq2, y2)
        torch.cuda.synchronize()
        outs.append((ws[: t * i * 4].clone(), hq, y, hq2, y2))
    (h0, hq0, y0, hqa, ya), (h1, hq1, y1, hqb, yb) = outs
    _same(h0, h1, "float32 H")
    _nvfp4_same(hq0, hq1, "H~")
    _same(y0, y1, "y (separate calls)")
    _nvfp4_same(hqa, hqb, "H~ (whole-MLP call)")
    _same(ya, yb, "y (whole-MLP call)")


@pytest.mark.parametrize("t", [5, 64])
def test_static_pair_tiled_bit_identical(t):
    import mlp_prefill_amd as m
    k, i = 256, 384
    announce(f"static-scale pair tiled vs row-major T={t} K={k} I={i}")
    wdev, _ = _weights(k, i, (940, 941, 942))
    wt = [_tiled(w) for w in wdev]
    xq = dev_quantize(bf16_normal(943, (t, k)))
    res = []
    for w in (wdev, wt):
        hq, yq = m.NVFP4.empty(t, i), m.NVFP4.empty(t, k)
        hq.gscale.fill_(0.003)
        yq.gscale.fill_(0.002)
        m.nvfp4_mlp_gu_act_static(xq, w[0], w[1], hq)
        m.nvfp4_mlp_down_quant(hq, w[2], yq)
        res.append((hq, yq))
    _nvfp4_same(res[0][0], res[1][0], "static H~")
    _nvfp4_same(res[0][1], res[1][1], "static y~")


def test_grouped_tiled_bit_identical():
    """Expert stacks: the GLU epilogue (requantised), the static-scale GLU
    epilogue and the store epilogue with a split K, 3 experts, one empty."""
    import mlp_prefill_amd as m
    announce("grouped gemm tiled vs row-major, 3 experts")
    e, t, k, n = 3, 40, 4096, 256
    offs = torch.tensor([0, 30, 30, 70], dtype=torch.int32, device="cuda")
    rows = torch.tensor([(5 * s) % t for s in range(70)], dtype=torch.int32, device="cuda")
    xq = dev_quantize(bf16_normal(950, (t, k)))
    g = m.NVFP4.stack([dev_quantize(bf16_normal(951 + x, (n, k), sigma=0.02)) for x in range(e)])
    u = m.NVFP4.stack([dev_quantize(bf16_normal(955 + x, (n, k), sigma=0.02)) for x in range(e)])
    gt, ut = _tiled(g), _tiled(u)
    res = []
    for wg, wu in ((g, u), (gt, ut)):
        hq = m.NVFP4.empty(70, n)
        m.nvfp4_grouped_gemm(xq, rows, offs, wg, wu, out_q=hq, epilogue=m.EPI_SILU_MUL_REQUANT, m=70)
        hs = m.NVFP4.empty(70, n)
        hs.gscale.fill_(0.003)
        m.nvfp4_grouped_gemm(xq, rows, offs, wg, wu, out_q=hs, epilogue=m.EPI_SILU_MUL_QUANT_GIVEN, m=70)
        y = torch.empty((70, n), dtype=torch.float32, device="cuda")
        m.nvfp4_grouped_gemm(xq, rows, offs, wg, out=y)
        torch.cuda.synchronize()
        res.append((hq, hs, y))
    _nvfp4_same(res[0][0], res[1][0], "grouped H~")
    _nvfp4_same(res[0][1], res[1][1], "grouped static H~")
    _same(res[0][2], res[1][2], "grouped store")


def test_mlp_tiled_against_oracle():
    announce("mlp with tiled weights vs the oracle, T=129 K=384 I=640")
    wdev, wref = _weights(384, 640, (960, 961, 962))
    check_mlp(bf16_normal(963, (129, 384)), [_tiled(w) for w in wdev], wref, "tiled T129")
