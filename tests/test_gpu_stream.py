"""The small-batch weight streams against the oracle.

One or two tokens (K >= 1024): every split width (1 to 5 units of 1024),
split K with a partial reduction (K = 8192: 2 splits of 4 units; a prime unit
count takes splits of 2 with a shorter last one: 7168 = 3 x 2 + 1, 11264 =
5 x 2 + 1, 17408 = 8 x 2 + 1), a partial last unit (K = 1152, 1536, 2560,
4608, 8704, 9984, and 13056 = 6 x 2 + a partial unit),
ragged N (columns past N), fp32 and bf16
outputs, the gate/up GLU with its requantisation, the quantising GLU
epilogue, and per-token independence (token 0 of a 2-token call is
bit-identical to the 1-token call: the accumulation order does not depend on
the batch).  Three to sixteen tokens (16x16x32 matrix core, K a multiple of
256; 8 token rows staged up to 8 tokens, 16 above): one to seventeen K
splits, even and uneven, with the split partial sums added by the
last-arriving wave of the gate/up pair's column tiles (and by the reduction
launch for a separate store), ragged N, the same epilogues and token
independence, also across the 8- and 16-row variants.  Shapes next to those
limits (K not a multiple of 256, 17-32 tokens) take the 32-row MFMA weight
stream and are checked the same way.
"""
import numpy as np
import pytest
import torch

from oracle import gemm as ogemm
from oracle import quant
from synthetic import bf16_bits_to_f32, bf16_normal
from tests.gpu_util import (announce, assert_bf16_rounding_close, assert_nvfp4_equal, bf16_tensor_to_f32,
                            dev_quantize, max_norm_err, require_gpu, to_host)
from tests.test_gpu_mlp import _weights, check_mlp

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


def _pair(m, n, k, xs, ws):
    xb = bf16_normal(xs, (m, k))
    wb = bf16_normal(ws, (n, k), sigma=0.02)
    a, b = dev_quantize(xb), dev_quantize(wb)
    ra, rb = quant.quantize(bf16_bits_to_f32(xb)), quant.quantize(bf16_bits_to_f32(wb))
    assert_nvfp4_equal(to_host(a), ra, "A")
    assert_nvfp4_equal(to_host(b), rb, "B")
    return a, b, ra, rb


def _gemm(a, b, m, n, dtype=torch.float32):
    import mlp_prefill_amd as mm
    c = torch.empty((m, n), dtype=dtype, device="cuda")
    mm.nvfp4_gemm(a, b, c)
    torch.cuda.synchronize()
    return c.cpu().numpy() if dtype == torch.float32 else bf16_tensor_to_f32(c)


# (M, N, K): K/1024 = 1, 2, 3, 4, 5 (one split), 8 (2 splits of 4), 7, 11, 17 (splits of 2,
# the last one of 1); N multiples of 16 and ragged
STREAM_SHAPES = [(1, 64, 1024), (2, 48, 2048), (1, 200, 3072), (2, 128, 4096), (1, 96, 5120), (2, 100, 5120),
                 (1, 36, 8192), (2, 160, 7168), (1, 5120, 17408), (2, 332, 17408),
                 # K not a multiple of 1024: the last unit is partial (lanes past K read nothing)
                 (1, 5120, 8704), (2, 64, 4608), (1, 48, 2560), (2, 40, 1152), (1, 96, 9984),
                 (1, 96, 11264), (2, 48, 13056)]


@pytest.mark.parametrize("m,n,k", STREAM_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in STREAM_SHAPES])
def test_stream_gemm(m, n, k):
    announce(f"stream gemm {m}x{n}x{k}")
    a, b, ra, rb = _pair(m, n, k, 500 + m + k // 1024, 600 + n)
    ref = ogemm.gemm(ra, rb)
    y = _gemm(a, b, m, n)
    err = max_norm_err(y, ref)
    print(f"max-normalised error fp32 {err:.3e}")
    assert err <= 1e-5
    if n % 8 == 0:   # a bf16 row stride must be a multiple of 16 bytes
        y16 = _gemm(a, b, m, n, torch.bfloat16)
        print(f"max-normalised error bf16 {max_norm_err(y16, ref):.3e}")
        assert_bf16_rounding_close(y16, ref)


def test_stream_token_independence():
    """Row 0 of a two-token product equals the one-token product bit for bit."""
    announce("stream gemm token independence 2x512x17408 vs 1x512x17408")
    xb = bf16_normal(801, (2, 17408))
    wb = bf16_normal(802, (512, 17408), sigma=0.02)
    a2, b = dev_quantize(xb), dev_quantize(wb)
    # quantise the first row alone with the two-row tensor's global scale so x~ is identical
    a1 = dev_quantize(xb[:1], gs_mode=1, gs=float(a2.gscale.cpu().numpy()[0]))
    assert np.array_equal(a1.codes.cpu().numpy().reshape(-1), a2.codes.cpu().numpy().reshape(-1)[: a1.codes.numel()])
    y2 = _gemm(a2, b, 2, 512)
    y1 = _gemm(a1, b, 1, 512)
    assert np.array_equal(y1[0].view(np.uint32), y2[0].view(np.uint32))


GLU_SHAPES = [(1, 1024, 256), (2, 2048, 384), (1, 3072, 128), (2, 5120, 640), (1, 4096, 1024), (1, 4608, 1152),
              (2, 1536, 2176)]


@pytest.mark.parametrize("t,k,i", GLU_SHAPES, ids=[f"T{t}_K{k}_I{i}" for t, k, i in GLU_SHAPES])
def test_stream_mlp(t, k, i):
    """Gate/up GLU + requantisation on the weight stream, then the down
    projection (K = I is not a multiple of 1024 for most shapes: it takes the
    MFMA weight-stream kernel), staged against the oracle."""
    announce(f"stream mlp T={t} K={k} I={i}")
    wdev, wref = _weights(k, i, (900 + t, 910 + t, 920 + t))
    check_mlp(bf16_normal(930 + t, (t, k)), wdev, wref, f"stream T{t}")


@pytest.mark.parametrize("t", [1, 2])
def test_stream_glu_quant_epilogue(t):
    """The quantising GLU epilogue (static scale) on the weight stream gives
    exactly the NVFP4 encoding, under that scale, of the float32 H the
    dynamic call writes."""
    import mlp_prefill_amd as m
    k, i = 5120, 1024
    announce(f"stream gate/up quantising epilogue T={t} K={k} I={i}")
    wdev, _ = _weights(k, i, (940, 941, 942))
    xq = dev_quantize(bf16_normal(943 + t, (t, k)))
    hq = m.NVFP4.empty(t, i)
    ws = m.nvfp4_mlp_gu_act(xq, wdev[0], wdev[1], hq)
    torch.cuda.synchronize()
    h = ws[: t * i * 4].view(torch.float32).view(t, i).cpu().numpy().copy()
    for gs in (float(hq.gscale.cpu().numpy()[0]), float(hq.gscale.cpu().numpy()[0]) * 0.37):
        hs = m.NVFP4.empty(t, i)
        hs.gscale.fill_(gs)
        m.nvfp4_mlp_gu_act_static(xq, wdev[0], wdev[1], hs)
        torch.cuda.synchronize()
        ref = quant.quantize(h, gs=np.float32(gs))
        got = to_host(hs)
        assert np.array_equal(got.scales, ref.scales)
        assert np.array_equal(got.codes, ref.codes)


# ---- the 3-8 token stream (16x16x32 matrix core) ------------------------------------
# (M, N, K): K / 256 stages cut into splits of about 8 stages -- one split (768,
# 1024, 1280, 2048), even splits (3072, 4096, 6144, 7168, 8192) and uneven ones
# (2304: 5 + 4, 4352: 6 + 6 + 5, 5120: 7 + 7 + 6, 17408: 8 x 8 + 4); N multiples
# of 32 and ragged
TILE_SHAPES = [(3, 64, 1024), (4, 48, 2048), (5, 200, 3072), (8, 128, 4096), (5, 96, 5120), (6, 100, 5120),
               (7, 36, 8192), (8, 160, 7168), (8, 20, 6144), (5, 5120, 17408), (3, 332, 17408),
               (3, 48, 768), (7, 40, 1280), (8, 100, 2304), (4, 36, 4352),
               # 9-16 tokens: 16 token rows staged
               (9, 64, 1280), (12, 200, 5120), (16, 96, 2048), (16, 100, 17408), (11, 5120, 17408), (13, 36, 4352)]


@pytest.mark.parametrize("m,n,k", TILE_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in TILE_SHAPES])
def test_tile_stream_gemm(m, n, k):
    test_stream_gemm(m, n, k)


def test_tile_stream_token_independence():
    """Rows 0-2 of a 5-token product equal the 3-token product bit for bit, row
    0 of the 3-token product does not depend on rows 1-2, and rows 0-4 of a
    12-token product (16 token rows staged) equal the 5-token product (8 rows
    staged): each token is a row of the matrix-core tile, and rows past the
    batch repeat the last token."""
    announce("tile stream token independence 5/3 x 256 x 5120")
    xb = bf16_normal(811, (5, 5120))
    wb = bf16_normal(812, (256, 5120), sigma=0.02)
    a5, b = dev_quantize(xb), dev_quantize(wb)
    gs = float(a5.gscale.cpu().numpy()[0])
    a3 = dev_quantize(xb[:3], gs_mode=1, gs=gs)
    xb2 = xb[:3].copy()
    xb2[1:] = bf16_normal(813, (2, 5120))
    a3b = dev_quantize(xb2, gs_mode=1, gs=gs)
    y5, y3, y3b = _gemm(a5, b, 5, 256), _gemm(a3, b, 3, 256), _gemm(a3b, b, 3, 256)
    assert np.array_equal(y3.view(np.uint32), y5[:3].view(np.uint32))
    assert np.array_equal(y3[0].view(np.uint32), y3b[0].view(np.uint32))
    # 16 token rows staged (12 tokens) against 8 (the 5-token product): the same rows
    xb12 = np.concatenate([xb, bf16_normal(814, (7, 5120))])
    a12 = dev_quantize(xb12, gs_mode=1, gs=gs)
    y12 = _gemm(a12, b, 12, 256)
    assert np.array_equal(y12[:5].view(np.uint32), y5.view(np.uint32))


# gate/up K in 1 split (1024, 1280), 2 (3072, 4096), 3 uneven (5120), 4 (7168)
TILE_GLU = [(3, 1024, 256), (4, 3072, 128), (5, 5120, 640), (6, 7168, 384), (8, 4096, 1024), (7, 1280, 512),
            (9, 1280, 256), (12, 5120, 640), (16, 2304, 384)]


@pytest.mark.parametrize("t,k,i", TILE_GLU, ids=[f"T{t}_K{k}_I{i}" for t, k, i in TILE_GLU])
def test_tile_stream_mlp(t, k, i):
    test_stream_mlp(t, k, i)


@pytest.mark.parametrize("t", [3, 5, 8, 12, 16])
def test_tile_stream_glu_quant_epilogue(t):
    test_stream_glu_quant_epilogue(t)


# ---- batches around the stream limits: K not a multiple of 256 (3 and 12 tokens) and
# 17-32 tokens, on the 32-row MFMA weight stream ------------------------------------------
MFMA_SHAPES = [(3, 48, 640), (12, 40, 1152), (17, 64, 1024), (24, 100, 2048), (32, 96, 5120), (20, 256, 17408)]


@pytest.mark.parametrize("m,n,k", MFMA_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in MFMA_SHAPES])
def test_mfma_stream_gemm(m, n, k):
    test_stream_gemm(m, n, k)


MFMA_GLU = [(17, 1280, 256), (24, 5120, 640), (32, 2304, 384)]


@pytest.mark.parametrize("t,k,i", MFMA_GLU, ids=[f"T{t}_K{k}_I{i}" for t, k, i in MFMA_GLU])
def test_mfma_stream_mlp(t, k, i):
    test_stream_mlp(t, k, i)


@pytest.mark.parametrize("t", [17, 32])
def test_mfma_stream_glu_quant_epilogue(t):
    test_stream_glu_quant_epilogue(t)


def test_stream_launch_counts():
    """One launch set per batch: the weight streams (1-16 tokens) expand the
    activation themselves, and an activation of at most 8192 blocks is
    quantised in one launch, so a dynamic-scale MLP call with the gate/up K in
    one split is 5 launches at every such T (quantise 1, gate/up 2, down 2) and
    the static-scale pair 1 + 2; larger batches add the expansion launch of
    each projection (7 here; static 2 + 3).  A gate/up K in several splits on
    the 3-16 token stream adds the launch that clears its tickets."""
    import mlp_prefill_amd as m
    from tests.test_gpu_mlp import run_device_mlp
    k, i = 1024, 2048
    wdev, _ = _weights(k, i, (960, 961, 962))
    dyn, sta = {}, {}
    for t in (1, 2, 3, 5, 8, 9, 16, 17, 64):
        announce(f"stream launch counts T={t}")
        xbits = bf16_normal(963, (t, k))
        b0 = m.launch_count()
        run_device_mlp(xbits, wdev)
        dyn[t] = m.launch_count() - b0
        xq = dev_quantize(xbits)
        hq = m.NVFP4.empty(t, i)
        hq.gscale.fill_(0.01)
        yq = m.NVFP4.empty(t, k)
        yq.gscale.fill_(0.01)
        b0 = m.launch_count()
        m.nvfp4_mlp_gu_act_static(xq, wdev[0], wdev[1], hq)
        b1 = m.launch_count()
        m.nvfp4_mlp_down_quant(hq, wdev[2], yq)
        sta[t] = (b1 - b0, m.launch_count() - b1)
    torch.cuda.synchronize()
    assert all(dyn[t] == 5 for t in (1, 2, 3, 5, 8, 9, 16)), dyn
    assert dyn[17] == dyn[64] == 7, dyn
    assert all(sta[t] == (1, 2) for t in (1, 2, 3, 5, 8, 9, 16)), sta
    assert sta[17] == sta[64] == (2, 3), sta
    k, i = 3072, 1024                              # gate/up in 2 splits at 3-16 tokens
    wdev, _ = _weights(k, i, (964, 965, 966))
    for t, want in ((2, 5), (5, 6), (12, 6)):
        b0 = m.launch_count()
        run_device_mlp(bf16_normal(967, (t, k)), wdev)
        assert m.launch_count() - b0 == want, (t, m.launch_count() - b0)
