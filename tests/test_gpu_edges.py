"""Edge sizes, padded output strides and guard canaries around every output.

- MLP token counts next to the tile edges (2, 15, 17, 1023 tokens, and 2
  tokens on the one/two-token weight stream), staged against the oracle like
  every MLP test.
- Outputs written into the middle of larger buffers whose guard rows (and,
  for dense float outputs, padding columns past N in each row of a padded
  stride) hold a known byte pattern: after the call the guards must be intact
  and the outputs equal to those of an unguarded call bit for bit.
- Dense GEMMs whose N is not a multiple of 4 or 16 (37, 100) with a padded row
  stride, on every contraction path (one/two-token stream, 3-8 token stream,
  32-row stream, large-batch kernel), against the oracle.
"""
import numpy as np
import pytest
import torch

from oracle import gemm as ogemm
from oracle import quant
from synthetic import bf16_bits_to_f32, bf16_normal
from tests.gpu_util import (announce, assert_bf16_rounding_close, assert_nvfp4_equal, bf16_tensor_to_f32,
                            dev_bf16, dev_quantize, max_norm_err, require_gpu, to_host)
from tests.test_gpu_mlp import _weights, check_mlp, run_device_mlp

pytestmark = pytest.mark.gpu

FILL = 0xA5


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


GUARD = 256          # guard bytes on each side (keeps the output 256-byte aligned)


def guarded(nbytes):
    """A byte buffer of GUARD + nbytes + GUARD bytes filled with FILL; returns (whole, middle)."""
    whole = torch.full((nbytes + 2 * GUARD,), FILL, dtype=torch.uint8, device="cuda")
    return whole, whole[GUARD:GUARD + nbytes]


def guards_intact(whole, nbytes):
    w = whole.cpu().numpy()
    return bool(np.all(w[:GUARD] == FILL) and np.all(w[GUARD + nbytes:] == FILL))


class GuardedNVFP4:
    """NVFP4 output [rows][cols] between guards (codes, scales and gscale)."""

    def __init__(self, rows, cols):
        import mlp_prefill_amd as m
        self.nc, self.ns = rows * cols // 2, rows * cols // 16
        self.wc, vc = guarded(self.nc)
        self.ws, vs = guarded(self.ns)
        self.wg = torch.full((3,), -7.0, dtype=torch.float32, device="cuda")
        self.q = m.NVFP4(vc.view(rows, cols // 2), vs.view(rows, cols // 16), self.wg[1:2], rows, cols)

    def intact(self):
        g = self.wg.cpu().numpy()
        return guards_intact(self.wc, self.nc) and guards_intact(self.ws, self.ns) and g[0] == -7.0 and g[2] == -7.0


def guarded_dense(rows, cols, ld, dtype):
    """A float32/bf16 output [rows][cols] with row stride ld between guards; the padding columns hold FILL too."""
    esz = 4 if dtype == torch.float32 else 2
    whole, mid = guarded(rows * ld * esz)
    return whole, mid.view(rows, ld * esz).view(dtype)[:, :cols]


def dense_intact(whole, rows, cols, ld, dtype):
    esz = 4 if dtype == torch.float32 else 2
    n = rows * ld * esz
    mid = whole.cpu().numpy()[GUARD:GUARD + n].reshape(rows, ld * esz)
    return guards_intact(whole, n) and bool(np.all(mid[:, cols * esz:] == FILL))


EDGE = [(2, 512, 1024), (15, 512, 1024), (17, 512, 1024), (1023, 512, 1024), (2, 1024, 2048)]


@pytest.mark.parametrize("t,k,i", EDGE, ids=[f"T{t}_K{k}_I{i}" for t, k, i in EDGE])
def test_mlp_edge_token_counts(t, k, i):
    announce(f"mlp edge T={t} K={k} I={i}")
    wdev, wref = _weights(k, i, (500 + t, 600 + t, 700 + t))
    check_mlp(bf16_normal(800 + t, (t, k)), wdev, wref, f"edge T{t}")


@pytest.mark.parametrize("t,k,i", [(1, 5120, 2048), (5, 5120, 2048), (17, 512, 1024), (300, 512, 1024)],
                         ids=["T1_stream", "T5_stream", "T17", "T300"])
def test_mlp_outputs_between_guards(t, k, i):
    """x~, H~ (codes, scales, global scales) and y written between guards equal the unguarded call."""
    import mlp_prefill_amd as m
    announce(f"mlp guards T={t} K={k} I={i}")
    wdev, _ = _weights(k, i, (900 + t, 901 + t, 902 + t))
    xbits = bf16_normal(903 + t, (t, k))
    xq0, _, hq0, y0 = run_device_mlp(xbits, wdev)
    x = dev_bf16(xbits)
    xq, hq = GuardedNVFP4(t, k), GuardedNVFP4(t, i)
    ld = k + 16
    wy, y = guarded_dense(t, k, ld, torch.float32)
    m.nvfp4_quantize_act(x, xq.q)
    m.nvfp4_mlp_gu_act(xq.q, wdev[0], wdev[1], hq.q)
    m.nvfp4_mlp_down(hq.q, wdev[2], y)
    torch.cuda.synchronize()
    assert xq.intact() and hq.intact(), "NVFP4 output guards overwritten"
    assert dense_intact(wy, t, k, ld, torch.float32), "y guards or padding overwritten"
    assert_nvfp4_equal(to_host(xq.q), to_host(xq0), "guarded x~")
    assert_nvfp4_equal(to_host(hq.q), to_host(hq0), "guarded H~")
    assert torch.equal(y, y0)


PADDED = [(1, 37, 1024), (1, 100, 2048), (5, 37, 1024), (5, 100, 2048), (20, 37, 256), (20, 100, 384),
          (300, 37, 256), (300, 100, 512)]


@pytest.mark.parametrize("m_,n,k", PADDED, ids=[f"{m}x{n}x{k}" for m, n, k in PADDED])
def test_gemm_unaligned_n_padded_stride(m_, n, k):
    import mlp_prefill_amd as mm
    announce(f"gemm N={n} padded stride, {m_}x{n}x{k}")
    xb, wb = bf16_normal(1200 + m_, (m_, k)), bf16_normal(1300 + n, (n, k), sigma=0.02)
    a, b = dev_quantize(xb), dev_quantize(wb)
    ref = ogemm.gemm(quant.quantize(bf16_bits_to_f32(xb)), quant.quantize(bf16_bits_to_f32(wb)))
    ld = (n + 7) // 8 * 8 + 8            # rows stay 16-byte aligned for both dtypes, with spare columns
    for dt in (torch.float32, torch.bfloat16):
        whole, c = guarded_dense(m_, n, ld, dt)
        amax = mm.amax_buffer()
        mm.nvfp4_gemm(a, b, c, amax=amax if dt == torch.bfloat16 else None)
        torch.cuda.synchronize()
        assert dense_intact(whole, m_, n, ld, dt), f"{dt}: guards or padding columns overwritten"
        if dt == torch.float32:
            err = max_norm_err(c.cpu().numpy(), ref)
            print(f"N={n} fp32 error {err:.2e}")
            assert err <= 1e-5
        else:
            y = bf16_tensor_to_f32(c.contiguous())
            assert_bf16_rounding_close(y, ref)
            assert amax.max().item() == float(np.max(np.abs(y)))


def test_grouped_outputs_between_guards():
    """The expert-grouped GLU output (NVFP4) and store output (padded stride) between guards."""
    import mlp_prefill_amd as m
    t, k, i, e = 40, 256, 384, 3
    announce("grouped guards")
    xq = dev_quantize(bf16_normal(1401, (t, k)))
    w = [m.NVFP4.stack([dev_quantize(bf16_normal(1410 + 3 * x + j, shp, sigma=0.02)) for x in range(e)])
         for j, shp in enumerate([(i, k), (i, k), (k, i)])]
    a_rows = torch.tensor(list(range(0, t, 2)) + list(range(1, t, 2)) + [3, 5, 7], dtype=torch.int32, device="cuda")
    offs = torch.tensor([0, 20, 20, 43], dtype=torch.int32, device="cuda")
    ms = 43
    hq0 = m.NVFP4.empty(ms, i)
    m.nvfp4_grouped_gemm(xq, a_rows, offs, w[0], w[1], out_q=hq0, epilogue=m.EPI_SILU_MUL_REQUANT, m=ms)
    y0 = torch.empty((ms, k), dtype=torch.float32, device="cuda")
    m.nvfp4_grouped_gemm(hq0, None, offs, w[2], out=y0, epilogue=m.EPI_STORE)
    hq = GuardedNVFP4(ms, i)
    m.nvfp4_grouped_gemm(xq, a_rows, offs, w[0], w[1], out_q=hq.q, epilogue=m.EPI_SILU_MUL_REQUANT, m=ms)
    ld = k + 32
    wy, y = guarded_dense(ms, k, ld, torch.float32)
    m.nvfp4_grouped_gemm(hq.q, None, offs, w[2], out=y, epilogue=m.EPI_STORE)
    torch.cuda.synchronize()
    assert hq.intact(), "grouped H~ guards overwritten"
    assert dense_intact(wy, ms, k, ld, torch.float32), "grouped y guards or padding overwritten"
    assert_nvfp4_equal(to_host(hq.q), to_host(hq0), "grouped guarded H~")
    assert torch.equal(y, y0)
