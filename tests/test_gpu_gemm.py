"""Device NVFP4 GEMM vs the oracle's exact-accumulation GEMM."""
import numpy as np
import pytest
import torch

from oracle import gemm as ogemm
from oracle import quant
from synthetic import WORKLOADS, bf16_bits_to_f32, bf16_normal
from tests.gpu_util import (announce, assert_bf16_rounding_close, assert_nvfp4_equal, bf16_tensor_to_f32,
                            dev_quantize, max_norm_err, require_gpu, to_host)

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


def _run(a, b, m, n, dtype):
    import mlp_prefill_amd as mm
    c = torch.empty((m, n), dtype=dtype, device="cuda")
    mm.nvfp4_gemm(a, b, c)
    torch.cuda.synchronize()
    return c.cpu().numpy() if dtype == torch.float32 else bf16_tensor_to_f32(c)


def test_gemm_16x256x512_workload():
    p = WORKLOADS["gemm_16x256x512"].params
    announce("gemm 16x256x512 (fp32 and bf16 out)")
    a, b, ra, rb = _pair(p["T"], p["N"], p["K"], p["x_seed"], p["w_seed"])
    ref = ogemm.gemm(ra, rb)
    e32 = max_norm_err(_run(a, b, p["T"], p["N"], torch.float32), ref)
    y16 = _run(a, b, p["T"], p["N"], torch.bfloat16)
    print(f"max-normalised error fp32 {e32:.3e}  bf16 {max_norm_err(y16, ref):.3e}")
    assert e32 <= 1e-5
    assert_bf16_rounding_close(y16, ref)


SHAPES = [(1, 64, 128), (5, 320, 384), (31, 128, 256), (33, 512, 256), (200, 384, 640), (130, 1000, 1024),
          (64, 8, 128), (7, 100, 256), (32, 1000, 384), (3, 40, 1152), (2, 96, 8192),
          # 27 x 19 = 513 tiles of 64 x 256, ragged in both: one more than the 512 persistent
          # work-groups, so work-group 0 takes a second tile after the epilogue of its first
          (1700, 4800, 256)]


@pytest.mark.parametrize("m,n,k", SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SHAPES])
def test_gemm_shapes_ragged(m, n, k):
    announce(f"gemm {m}x{n}x{k}")
    a, b, ra, rb = _pair(m, n, k, 10 + m, 20 + n)
    y = _run(a, b, m, n, torch.float32)
    err = max_norm_err(y, ogemm.gemm(ra, rb))
    print(f"max-normalised error {err:.3e}")
    assert err <= 1e-5


def test_gemm_down_projection_full_size():
    # the prefill down projection: 1024 x 5120 x 17408
    announce("gemm 1024x5120x17408")
    a, b, ra, rb = _pair(1024, 5120, 17408, 3101, 3004)
    y = _run(a, b, 1024, 5120, torch.float32)
    err = max_norm_err(y, ogemm.gemm(ra, rb))
    print(f"max-normalised error {err:.3e}")
    assert err <= 1e-5


def test_gemm_is_deterministic():
    announce("gemm determinism 200x384x640")
    a, b, _, _ = _pair(200, 384, 640, 5, 6)
    y1 = _run(a, b, 200, 384, torch.float32)
    y2 = _run(a, b, 200, 384, torch.float32)
    assert np.array_equal(y1, y2)


AMAX_SHAPES = [(1, 512, 1024), (2, 640, 3072), (5, 512, 2048), (20, 384, 256), (300, 640, 512), (1024, 5120, 17408)]


@pytest.mark.parametrize("m,n,k", AMAX_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in AMAX_SHAPES])
def test_output_amax_epilogue(m, n, k):
    """The largest of the c_amax slots is max|c| as stored, bit-exact (float32
    and bf16 outputs); every slot is written (the buffer is pre-filled with a
    larger value); the output itself is unchanged by asking for it; the next
    quantisation formed from the slots (NVFP4_GS_FROM_AMAX, one launch) equals
    the computed-scale quantisation."""
    import mlp_prefill_amd as mm
    announce(f"output amax {m}x{n}x{k}")
    a, b, ra, rb = _pair(m, n, k, 900 + m, 950 + n)
    for dt in (torch.float32, torch.bfloat16):
        c0 = torch.empty((m, n), dtype=dt, device="cuda")
        mm.nvfp4_gemm(a, b, c0)
        c = torch.empty((m, n), dtype=dt, device="cuda")
        amax = mm.amax_buffer().fill_(3.0e38)
        mm.nvfp4_gemm(a, b, c, amax=amax)
        torch.cuda.synchronize()
        assert torch.equal(c, c0), f"{dt}: output changed by the amax epilogue"
        want = c.float().abs().max()
        assert amax.max().item() == want.item(), (dt, amax.max().item(), want.item())
        if n % 16 == 0:
            q1, q2 = mm.NVFP4.empty(m, n), mm.NVFP4.empty(m, n)
            mm.nvfp4_quantize_act(c, q1)
            before = mm.launch_count()
            mm.nvfp4_quantize_act(c, q2, gs_mode=mm.GS_FROM_AMAX, ws=amax)
            assert mm.launch_count() - before == 1
            assert_nvfp4_equal(to_host(q2), to_host(q1), f"{dt} quantise from the output amax")
