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
          (64, 8, 128), (7, 100, 256), (32, 1000, 384), (3, 40, 1152), (2, 96, 8192)]


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
