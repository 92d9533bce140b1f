"""RMSNorm fused into the NVFP4 activation quantiser vs the oracle (oracle.norm).

Staged: (1) the device's inverse rms per row (kept in the workspace) within
1e-5 of the float64 value; (2) codes, scales and global scale bit-exact
against the oracle quantiser applied to RN32(RN32(x * rinv) * gamma) formed
with the device's rinv -- the same float32 products the kernel forms, so
every rounding decision is pinned; (3) against the oracle's own float64
RMSNorm, differences only at decisions within 2^-14 of a boundary.
"""
import numpy as np
import pytest
import torch

from oracle import norm, quant
from synthetic import WORKLOADS, bf16_bits_to_f32, bf16_normal, outlier_channels
from tests.gpu_util import announce, assert_nvfp4_equal, legit_requant_flips, require_gpu, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


def check(x, gamma, eps, label):
    import mlp_prefill_amd as m
    announce(f"rmsnorm-quantise: {label}")
    rows, cols = x.shape
    xd = torch.from_numpy(x).cuda() if x.dtype == np.float32 else \
        torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    xf = x if x.dtype == np.float32 else bf16_bits_to_f32(x)
    g = torch.from_numpy(gamma).cuda()
    out = m.NVFP4.empty(rows, cols)
    ws = m.nvfp4_rmsnorm_quantize_act(xd, g, eps, out)
    torch.cuda.synchronize()
    rinv = ws[: rows * 4].view(torch.float32).cpu().numpy()
    ref_rinv = norm.inv_rms(xf, np.float32(eps))
    err = float(np.max(np.abs(rinv / ref_rinv - 1.0)))
    print(f"{label}: rinv max rel err {err:.2e}")
    assert err <= 1e-5
    y32 = (xf * rinv[:, None]).astype(np.float32) * gamma[None, :]        # float32 products, as on the device
    got = to_host(out)
    assert_nvfp4_equal(got, quant.quantize(y32.astype(np.float32)), "given the device's rinv")
    ref = norm.rmsnorm_quantize(xf, gamma, np.float32(eps))
    yref = norm.rmsnorm(xf, gamma, np.float32(eps)).astype(np.float32)
    n, nb = legit_requant_flips(yref, got, ref)
    print(f"{label}: vs float64 RMSNorm: {n} element / {nb} block decisions flipped near boundaries")


def _gamma(seed, cols):
    return (1.0 + 0.1 * np.random.default_rng(seed).standard_normal(cols)).astype(np.float32)


def test_prefill_activation_with_outliers():
    p = WORKLOADS["mlp_prefill_1024x5120x17408"].params
    x = bf16_normal(p["x_seed"], (p["T"], p["K"]), outliers=outlier_channels(p["outlier_seed"], p["K"]))
    check(x, _gamma(7, p["K"]), 1e-6, "1024x5120 bf16 with outliers")


@pytest.mark.parametrize("rows,cols", [(1, 5120), (5, 5120), (37, 272), (1000, 64)])
def test_shapes(rows, cols):
    check(bf16_normal(rows + cols, (rows, cols)), _gamma(cols, cols), 1e-5, f"{rows}x{cols}")


def test_float32_input_zero_rows_and_large_eps():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((40, 128)) * np.exp(rng.uniform(-8, 8, (40, 1)))).astype(np.float32)
    x[3] = 0.0                                   # rinv = 1/sqrt(eps): all codes 0
    x[11] = 0.0
    check(x, _gamma(3, 128), 1e-6, "float32, wide row scales, zero rows")
    check(x, _gamma(4, 128), 0.5, "large eps")


def test_two_launches():
    import mlp_prefill_amd as m
    x = torch.randn(16, 256, device="cuda").to(torch.bfloat16)
    out = m.NVFP4.empty(16, 256)
    before = m.launch_count()
    m.nvfp4_rmsnorm_quantize_act(x, torch.ones(256, device="cuda"), 1e-6, out)
    assert m.launch_count() - before == 2
