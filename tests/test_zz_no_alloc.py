"""The allocation-free quantiser (nvfp4_quantize_act_noalloc) against the
workspace call (nvfp4_quantize_act) on the same inputs: codes, scales and
global scale bit-identical, on two calls in a row (the second on a smaller
tensor, so it reads fewer of the scratch array's partial maxima than the first
left behind), through the C ABI."""
import numpy as np
import pytest
import torch

from synthetic import bf16_normal
from tests.gpu_util import announce, assert_nvfp4_equal, dev_bf16, require_gpu, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


def _both(x, gs_mode, gs=None):
    import mlp_prefill_amd as m
    rows, cols = x.shape
    a, b = m.NVFP4.empty(rows, cols), m.NVFP4.empty(rows, cols)
    if gs is not None:
        a.gscale.fill_(gs)
        b.gscale.fill_(gs)
    ws = torch.empty(m.ws_bytes_quantize(rows, cols, gs_mode), dtype=torch.uint8, device="cuda")
    m.nvfp4_quantize_act(x, a, gs_mode=gs_mode, ws=ws)
    m.nvfp4_quantize_act_noalloc(x, b, gs_mode=gs_mode)
    return to_host(a), to_host(b)


@pytest.mark.parametrize("shapes", [[(4096, 5120), (300, 5120)], [(2048, 17408), (1, 5120)]],
                         ids=["large_then_smaller", "large_then_decode"])
def test_noalloc_equals_workspace_call(shapes):
    for j, (rows, cols) in enumerate(shapes):
        announce(f"noalloc quantise call {j}: {rows}x{cols}")
        xb = bf16_normal(8100 + j, (rows, cols))
        xb[rows // 2, cols // 3] = 0x4480          # one large value (1024): the amax lies in one partial
        x = dev_bf16(xb)
        a, b = _both(x, 0)
        assert_nvfp4_equal(b, a, f"noalloc vs workspace call {j}")
        assert a.gs == np.float32(1024.0 / 2688.0)


def test_noalloc_float32_and_given_scale():
    rows, cols = 1000, 4096
    announce("noalloc quantise float32, computed then given scale")
    x = torch.from_numpy(np.random.default_rng(5).standard_normal((rows, cols)).astype(np.float32)).cuda()
    a, b = _both(x, 0)
    assert_nvfp4_equal(b, a, "float32 computed scale")
    a, b = _both(x, 1, gs=0.0005)
    assert_nvfp4_equal(b, a, "float32 given scale")
