"""The timing window brackets exactly the launches of the chosen kernel class."""
import pytest
import torch

from synthetic import bf16_normal
from tests.gpu_util import announce, dev_bf16, dev_quantize, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


def test_timing_window_counts_and_drops():
    import mlp_prefill_amd as m
    announce("timing window: gate/up contraction, 3 calls, room for 2")
    t, k, i = 64, 256, 384
    x = dev_bf16(bf16_normal(1, (t, k)))
    wg, wu = dev_quantize(bf16_normal(2, (i, k), sigma=0.02)), dev_quantize(bf16_normal(3, (i, k), sigma=0.02))
    xq, hq = m.NVFP4.empty(t, k), m.NVFP4.empty(t, i)
    ws = torch.empty(m.mlp_gu_act_ws_bytes(t, k, i), dtype=torch.uint8, device="cuda")
    m.nvfp4_quantize_act(x, xq)
    m.nvfp4_timing_begin(m.KC_GEMM_GLU, 2)
    for _ in range(3):
        m.nvfp4_mlp_gu_act(xq, wg, wu, hq, ws=ws)
    n, dropped, ms = m.nvfp4_timing_end()
    print(f"timed {n}, dropped {dropped}, {ms * 1e3:.1f} us total")
    assert (n, dropped) == (2, 1)
    assert 0.0 < ms < 1000.0
    # a window on another class sees none of these launches
    m.nvfp4_timing_begin(m.KC_GEMM_STORE, 8)
    m.nvfp4_mlp_gu_act(xq, wg, wu, hq, ws=ws)
    assert m.nvfp4_timing_end() == (0, 0, 0.0)
