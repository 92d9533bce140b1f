"""The decode-shaped MLP stack captured in a HIP graph replays bit-identically.

Every library call is capture-safe: it allocates nothing, never synchronises,
issues no memset and enqueues only kernels on the caller's stream.  A
2-layer stack of full-size layers (hidden 5120, intermediate 17408) at T = 1
and T = 5 is captured once and replayed three times, with eager library work
on other buffers between the replays; every replay must equal the eager run
of the same stack bit for bit (same kernels, same inputs, fixed reduction
order).
"""
import pytest
import torch

from synthetic import WORKLOADS, bf16_normal, layer_seeds
from tests.gpu_util import announce, dev_bf16, dev_quantize, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


class Stack:
    def __init__(self, m, layers, t, k, i):
        self.m, self.layers, self.t = m, layers, t
        self.xq = m.NVFP4.empty(t, k)
        self.hq = m.NVFP4.empty(t, i)
        self.ws_q = torch.empty(m.ws_bytes_quantize(t, k), dtype=torch.uint8, device="cuda")
        self.ws_gu = torch.empty(m.mlp_gu_act_ws_bytes(t, k, i), dtype=torch.uint8, device="cuda")
        self.ws_dn = torch.empty(max(m.mlp_down_ws_bytes(t, i, k), 256), dtype=torch.uint8, device="cuda")
        self.mid = torch.empty((t, k), dtype=torch.bfloat16, device="cuda")
        self.out = torch.empty((t, k), dtype=torch.bfloat16, device="cuda")

    def __call__(self, x):
        m = self.m
        cur = x
        for li, w in enumerate(self.layers):
            dst = self.out if li == len(self.layers) - 1 else self.mid
            m.nvfp4_quantize_act(cur, self.xq, ws=self.ws_q)
            m.nvfp4_mlp_gu_act(self.xq, w[0], w[1], self.hq, ws=self.ws_gu)
            m.nvfp4_mlp_down(self.hq, w[2], dst, ws=self.ws_dn)
            cur = dst


@pytest.mark.parametrize("t", [1, 5])
def test_decode_stack_graph_replays_match_eager(t):
    import mlp_prefill_amd as m
    p = WORKLOADS["mlp_long_prefill_16x1024_4layers"].params
    k, i = p["K"], p["I"]
    announce(f"graph: 2-layer decode stack T={t}")
    layers = [[dev_quantize(bf16_normal(s, shp, sigma=p["w_sigma"]))
               for s, shp in zip(layer_seeds(p["layer_seed0"], li), [(i, k), (i, k), (k, i)])] for li in range(2)]
    x = dev_bf16(bf16_normal(77 + t, (t, k)))
    stack = Stack(m, layers, t, k, i)
    other = Stack(m, layers, t, k, i)
    stack(x)                                   # eager reference (also warms up the library)
    torch.cuda.synchronize()
    ref = stack.out.clone()
    ref_hq = stack.hq.codes.clone()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            stack(x)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    launches_before = m.launch_count()
    for rep in range(3):
        stack.out.zero_()
        stack.hq.codes.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(stack.out, ref), f"replay {rep}: output differs from the eager run"
        assert torch.equal(stack.hq.codes, ref_hq), f"replay {rep}: H~ differs from the eager run"
        other(x * 0.5)                         # eager work between replays
        torch.cuda.synchronize()
    # replays enqueue no new host-side launches; the eager calls between them
    # do (5 per MLP call on the decode weight streams: quantise 1, gate/up 2, down 2)
    assert m.launch_count() - launches_before == 3 * 2 * 5
