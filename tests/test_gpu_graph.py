"""The decode-shaped MLP stack captured in a HIP graph: replays against the
eager run and against the oracle.

Every library call is capture-safe: it allocates nothing, never synchronises,
issues no memset and enqueues only kernels on the caller's stream.  A
2-layer stack of full-size layers (hidden 5120, intermediate 17408) at T = 1
and T = 5 is captured once and replayed three times, with eager library work
on other buffers between the replays; every replay must equal the eager run
of the same stack bit for bit (same kernels, same inputs, fixed reduction
order).  The last replay's outputs are then staged against the oracle layer
by layer, as the stacked-layer test does: layer 0 on the seeded input, layer
1 on the device's own bf16 output of layer 0 (x~ bit-exact, H~ flips only at
rounding boundaries, Y within one bf16 rounding of the flip-corrected oracle).
"""
import numpy as np
import pytest
import torch

from oracle import gemm as ogemm
from oracle import mlp as omlp
from oracle import quant
from synthetic import WORKLOADS, bf16_bits_to_f32, bf16_normal, layer_seeds
from tests.gpu_util import (announce, assert_bf16_rounding_close, assert_nvfp4_equal, bf16_tensor_to_f32, dev_bf16,
                            dev_quantize, legit_requant_flips, max_norm_err, record, require_gpu, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


class Stack:
    """Per-layer x~, H~ and bf16 outputs stay in their own buffers, so a replay
    can be staged layer by layer afterwards."""

    def __init__(self, m, layers, t, k, i):
        self.m, self.layers, self.t = m, layers, t
        n = len(layers)
        self.xq = [m.NVFP4.empty(t, k) for _ in range(n)]
        self.hq = [m.NVFP4.empty(t, i) for _ in range(n)]
        self.ws_q = torch.empty(m.ws_bytes_quantize(t, k), dtype=torch.uint8, device="cuda")
        self.ws_gu = torch.empty(m.mlp_gu_act_ws_bytes(t, k, i), dtype=torch.uint8, device="cuda")
        self.ws_dn = torch.empty(max(m.mlp_down_ws_bytes(t, i, k), 256), dtype=torch.uint8, device="cuda")
        self.ys = [torch.empty((t, k), dtype=torch.bfloat16, device="cuda") for _ in range(n)]
        self.out = self.ys[-1]

    def __call__(self, x):
        m = self.m
        cur = x
        for li, w in enumerate(self.layers):
            m.nvfp4_quantize_act(cur, self.xq[li], ws=self.ws_q)
            m.nvfp4_mlp_gu_act(self.xq[li], w[0], w[1], self.hq[li], ws=self.ws_gu)
            m.nvfp4_mlp_down(self.hq[li], w[2], self.ys[li], ws=self.ws_dn)
            cur = self.ys[li]


def stage_against_oracle(stack, xbits, wref, label):
    """Layer-by-layer parity of the stack's current outputs with the oracle."""
    layer_in = bf16_bits_to_f32(xbits)
    for li in range(len(wref)):
        ref = omlp.mlp(layer_in, *wref[li])
        assert_nvfp4_equal(to_host(stack.xq[li]), ref["xq"], f"{label} layer {li} x~")
        got_hq = to_host(stack.hq[li])
        nflip, nsflip = legit_requant_flips(ref["h"].astype(np.float32), got_hq, ref["hq"])
        corr = ref["y"] + ogemm.gemm(got_hq, wref[li][2]) - ogemm.gemm(ref["hq"], wref[li][2])
        y = bf16_tensor_to_f32(stack.ys[li])
        err = max_norm_err(y, corr)
        print(f"{label} layer {li}: flips {nflip}/{nsflip}  Y err (bf16 out, flip-corrected) {err:.2e}")
        record(f"{label} layer {li}", code_flips=nflip, scale_flips=nsflip, y_err_flip_corrected_bf16=err,
               y_err_e2e_bf16=max_norm_err(y, ref["y"]))
        assert_bf16_rounding_close(y, corr)
        layer_in = y


@pytest.mark.parametrize("t", [1, 5])
def test_decode_stack_graph_replays_match_eager(t):
    import mlp_prefill_amd as m
    p = WORKLOADS["mlp_long_prefill_16x1024_4layers"].params
    k, i = p["K"], p["I"]
    announce(f"graph: 2-layer decode stack T={t}")
    bits = [[bf16_normal(s, shp, sigma=p["w_sigma"])
             for s, shp in zip(layer_seeds(p["layer_seed0"], li), [(i, k), (i, k), (k, i)])] for li in range(2)]
    layers = [[dev_quantize(b) for b in lb] for lb in bits]
    wref = [[quant.quantize(bf16_bits_to_f32(b)) for b in lb] for lb in bits]
    xbits = bf16_normal(77 + t, (t, k))
    x = dev_bf16(xbits)
    stack = Stack(m, layers, t, k, i)
    other = Stack(m, layers, t, k, i)
    stack(x)                                   # eager reference (also warms up the library)
    torch.cuda.synchronize()
    ref = stack.out.clone()
    ref_hq = stack.hq[-1].codes.clone()

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
        for buf in stack.ys:
            buf.zero_()
        for q in stack.hq:
            q.codes.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(stack.out, ref), f"replay {rep}: output differs from the eager run"
        assert torch.equal(stack.hq[-1].codes, ref_hq), f"replay {rep}: H~ differs from the eager run"
        other(x * 0.5)                         # eager work between replays
        torch.cuda.synchronize()
    # replays enqueue no new host-side launches; the eager calls between them
    # do (per MLP call on the decode weight streams: quantise 1, gate/up 2, down 2,
    # and at 3-8 tokens one more that clears the split gate/up's tickets)
    assert m.launch_count() - launches_before == 3 * 2 * (5 if t <= 2 else 6)
    # the buffers now hold the last replay (the eager calls between replays used `other`)
    stage_against_oracle(stack, xbits, wref, f"graph replay T={t}")


class WholeStack(Stack):
    """The same stack through the whole-MLP call (nvfp4_mlp, 4 launches per layer on decode batches)."""

    def __init__(self, m, layers, t, k, i):
        super().__init__(m, layers, t, k, i)
        self.ws = torch.empty(m.mlp_ws_bytes(t, k, i), dtype=torch.uint8, device="cuda")

    def __call__(self, x):
        cur = x
        for li, w in enumerate(self.layers):
            self.m.nvfp4_mlp(cur, w[0], w[1], w[2], self.xq[li], self.hq[li], self.ys[li], ws=self.ws)
            cur = self.ys[li]


@pytest.mark.parametrize("t", [1, 5])
def test_whole_mlp_stack_graph_replays_match_eager_and_oracle(t):
    """Graph capture of the whole-MLP decode path: its first launch clears the
    down stream's tickets with a kernel (no memset node), so every replay
    starts from cleared tickets; replays equal the eager run bit for bit and
    are staged against the oracle layer by layer."""
    import mlp_prefill_amd as m
    p = WORKLOADS["mlp_long_prefill_16x1024_4layers"].params
    k, i = p["K"], p["I"]
    announce(f"graph: 2-layer whole-MLP decode stack T={t}")
    bits = [[bf16_normal(s, shp, sigma=p["w_sigma"])
             for s, shp in zip(layer_seeds(p["layer_seed0"], li), [(i, k), (i, k), (k, i)])] for li in range(2)]
    layers = [[dev_quantize(b) for b in lb] for lb in bits]
    wref = [[quant.quantize(bf16_bits_to_f32(b)) for b in lb] for lb in bits]
    xbits = bf16_normal(177 + t, (t, k))
    x = dev_bf16(xbits)
    stack = WholeStack(m, layers, t, k, i)
    other = WholeStack(m, layers, t, k, i)
    stack(x)
    torch.cuda.synchronize()
    ref = stack.out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            stack(x)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for buf in stack.ys:
            buf.zero_()
        stack.ws.fill_(0xFF)                   # tickets and partial sums left dirty on purpose
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(stack.out, ref), f"replay {rep}: output differs from the eager run"
        other(x * 0.5)
        torch.cuda.synchronize()
    stage_against_oracle(stack, xbits, wref, f"whole-MLP graph replay T={t}")
