"""Stacked NVFP4 MLP layers with device-resident bf16 activations vs the oracle.

The long-prefill workload (hidden 5120, intermediate 17408, 4 layers,
1024-token ubatches) on a reduced number of tokens: two 128-token ubatches
through all four full-size layers, chained as the benchmark chains them: each
layer's down projection also writes max|y|, and the next layer quantises its
input with the global scale formed from that amax (one launch).  Layer 1 is
compared with the oracle end to end; every later layer is compared with the
oracle applied to the layer's actual (device) bf16 input, so that legitimate
requantisation flips in one layer are not charged to the next; every layer's
x~ must equal the oracle's quantisation of that input bit for bit.  The drift
of the whole 4-layer chain against the pure oracle chain is reported.
"""
import numpy as np
import pytest
import torch

from oracle import gemm as ogemm
from oracle import mlp as omlp
from oracle import quant
from synthetic import WORKLOADS, bf16_bits_to_f32, bf16_normal, layer_seeds
from tests.gpu_util import (announce, assert_bf16_rounding_close, assert_nvfp4_equal, bf16_tensor_to_f32, dev_bf16,
                            dev_quantize,
                            legit_requant_flips, max_norm_err, record, require_gpu, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


def test_stacked_layers_device_resident_bf16_chain():
    import mlp_prefill_amd as m
    p = WORKLOADS["mlp_long_prefill_16x1024_4layers"].params
    k, i, nl = p["K"], p["I"], p["layers"]
    ub, nub = 128, 2
    announce(f"stacked: {nub} ubatches x {ub} tokens x {nl} layers (full-size layers)")
    xbits = bf16_normal(p["x_seed"], (p["T"], k))[: ub * nub]
    wdev, wref = [], []
    for li in range(nl):
        bits = [bf16_normal(s, shp, sigma=p["w_sigma"])
                for s, shp in zip(layer_seeds(p["layer_seed0"], li), [(i, k), (i, k), (k, i)])]
        wdev.append([dev_quantize(b) for b in bits])
        wref.append([quant.quantize(bf16_bits_to_f32(b)) for b in bits])

    x_all = dev_bf16(xbits)
    xq = m.NVFP4.empty(ub, k)
    hq = m.NVFP4.empty(ub, i)
    ws_gu = torch.empty(m.mlp_gu_act_ws_bytes(ub, k, i), dtype=torch.uint8, device="cuda")
    outs = [[None] * nl for _ in range(nub)]
    hqs = [[None] * nl for _ in range(nub)]
    xqs = [[None] * nl for _ in range(nub)]
    amax = m.amax_buffer()
    for u in range(nub):
        cur = x_all[u * ub:(u + 1) * ub]
        for li in range(nl):
            if li == 0:
                m.nvfp4_quantize_act(cur, xq)
            else:                                # the previous down projection's max|y|
                m.nvfp4_quantize_act(cur, xq, gs_mode=m.GS_FROM_AMAX, ws=amax)
            m.nvfp4_mlp_gu_act(xq, wdev[li][0], wdev[li][1], hq, ws=ws_gu)
            y = torch.empty((ub, k), dtype=torch.bfloat16, device="cuda")
            m.nvfp4_mlp_down(hq, wdev[li][2], y, amax=amax)
            xqs[u][li] = to_host(xq)
            hqs[u][li] = to_host(hq)
            outs[u][li] = y
            cur = y                              # stays on the device
    torch.cuda.synchronize()

    x0 = bf16_bits_to_f32(xbits)
    for u in range(nub):
        layer_in = x0[u * ub:(u + 1) * ub]
        for li in range(nl):
            ref = omlp.mlp(layer_in, *wref[li])
            assert_nvfp4_equal(xqs[u][li], ref["xq"], f"ubatch {u} layer {li} x~")
            got_hq = hqs[u][li]
            nflip, nsflip = legit_requant_flips(ref["h"].astype(np.float32), got_hq, ref["hq"])
            corr = ref["y"] + ogemm.gemm(got_hq, wref[li][2]) - ogemm.gemm(ref["hq"], wref[li][2])
            y = bf16_tensor_to_f32(outs[u][li])
            print(f"ubatch {u} layer {li}: input rms {np.sqrt(np.mean(layer_in.astype(np.float64) ** 2)):.3g}  "
                  f"flips {nflip}/{nsflip}  Y err (bf16 out) {max_norm_err(y, corr):.2e}")
            record(f"stacked ubatch {u} layer {li}", code_flips=nflip, scale_flips=nsflip,
                   y_err_flip_corrected_bf16=max_norm_err(y, corr), y_err_e2e_bf16=max_norm_err(y, ref["y"]))
            assert_bf16_rounding_close(y, corr)
            layer_in = y                         # the device's bf16 activation is the next layer's input

    # drift of the whole chain against the pure oracle chain (reported)
    y_last, _ = omlp.stacked_mlp(x0, wref, ubatch=ub)
    got = np.concatenate([bf16_tensor_to_f32(outs[u][nl - 1]) for u in range(nub)])
    drift = max_norm_err(got, y_last)
    print(f"4-layer chain vs pure oracle chain: max-normalised error {drift:.2e}")
    record("stacked 4-layer chain vs pure oracle chain", y_err_e2e_bf16=drift, tokens=ub * nub)
