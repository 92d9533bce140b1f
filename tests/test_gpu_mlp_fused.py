"""The whole-MLP call (nvfp4_mlp) against the separate calls and the oracle.

- Bit-identical to nvfp4_quantize_act + nvfp4_mlp_gu_act + nvfp4_mlp_down on
  the same inputs (x~, H~ with their global scales, y in float32 and bf16):
  the decode path runs the same kernels, and its in-kernel split-K finish adds
  the same partial sums in the same order as the reduction launch it replaces.
- Launches: 4 for every decode batch (1 to 16 tokens at the full 5120 / 17408
  shape); otherwise the separate calls' count minus their two expansion
  launches (the quantisers write the f16 operand copies).
- Staged against the oracle at T = 1 and 5 (full size) like every MLP test.
- The output amax slots and a chained second layer that takes them as x_amax.
- Two calls in a row give identical results (the tickets are cleared by each
  call's first launch, whatever the workspace held).
"""
import numpy as np
import pytest
import torch

from oracle import gemm as ogemm
from oracle import mlp as omlp
from oracle import quant
from synthetic import WORKLOADS, bf16_bits_to_f32, bf16_normal
from tests.gpu_util import (TOL, announce, assert_nvfp4_equal, dev_bf16, legit_requant_flips, max_norm_err, record,
                            require_gpu, to_host)
from tests.test_gpu_mlp import _weights, run_device_mlp

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


@pytest.fixture(scope="module")
def decode_weights():
    p = WORKLOADS["mlp_decode_5120x17408"].params
    return _weights(p["K"], p["I"], (p["wg_seed"], p["wu_seed"], p["wd_seed"]))


def decode_launches(t):
    return 4


def run_fused(xbits, wdev, y_dtype=torch.float32, x_amax=None, y_amax=None, ws=None, x=None):
    import mlp_prefill_amd as m
    t, k = xbits.shape if x is None else x.shape
    i = wdev[0].rows
    x = dev_bf16(xbits) if x is None else x
    xq, hq = m.NVFP4.empty(t, k), m.NVFP4.empty(t, i)
    y = torch.empty((t, k), dtype=y_dtype, device="cuda")
    before = m.launch_count()
    m.nvfp4_mlp(x, wdev[0], wdev[1], wdev[2], xq, hq, y, x_amax=x_amax, y_amax=y_amax, ws=ws)
    launches = m.launch_count() - before
    torch.cuda.synchronize()
    return xq, hq, y, launches


def assert_same_as_separate(xbits, wdev, label):
    """x~, H~ and y (float32 and bf16) bit-identical to the separate calls."""
    for dt in (torch.float32, torch.bfloat16):
        xq0, _, hq0, y0 = run_device_mlp(xbits, wdev, y_dtype=dt)
        xq, hq, y, launches = run_fused(xbits, wdev, dt)
        assert_nvfp4_equal(to_host(xq), to_host(xq0), f"{label} x~")
        assert_nvfp4_equal(to_host(hq), to_host(hq0), f"{label} H~")
        assert torch.equal(y, y0), f"{label} {dt}: y differs from the separate calls"
    return launches


@pytest.mark.parametrize("t", [1, 2, 3, 4, 5, 8, 9, 12, 16])
def test_decode_equals_separate_calls(decode_weights, t):
    p = WORKLOADS["mlp_decode_5120x17408"].params
    announce(f"whole MLP decode T={t} vs separate calls")
    launches = assert_same_as_separate(bf16_normal(p["x_seed"] + t, (t, p["K"])), decode_weights[0], f"T{t}")
    assert launches == decode_launches(t), launches


SHAPES = [(2, 1152, 3072), (1, 1024, 1024), (5, 2048, 3072), (7, 1024, 2048), (16, 512, 1024), (300, 512, 1024)]


@pytest.mark.parametrize("t,k,i", SHAPES, ids=[f"T{t}_K{k}_I{i}" for t, k, i in SHAPES])
def test_shapes_equal_separate_calls(t, k, i):
    import mlp_prefill_amd as m
    announce(f"whole MLP T={t} K={k} I={i} vs separate calls")
    wdev, _ = _weights(k, i, (1500 + t, 1501 + t, 1502 + t))
    xbits = bf16_normal(1503 + t, (t, k))
    launches = assert_same_as_separate(xbits, wdev, f"T{t} K{k} I{i}")
    before = m.launch_count()
    run_device_mlp(xbits, wdev)
    separate = m.launch_count() - before
    assert launches == (decode_launches(t) if t <= 16 else separate - 2), (launches, separate)


@pytest.mark.parametrize("t", [1, 2])
def test_float32_input_equals_separate_calls(decode_weights, t):
    """float32 x through the whole-MLP call equals the separate calls."""
    import mlp_prefill_amd as m
    p = WORKLOADS["mlp_decode_5120x17408"].params
    announce(f"whole MLP float32 x T={t}")
    x = torch.from_numpy(np.random.default_rng(31 + t).standard_normal((t, p["K"])).astype(np.float32)).cuda()
    wdev = decode_weights[0]
    xq0, hq0 = m.NVFP4.empty(t, p["K"]), m.NVFP4.empty(t, p["I"])
    y0 = torch.empty((t, p["K"]), dtype=torch.float32, device="cuda")
    m.nvfp4_quantize_act(x, xq0)
    m.nvfp4_mlp_gu_act(xq0, wdev[0], wdev[1], hq0)
    m.nvfp4_mlp_down(hq0, wdev[2], y0)
    xq, hq, y, launches = run_fused(None, wdev, x=x)
    assert launches == decode_launches(t)
    assert_nvfp4_equal(to_host(xq), to_host(xq0), "x~")
    assert_nvfp4_equal(to_host(hq), to_host(hq0), "H~")
    assert torch.equal(y, y0)


@pytest.mark.parametrize("t", [1, 5])
def test_decode_staged_against_oracle(decode_weights, t):
    p = WORKLOADS["mlp_decode_5120x17408"].params
    wdev, wref = decode_weights
    announce(f"whole MLP decode T={t} vs oracle")
    xbits = bf16_normal(p["x_seed"], (t, p["K"]))
    xq, hq, y, _ = run_fused(xbits, wdev)
    ref = omlp.mlp(bf16_bits_to_f32(xbits), *wref)
    assert_nvfp4_equal(to_host(xq), ref["xq"], "x~")
    hq_dev = to_host(hq)
    nflip, nsflip = legit_requant_flips(ref["h"].astype(np.float32), hq_dev, ref["hq"])
    y = y.cpu().numpy()
    corr = ref["y"] + ogemm.gemm(hq_dev, wref[2]) - ogemm.gemm(ref["hq"], wref[2])
    e2e, ecorr = max_norm_err(y, ref["y"]), max_norm_err(y, corr)
    print(f"whole MLP T={t}: flips {nflip}/{nsflip}  Y e2e {e2e:.2e}  flip-corrected {ecorr:.2e}")
    record(f"whole MLP decode T{t}", code_flips=nflip, scale_flips=nsflip, y_err_e2e=e2e,
           y_err_flip_corrected=ecorr, tokens=t, hidden=int(p["K"]), intermediate=int(p["I"]))
    assert ecorr <= TOL


@pytest.mark.parametrize("t", [1, 5, 300])
def test_output_amax_and_chained_layer(t):
    """y_amax holds max|y| (every slot written); a second layer with x_amax =
    the first layer's y_amax quantises its input exactly as a computed scale."""
    import mlp_prefill_amd as m
    k, i = (1024, 2048) if t <= 8 else (512, 1024)
    announce(f"whole MLP amax chain T={t}")
    w1, _ = _weights(k, i, (1600, 1601, 1602))
    w2, _ = _weights(k, i, (1603, 1604, 1605))
    amax = m.amax_buffer().fill_(3.0e38)
    _, _, y1, _ = run_fused(bf16_normal(1606 + t, (t, k)), w1, torch.bfloat16, y_amax=amax)
    assert amax.max().item() == y1.float().abs().max().item()
    xq_a, hq_a, y_a, la = run_fused(None, w2, torch.float32, x_amax=amax, x=y1)
    xq_b, hq_b, y_b, lb = run_fused(None, w2, torch.float32, x=y1)
    assert_nvfp4_equal(to_host(xq_a), to_host(xq_b), "x~ from the amax slots")
    assert_nvfp4_equal(to_host(hq_a), to_host(hq_b), "H~")
    assert torch.equal(y_a, y_b)
    assert la == (decode_launches(t) if t <= 16 else lb - 1), (la, lb)


@pytest.mark.parametrize("t", [64, 1024])
def test_large_batch_full_size_equals_separate_calls(t):
    """Large batches at the full 5120 / 17408 shape (the long-prefill ubatch):
    the quantisers' f16 operand copies replace the expansion launches, and x~,
    H~ and y stay bit-identical to the separate calls; 6 launches (5 when the
    input amax comes from the previous layer's slots)."""
    import mlp_prefill_amd as m
    p = WORKLOADS["mlp_prefill_1024x5120x17408"].params
    announce(f"whole MLP large batch T={t} full size vs separate calls")
    wdev, _ = _weights(p["K"], p["I"], (p["wg_seed"], p["wu_seed"], p["wd_seed"]))
    launches = assert_same_as_separate(bf16_normal(p["x_seed"] + t, (t, p["K"])), wdev, f"T{t}")
    assert launches == 6, launches


def test_repeated_calls_any_workspace(decode_weights):
    """The tickets live in the workspace and are cleared by the call itself:
    workspaces pre-filled with different bytes give identical results, call
    after call."""
    import mlp_prefill_amd as m
    p = WORKLOADS["mlp_decode_5120x17408"].params
    announce("whole MLP repeated calls, dirty workspaces")
    xbits = bf16_normal(1700, (2, p["K"]))
    need = m.mlp_ws_bytes(2, p["K"], p["I"])
    outs = []
    for fill in (0x00, 0xFF, 0x01, 0x01):
        ws = torch.full((need,), fill, dtype=torch.uint8, device="cuda")
        _, hq, y, _ = run_fused(xbits, decode_weights[0], ws=ws)
        outs.append((to_host(hq), y.clone()))
    for hq, y in outs[1:]:
        assert_nvfp4_equal(hq, outs[0][0], "H~ across workspaces")
        assert torch.equal(y, outs[0][1])
