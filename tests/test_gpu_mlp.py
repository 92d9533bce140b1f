"""Device MLP (quantise -> gate/up + SiLU*up + requant -> down) vs the oracle.

Stages compared (all against the oracle's own end-to-end run):
  S1  x~ bit-exact;
  S2  the float32 GLU output H the device quantised vs the oracle's H
      (max-normalised error gated), and the device's requantisation of its own
      H bit-exact: gs_h equals the oracle's global scale of the device's H,
      and the oracle's quantisation of the device's H with that scale equals
      the device's H~ code for code; gs_h within 2^-20 (relative) of the
      oracle's own gs_h;
  S3  H~ against the oracle's H~: every code or scale that differs must be a
      rounding decision the oracle takes within 2^-14 (relative) of a
      boundary -- the device's float32 accumulation moves H by ~1e-7, so
      such decisions can legitimately go either way;
  S4  Y vs the oracle's Y after accounting for those boundary flips
      (the oracle's down projection of the difference of the two H~), gate
      2e-3 max-normalised.  The raw end-to-end error is recorded (it can
      exceed 2e-3 when a block scale of H~ flips: one flipped E4M3 scale moves
      16 H~ values by 1/8 of their scale).
"""
import numpy as np
import pytest
import torch

from oracle import gemm as ogemm
from oracle import mlp as omlp
from oracle import quant
from synthetic import WORKLOADS, bf16_bits_to_f32, bf16_normal, outlier_channels
from tests.gpu_util import (TOL, announce, assert_nvfp4_equal, dev_bf16, dev_quantize, legit_requant_flips,
                            max_norm_err, record, require_gpu, to_host)

H_TOL = 1e-6          # float32 accumulation of exact products, SiLU in float32 (measured <= 1.8e-7)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


def _weights(k, i, seeds, sigma=0.02):
    gb = bf16_normal(seeds[0], (i, k), sigma=sigma)
    ub = bf16_normal(seeds[1], (i, k), sigma=sigma)
    db = bf16_normal(seeds[2], (k, i), sigma=sigma)
    dev = [dev_quantize(b) for b in (gb, ub, db)]
    ref = [quant.quantize(bf16_bits_to_f32(b)) for b in (gb, ub, db)]
    return dev, ref


def run_device_mlp(xbits, wdev, y_dtype=torch.float32):
    """quantize_act -> mlp_gu_act -> mlp_down on the device; returns (x~, H, H~, Y)."""
    import mlp_prefill_amd as m
    t, k = xbits.shape
    i = wdev[0].rows
    x = dev_bf16(xbits)
    xq = m.NVFP4.empty(t, k)
    m.nvfp4_quantize_act(x, xq)
    hq = m.NVFP4.empty(t, i)
    ws = m.nvfp4_mlp_gu_act(xq, wdev[0], wdev[1], hq)
    y = torch.empty((t, k), dtype=y_dtype, device="cuda")
    m.nvfp4_mlp_down(hq, wdev[2], y)
    torch.cuda.synchronize()
    h = ws[: t * i * 4].view(torch.float32).view(t, i).cpu().numpy()
    return xq, h, hq, y


def check_mlp(xbits, wdev, wref, label):
    t, k = xbits.shape
    x = bf16_bits_to_f32(xbits)
    xq, h, hq, y = run_device_mlp(xbits, wdev)
    ref = omlp.mlp(x, *wref)
    assert_nvfp4_equal(to_host(xq), ref["xq"], f"{label} x~")                       # S1
    eh = max_norm_err(h, ref["h"])                                                  # S2
    hq_dev = to_host(hq)
    # the device requantised its own float32 H exactly: same global scale, same codes
    assert hq_dev.gs.view(np.uint32) == quant.global_scale(h).view(np.uint32), (hq_dev.gs, quant.global_scale(h))
    assert_nvfp4_equal(hq_dev, quant.quantize(h, gs=hq_dev.gs), f"{label} H~ of the device's own H")
    gs_rel = abs(float(hq_dev.gs) / float(ref["hq"].gs) - 1.0)
    nflip, nsflip = legit_requant_flips(ref["h"].astype(np.float32), hq_dev, ref["hq"])  # S3
    y = y.cpu().numpy()
    e2e = max_norm_err(y, ref["y"])
    corr = ref["y"] + ogemm.gemm(hq_dev, wref[2]) - ogemm.gemm(ref["hq"], wref[2])
    ecorr = max_norm_err(y, corr)                                                   # S4
    print(f"{label}: H err {eh:.2e}  gs_h rel {gs_rel:.2e}  requant flips {nflip} codes / {nsflip} scales  "
          f"Y err e2e {e2e:.2e}  flip-corrected {ecorr:.2e}")
    record(label, h_err=eh, gs_h_rel=gs_rel, code_flips=nflip, scale_flips=nsflip, y_err_e2e=e2e,
           y_err_flip_corrected=ecorr, tokens=int(t), hidden=int(k), intermediate=int(h.shape[1]))
    assert eh <= H_TOL
    # gs_h = RN32(amax(H)/2688) moves with the device's H by at most its error
    assert gs_rel <= 2.0 ** -20
    assert ecorr <= TOL
    return e2e


# the last: 27 x 19 = 513 gate/up tiles of 64 x 128 (one more than the 512 persistent work-groups)
SMALL = [(1, 256, 384), (37, 256, 384), (64, 512, 256), (129, 384, 640), (1700, 256, 2432)]


@pytest.mark.parametrize("t,k,i", SMALL, ids=[f"T{t}_K{k}_I{i}" for t, k, i in SMALL])
def test_mlp_small_shapes(t, k, i):
    announce(f"mlp T={t} K={k} I={i}")
    wdev, wref = _weights(k, i, (100 + t, 200 + t, 300 + t))
    check_mlp(bf16_normal(400 + t, (t, k)), wdev, wref, f"T{t}")


@pytest.fixture(scope="module")
def decode_weights():
    p = WORKLOADS["mlp_decode_5120x17408"].params
    return _weights(p["K"], p["I"], (p["wg_seed"], p["wu_seed"], p["wd_seed"]))


def test_mlp_decode_T1_T5(decode_weights):
    import mlp_prefill_amd as m
    p = WORKLOADS["mlp_decode_5120x17408"].params
    wdev, wref = decode_weights
    launches = {}
    for t in p["Ts"]:
        announce(f"decode mlp T={t}")
        xbits = bf16_normal(p["x_seed"], (t, p["K"]))
        before = m.launch_count()
        run_device_mlp(xbits, wdev)
        launches[t] = m.launch_count() - before
        check_mlp(xbits, wdev, wref, f"decode T{t}")
    # one launch set per batch (quantise 1, gate/up 2, down 2); at 3-8 tokens the
    # gate/up K = 5120 runs in splits whose tickets take one clearing launch
    assert launches == {1: 5, 5: 6}, launches
    # the whole-MLP call is four launches at both batch sizes
    for t in p["Ts"]:
        x = dev_bf16(bf16_normal(p["x_seed"], (t, p["K"])))
        xq, hq = m.NVFP4.empty(t, p["K"]), m.NVFP4.empty(t, p["I"])
        y = torch.empty((t, p["K"]), dtype=torch.float32, device="cuda")
        before = m.launch_count()
        m.nvfp4_mlp(x, wdev[0], wdev[1], wdev[2], xq, hq, y)
        launches[t] = m.launch_count() - before
    torch.cuda.synchronize()
    assert launches == {1: 4, 5: 4}, launches


def test_mlp_prefill_1024_outliers():
    p = WORKLOADS["mlp_prefill_1024x5120x17408"].params
    announce("prefill mlp T=1024 (full size)")
    wdev, wref = _weights(p["K"], p["I"], (p["wg_seed"], p["wu_seed"], p["wd_seed"]))
    xbits = bf16_normal(p["x_seed"], (p["T"], p["K"]), outliers=outlier_channels(p["outlier_seed"], p["K"]))
    check_mlp(xbits, wdev, wref, "prefill T1024")


@pytest.mark.parametrize("t", [256, 1])
def test_mlp_tp2_shard_shapes(t):
    """The tensor-parallel (tp = 2) shard of the MLP on one GPU: gate/up
    [5120 -> 2 x 8704], down [8704 -> 5120] (8704 is the per-shard width of the
    vllm.cpp issue's trace, "Problem")."""
    announce(f"mlp tp=2 shard T={t}")
    p = WORKLOADS["mlp_prefill_1024x5120x17408"].params
    k, i = p["K"], p["I"] // 2
    wdev, wref = _weights(k, i, (6001, 6002, 6003))
    xb = bf16_normal(6004 + t, (t, k), outliers=outlier_channels(p["outlier_seed"], k))
    check_mlp(xb, wdev, wref, f"tp2 shard T={t}")


def test_launch_count_independent_of_T():
    """One launch set per batch, never one per token: the count is the same
    for every T of a size range -- 7 while the activation has at most 8192
    blocks of 16 (one-launch quantiser: T <= 341 at K = 384), 8 above -- and
    never exceeds 8.  (K = I = 384 is too short for the one/two-token stream and
    not a multiple of 256, so no weight stream is involved.)"""
    import mlp_prefill_amd as m
    wdev, _ = _weights(384, 384, (1, 2, 3))
    counts = {}
    for t in (1, 5, 64, 341, 342, 1024):
        announce(f"launch count T={t}")
        before = m.launch_count()
        run_device_mlp(bf16_normal(9, (t, 384)), wdev)
        counts[t] = m.launch_count() - before
    assert counts[1] == counts[5] == counts[64] == counts[341] == 7, counts     # T * 24 <= 8192 blocks
    assert counts[342] == counts[1024] == 8, counts                           # quantise 2, gate/up 3, down 3


@pytest.mark.parametrize("t,k,i", [(1000, 384, 1024), (1024, 5120, 17408)], ids=["T1000_K384_I1024", "T1024_K5120_I17408"])
def test_gate_up_deterministic_any_workspace(t, k, i):
    """Gate/up output (float32 H and H~) is bit-identical across calls
    whatever the workspace holds beforehand: no workspace word is read before
    the call writes it, and every reduction runs in a fixed order."""
    import mlp_prefill_amd as m
    announce(f"gate/up determinism T={t} K={k} I={i}")
    wdev, _ = _weights(k, i, (7001, 7002, 7003))
    xq = dev_quantize(bf16_normal(7004, (t, k)))
    need = m.mlp_gu_act_ws_bytes(t, k, i)
    outs = []
    for fill in (0x00, 0xFF, 0x5A):
        ws = torch.full((need,), fill, dtype=torch.uint8, device="cuda")
        hq = m.NVFP4.empty(t, i)
        m.nvfp4_mlp_gu_act(xq, wdev[0], wdev[1], hq, ws=ws)
        torch.cuda.synchronize()
        outs.append((ws[: t * i * 4].clone().cpu().numpy(), to_host(hq)))
    for h, hq in outs[1:]:
        assert np.array_equal(h, outs[0][0])
        assert_nvfp4_equal(hq, outs[0][1], "H~ across workspaces")
