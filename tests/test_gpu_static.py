"""Static global scales on the device (warm-up scales, quantising GLU
epilogue, NVFP4-emitting down projection) vs the oracle.

Two kinds of check:
  * exact: the quantising epilogues must produce exactly the NVFP4 encoding
    of the float32 values the device's float32 paths compute (the float32 H
    of nvfp4_mlp_gu_act, the float32 Y of nvfp4_mlp_down), with the given
    global scale -- the quantisation itself is bit-exact;
  * staged end to end against the oracle's static MLP (x~ bit-exact, H~ flips
    only at rounding boundaries, flip-corrected Y within the tolerance).
"""
import numpy as np
import pytest
import torch

from oracle import gemm as ogemm
from oracle import mlp as omlp
from oracle import quant
from synthetic import WORKLOADS, bf16_bits_to_f32, bf16_normal, outlier_channels
from tests.gpu_util import (TOL, announce, assert_nvfp4_equal, dev_bf16, dev_quantize, legit_requant_flips,
                            max_norm_err, require_gpu, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


def _weights(k, i, seeds):
    mats = [bf16_normal(seeds[0], (i, k), sigma=0.02), bf16_normal(seeds[1], (i, k), sigma=0.02),
            bf16_normal(seeds[2], (k, i), sigma=0.02)]
    return [dev_quantize(b) for b in mats], [quant.quantize(bf16_bits_to_f32(b)) for b in mats]


def _with_gs(rows, cols, gs):
    import mlp_prefill_amd as m
    q = m.NVFP4.empty(rows, cols)
    q.gscale.fill_(float(gs))
    return q


GU_SHAPES = [(1, 256, 384), (5, 256, 384), (32, 384, 256), (37, 256, 384), (129, 384, 640), (1024, 5120, 17408)]


@pytest.mark.parametrize("t,k,i", GU_SHAPES, ids=[f"T{t}_K{k}_I{i}" for t, k, i in GU_SHAPES])
def test_gu_act_static_is_the_exact_quantisation_of_the_device_H(t, k, i):
    import mlp_prefill_amd as m
    announce(f"gu_act_static T={t} K={k} I={i}")
    wdev, _ = _weights(k, i, (8001, 8002, 8003))
    xq = dev_quantize(bf16_normal(8004 + t, (t, k)))
    hq_dyn = m.NVFP4.empty(t, i)
    ws = m.nvfp4_mlp_gu_act(xq, wdev[0], wdev[1], hq_dyn)
    torch.cuda.synchronize()
    h32 = ws[: t * i * 4].view(torch.float32).view(t, i).cpu().numpy().copy()
    gs_dyn = np.float32(hq_dyn.gscale.cpu().numpy()[0])
    # the dynamic scale itself, a coarser one and a finer one (saturating blocks)
    for gs in (gs_dyn, np.float32(gs_dyn * 2.5), np.float32(gs_dyn * 0.125)):
        hq = _with_gs(t, i, gs)
        m.nvfp4_mlp_gu_act_static(xq, wdev[0], wdev[1], hq)
        got = to_host(hq)
        ref = quant.quantize(h32, gs=gs)
        assert_nvfp4_equal(got, ref, f"T{t} gs={gs!r}")
        if gs == gs_dyn:
            assert_nvfp4_equal(got, to_host(hq_dyn), "static with the dynamic scale")
    assert (to_host(hq).scales == 0x7E).any()        # the finer scale saturated some blocks


DOWN_SHAPES = [(1, 384, 256), (5, 256, 384), (64, 512, 256), (129, 640, 384), (1024, 17408, 5120)]


@pytest.mark.parametrize("t,i,k", DOWN_SHAPES, ids=[f"T{t}_I{i}_K{k}" for t, i, k in DOWN_SHAPES])
def test_down_quant_is_the_exact_quantisation_of_the_device_Y(t, i, k):
    import mlp_prefill_amd as m
    announce(f"down_quant T={t} I={i} K={k}")
    hq = dev_quantize(bf16_normal(8101 + t, (t, i)))
    wd = dev_quantize(bf16_normal(8102, (k, i), sigma=0.02))
    y32 = torch.empty((t, k), dtype=torch.float32, device="cuda")
    m.nvfp4_mlp_down(hq, wd, y32)
    torch.cuda.synchronize()
    y = y32.cpu().numpy()
    gs0 = np.float32(np.abs(y).max() / 2688.0)
    for gs in (gs0, np.float32(gs0 * 0.2)):
        yq = _with_gs(t, k, gs)
        m.nvfp4_mlp_down_quant(hq, wd, yq)
        assert_nvfp4_equal(to_host(yq), quant.quantize(y, gs=gs), f"T{t} gs={gs!r}")
    # and the float32 Y itself is the oracle's product
    assert max_norm_err(y, ogemm.gemm(to_host(hq), quant.quantize(bf16_bits_to_f32(
        bf16_normal(8102, (k, i), sigma=0.02))))) <= 1e-5


def test_static_launch_counts_independent_of_T():
    """Expansion + contraction, and expansion + contraction + quantising
    reduction, at every T (K = I = 384: too short for the one/two-token stream
    and not a multiple of 256, so no weight stream is involved)."""
    import mlp_prefill_amd as m
    wdev, _ = _weights(384, 384, (8201, 8202, 8203))
    counts = []
    for t in (1, 5, 64, 1024):
        announce(f"static launch count T={t}")
        xq = dev_quantize(bf16_normal(8204, (t, 384)))
        hq = _with_gs(t, 384, 0.01)
        yq = _with_gs(t, 384, 0.01)
        b0 = m.launch_count()
        m.nvfp4_mlp_gu_act_static(xq, wdev[0], wdev[1], hq)
        b1 = m.launch_count()
        m.nvfp4_mlp_down_quant(hq, wdev[2], yq)
        b2 = m.launch_count()
        counts.append((b1 - b0, b2 - b1))
    assert set(counts) == {(2, 3)}, counts


def _device_warmup(xw_bits, wdev):
    """Dynamic device pass on the warm-up batch; returns its (gs_x, gs_h) as read back."""
    import mlp_prefill_amd as m
    xq = dev_quantize(xw_bits)
    hq = m.NVFP4.empty(xq.rows, wdev[0].rows)
    m.nvfp4_mlp_gu_act(xq, wdev[0], wdev[1], hq)
    torch.cuda.synchronize()
    return np.float32(xq.gscale.cpu().numpy()[0]), np.float32(hq.gscale.cpu().numpy()[0])


@pytest.mark.parametrize("t,k,i", [(37, 256, 384), (256, 1024, 2048), (1024, 5120, 17408)],
                         ids=["T37", "T256", "T1024_full"])
def test_static_mlp_end_to_end_vs_oracle(t, k, i):
    import mlp_prefill_amd as m
    announce(f"static mlp T={t} K={k} I={i}")
    wdev, wref = _weights(k, i, (8301, 8302, 8303))
    outl = outlier_channels(8305, k)
    gs_x, gs_h = _device_warmup(bf16_normal(8306, (t, k), outliers=outl), wdev)     # warm-up batch
    xbits = bf16_normal(8307, (t, k), outliers=outl)                               # the timed batch
    xq = dev_quantize(xbits, gs_mode=m.GS_GIVEN, gs=gs_x)
    hq = _with_gs(t, i, gs_h)
    m.nvfp4_mlp_gu_act_static(xq, wdev[0], wdev[1], hq)
    y = torch.empty((t, k), dtype=torch.float32, device="cuda")
    m.nvfp4_mlp_down(hq, wdev[2], y)
    torch.cuda.synchronize()
    ref = omlp.mlp_static(bf16_bits_to_f32(xbits), *wref, gs_x, gs_h)
    assert_nvfp4_equal(to_host(xq), ref["xq"], "x~ (static scale)")                      # S1
    hq_dev = to_host(hq)
    nflip, nsflip = legit_requant_flips(ref["h"].astype(np.float32), hq_dev, ref["hq"])  # S3
    yd = y.cpu().numpy()
    corr = ref["y"] + ogemm.gemm(hq_dev, wref[2]) - ogemm.gemm(ref["hq"], wref[2])
    e2e, ecorr = max_norm_err(yd, ref["y"]), max_norm_err(yd, corr)
    print(f"static T{t}: flips {nflip} codes / {nsflip} scales; Y e2e {e2e:.2e} flip-corrected {ecorr:.2e}")
    assert ecorr <= TOL                                                                  # S4


def test_two_layer_static_chain_through_down_quant():
    """Layer 0's down projection emits layer 1's NVFP4 input with layer 1's
    warm-up scale; the chain equals the oracle's static layers fed with the
    same encodings (each hand-over is checked exactly against the device's
    float32 Y of the same call)."""
    import mlp_prefill_amd as m
    t, k, i = 64, 512, 768
    announce("static 2-layer chain T=64")
    layers = [_weights(k, i, (8401 + 3 * l, 8402 + 3 * l, 8403 + 3 * l)) for l in range(2)]
    xw = bf16_normal(8410, (t, k))
    # warm-up: dynamic layer 0 (its bf16 output feeds layer 1's dynamic warm-up)
    gs_x0, gs_h0 = _device_warmup(xw, layers[0][0])
    xq0 = dev_quantize(xw)
    h0 = m.NVFP4.empty(t, i)
    m.nvfp4_mlp_gu_act(xq0, layers[0][0][0], layers[0][0][1], h0)
    yb = torch.empty((t, k), dtype=torch.bfloat16, device="cuda")
    m.nvfp4_mlp_down(h0, layers[0][0][2], yb)
    gs_x1, gs_h1 = _device_warmup(yb.view(torch.uint16).cpu().numpy(), layers[1][0])
    # the static chain on a new batch
    xbits = bf16_normal(8411, (t, k))
    xq = dev_quantize(xbits, gs_mode=m.GS_GIVEN, gs=gs_x0)
    hq0 = _with_gs(t, i, gs_h0)
    m.nvfp4_mlp_gu_act_static(xq, layers[0][0][0], layers[0][0][1], hq0)
    x1 = _with_gs(t, k, gs_x1)
    m.nvfp4_mlp_down_quant(hq0, layers[0][0][2], x1)
    hq1 = _with_gs(t, i, gs_h1)
    m.nvfp4_mlp_gu_act_static(x1, layers[1][0][0], layers[1][0][1], hq1)
    y = torch.empty((t, k), dtype=torch.float32, device="cuda")
    m.nvfp4_mlp_down(hq1, layers[1][0][2], y)
    y0 = torch.empty((t, k), dtype=torch.float32, device="cuda")
    m.nvfp4_mlp_down(hq0, layers[0][0][2], y0)
    torch.cuda.synchronize()
    # hand-over: exactly the quantisation of layer 0's float32 Y
    assert_nvfp4_equal(to_host(x1), quant.quantize(y0.cpu().numpy(), gs=gs_x1), "layer-1 input")
    # layer 0's H~ and layer 1 against the oracle, staged
    ref0 = omlp.mlp_static(bf16_bits_to_f32(xbits), *layers[0][1], gs_x0, gs_h0)
    legit_requant_flips(ref0["h"].astype(np.float32), to_host(hq0), ref0["hq"])
    h1, ref_hq1 = omlp.mlp_gu_act_static(to_host(x1), layers[1][1][0], layers[1][1][1], gs_h1)
    legit_requant_flips(h1.astype(np.float32), to_host(hq1), ref_hq1)
    corr = omlp.mlp_down(to_host(hq1), layers[1][1][2])
    assert max_norm_err(y.cpu().numpy(), corr) <= TOL


def _grouped_static_check(t, e, k, i, top, seed, sample_rows=None):
    """The expert-grouped gate/up with a given scale must give exactly the NVFP4
    encoding of the float32 GLU output the dynamic grouped call computes."""
    import mlp_prefill_amd as m
    from oracle import moe as omoe
    from synthetic import expert_seeds, router_logits
    r = omoe.route(router_logits(seed, t, e), top)
    slots = len(r.a_rows)
    mats = [[], []]
    for x in range(e):
        for j, (s, shp) in enumerate(zip(expert_seeds(seed + 1, x)[:2], [(i, k), (i, k)])):
            mats[j].append(dev_quantize(bf16_normal(s, shp, sigma=0.02)))
    wg, wu = m.NVFP4.stack(mats[0]), m.NVFP4.stack(mats[1])
    xq = dev_quantize(bf16_normal(seed + 2, (t, k)))
    rows = torch.from_numpy(np.ascontiguousarray(r.a_rows, dtype=np.int32)).cuda()
    offs = torch.from_numpy(np.ascontiguousarray(r.group_offsets, dtype=np.int32)).cuda()
    hq_dyn = m.NVFP4.empty(slots, i)
    ws = m.nvfp4_grouped_gemm(xq, rows, offs, wg, wu, out_q=hq_dyn, epilogue=m.EPI_SILU_MUL_REQUANT, m=slots)
    torch.cuda.synchronize()
    sel = np.arange(slots) if sample_rows is None else np.unique(np.linspace(0, slots - 1, sample_rows).astype(int))
    h32 = ws[: slots * i * 4].view(torch.float32).view(slots, i)[torch.from_numpy(sel).cuda()].cpu().numpy()
    gs_dyn = np.float32(hq_dyn.gscale.cpu().numpy()[0])
    need = m.grouped_ws_bytes(slots, i, k, e, m.EPI_SILU_MUL_QUANT_GIVEN)
    assert need == slots * k * 2 + (-(slots * k * 2)) % 256      # only the f16 copy of the gathered x~
    for gs in (gs_dyn, np.float32(gs_dyn * 0.25)):
        hq = _with_gs(slots, i, gs)
        m.nvfp4_grouped_gemm(xq, rows, offs, wg, wu, out_q=hq, epilogue=m.EPI_SILU_MUL_QUANT_GIVEN, m=slots)
        got = to_host(hq)
        got_sel = quant.NVFP4(got.codes[sel], got.scales[sel], got.gs, len(sel), i)
        assert_nvfp4_equal(got_sel, quant.quantize(h32, gs=gs), f"grouped static gs={gs!r}")


def test_grouped_static_scale_small_routed():
    announce("grouped gate/up static scale: 200 tokens, top-2 of 8 experts")
    _grouped_static_check(200, 8, 256, 384, 2, 9101)


def test_grouped_static_scale_moe_workload_sampled():
    p = WORKLOADS["moe_4096_top8_of_64"].params
    announce("grouped gate/up static scale: 4096 tokens, top-8 of 64 (sampled rows)")
    _grouped_static_check(p["T"], p["E"], p["K"], p["I"], p["topk"], 9201, sample_rows=3000)
