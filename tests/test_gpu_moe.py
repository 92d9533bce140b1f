"""Device expert routing and combine vs the oracle (oracle.moe).

Routing is integer work and compared bit for bit (expert ids, group offsets,
slot rows, slot of every choice); the float32 combine weights within 2e-6
(absolute, they lie in [0, 1]) of the float64 ones.  The combine is compared
with the oracle's float64 combine of the same slot outputs.  The full
expert-grouped MLP with device routing and combine is checked at a small
size; the 4096-token top-8-of-64 routing at full size.
"""
import numpy as np
import pytest
import torch

from oracle import moe as omoe
from synthetic import WORKLOADS, router_logits
from tests.gpu_util import announce, assert_bf16_rounding_close, bf16_tensor_to_f32, max_norm_err, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


def device_route(logits, k):
    import mlp_prefill_amd as m
    t, e = logits.shape
    lg = torch.from_numpy(np.ascontiguousarray(logits)).cuda()
    off = torch.full((e + 1,), -7, dtype=torch.int32, device="cuda")
    rows = torch.full((t * k,), -7, dtype=torch.int32, device="cuda")
    slot = torch.full((t, k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((t, k), -7.0, dtype=torch.float32, device="cuda")
    ws = torch.full((max(m.moe_route_ws_bytes(t, e, k), 256),), 0xAB, dtype=torch.uint8, device="cuda")  # garbage
    m.nvfp4_moe_route(lg, k, off, rows, slot, w, ws=ws)
    torch.cuda.synchronize()
    return off.cpu().numpy(), rows.cpu().numpy(), slot.cpu().numpy(), w.cpu().numpy()


def check_route(logits, k, label):
    announce(f"route: {label}")
    ref = omoe.route(logits, k)
    off, rows, slot, w = device_route(logits, k)
    assert np.array_equal(off, ref.group_offsets), "group offsets"
    assert np.array_equal(rows, ref.a_rows), "slot rows"
    assert np.array_equal(slot, ref.slot_of), "slot of each choice"
    err = float(np.max(np.abs(w - ref.weights))) if w.size else 0.0
    print(f"{label}: weights max abs err {err:.2e}")
    assert err <= 2e-6
    return ref


@pytest.mark.parametrize("t,e,k", [(1, 8, 2), (63, 8, 2), (64, 64, 8), (200, 64, 8), (333, 16, 16), (70, 300, 3),
                                   (100, 256, 8), (64, 65, 4), (65, 255, 16), (90, 128, 16), (64, 129, 8),
                                   (5, 4, 4), (129, 5, 1)])
def test_route_matches_oracle(t, e, k):
    check_route(router_logits(1000 + t + e + k, t, e), k, f"T={t} E={e} k={k}")


def test_route_ties_and_constant_rows():
    logits = router_logits(31, 130, 12)
    logits[::3] = np.round(logits[::3])          # many exact ties
    logits[5] = 0.25                             # one constant row
    logits[7, :] = -0.0
    logits[7, ::2] = 0.0                         # +0 and -0 tie
    check_route(logits, 5, "ties")


def test_route_full_size_moe_workload():
    p = WORKLOADS["moe_4096_top8_of_64"].params
    check_route(router_logits(p["router_seed"], p["T"], p["E"]), p["topk"], "T=4096 E=64 k=8")


def test_route_launch_count_independent_of_T():
    import mlp_prefill_amd as m
    counts = []
    for t in (1, 64, 4096):
        before = m.launch_count()
        device_route(router_logits(5, t, 64), 8)
        counts.append(m.launch_count() - before)
    assert counts == [3, 3, 3]


@pytest.mark.parametrize("in_dtype,out_dtype", [(torch.float32, torch.float32), (torch.bfloat16, torch.bfloat16),
                                                (torch.bfloat16, torch.float32)])
def test_combine_matches_oracle(in_dtype, out_dtype):
    import mlp_prefill_amd as m
    t, e, k, n = 150, 16, 4, 72
    announce(f"combine {in_dtype} -> {out_dtype}")
    ref = omoe.route(router_logits(44, t, e), k)
    rng = np.random.default_rng(45)
    ys = torch.from_numpy(rng.standard_normal((t * k, n)).astype(np.float32)).cuda().to(in_dtype)
    slot = torch.from_numpy(ref.slot_of).cuda()
    w = torch.from_numpy(ref.weights.astype(np.float32)).cuda()
    y = torch.empty((t, n), dtype=out_dtype, device="cuda")
    m.nvfp4_moe_combine(ys, slot, w, y)
    torch.cuda.synchronize()
    ys_h = ys.float().cpu().numpy()
    want = omoe.combine(ys_h, ref.slot_of, ref.weights.astype(np.float32))
    got = bf16_tensor_to_f32(y) if out_dtype == torch.bfloat16 else y.cpu().numpy()
    if out_dtype == torch.bfloat16:
        assert_bf16_rounding_close(got, want)
    else:
        err = max_norm_err(got, want)
        print(f"combine err {err:.2e}")
        assert err <= 1e-6


def test_moe_layer_with_device_routing_and_combine():
    """x -> quantise -> route (device) -> grouped gate/up + SiLU*up + requant ->
    grouped down -> combine, vs the oracle: routing bit-exact, the grouped MLP
    staged as in the grouped tests (requantisation flips near boundaries
    accounted for), the combine of the device's slot outputs tight, the end
    to end result reported."""
    import mlp_prefill_amd as m
    from oracle import mlp as omlp
    from oracle import quant
    from synthetic import bf16_bits_to_f32, bf16_normal, expert_seeds
    from tests.gpu_util import TOL, dev_bf16, dev_quantize, legit_requant_flips, to_host
    t, e, k, kk, ii = 96, 8, 2, 256, 384
    announce("moe layer: device routing, grouped MLP, combine")
    logits = router_logits(61, t, e)
    xb = bf16_normal(62, (t, kk))
    wd, wr = [[], [], []], [[], [], []]
    for x_ in range(e):
        for j, (sd, shp) in enumerate(zip(expert_seeds(6300, x_), [(ii, kk), (ii, kk), (kk, ii)])):
            bits = bf16_normal(sd, shp, sigma=0.02)
            wd[j].append(dev_quantize(bits))
            wr[j].append(quant.quantize(bf16_bits_to_f32(bits)))
    wd = [m.NVFP4.stack(v) for v in wd]
    # device
    lg = torch.from_numpy(logits).cuda()
    off = torch.empty(e + 1, dtype=torch.int32, device="cuda")
    rows = torch.empty(t * k, dtype=torch.int32, device="cuda")
    slot = torch.empty((t, k), dtype=torch.int32, device="cuda")
    w = torch.empty((t, k), dtype=torch.float32, device="cuda")
    m.nvfp4_moe_route(lg, k, off, rows, slot, w)
    xq = m.NVFP4.empty(t, kk)
    m.nvfp4_quantize_act(dev_bf16(xb), xq)
    hq = m.NVFP4.empty(t * k, ii)
    ws = m.nvfp4_grouped_gemm(xq, rows, off, wd[0], wd[1], out_q=hq, epilogue=m.EPI_SILU_MUL_REQUANT, m=t * k)
    ys = torch.empty((t * k, kk), dtype=torch.float32, device="cuda")
    m.nvfp4_grouped_gemm(hq, None, off, wd[2], out=ys, epilogue=m.EPI_STORE)
    y = torch.empty((t, kk), dtype=torch.float32, device="cuda")
    m.nvfp4_moe_combine(ys, slot, w, y)
    torch.cuda.synchronize()
    # oracle, staged
    r = omoe.route(logits, k)
    assert np.array_equal(off.cpu().numpy(), r.group_offsets) and np.array_equal(rows.cpu().numpy(), r.a_rows)
    assert np.array_equal(slot.cpu().numpy(), r.slot_of)
    xq_ref = quant.quantize(bf16_bits_to_f32(xb))
    g = omlp.grouped_mlp(xq_ref, r.a_rows, r.group_offsets, *wr)
    h = ws[: t * k * ii * 4].view(torch.float32).view(t * k, ii).cpu().numpy()
    assert max_norm_err(h, g["h"]) <= 1e-4
    hq_h = to_host(hq)
    legit_requant_flips(g["h"].astype(np.float32), hq_h, g["hq"])
    ys_h = ys.cpu().numpy()
    ys_corr = g["y"] + omlp.grouped_gemm(hq_h, None, r.group_offsets, wr[2]) - \
        omlp.grouped_gemm(g["hq"], None, r.group_offsets, wr[2])
    assert max_norm_err(ys_h, ys_corr) <= TOL
    comb = omoe.combine(ys_h, r.slot_of, w.cpu().numpy())            # combine of the device's slot outputs
    assert max_norm_err(y.cpu().numpy(), comb) <= 1e-6
    e2e = max_norm_err(y.cpu().numpy(), omoe.combine(g["y"], r.slot_of, r.weights))
    print(f"moe layer: end-to-end max-normalised error {e2e:.2e}")
