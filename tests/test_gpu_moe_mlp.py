"""The expert MLP in one call (nvfp4_moe_mlp) against the separate calls.

nvfp4_moe_mlp quantises x once (also writing its f16 copy), runs the grouped
gate/up staging each slot's token row of that copy (no gathering expansion),
requantises H (also writing the f16 copy of H~) and runs the grouped down
projection on that copy (no expansion).  Its outputs must equal, bit for bit,
those of nvfp4_quantize_act + nvfp4_grouped_gemm (SiLU*up + requantisation) +
nvfp4_grouped_gemm (store), which are staged against the oracle in
test_gpu_grouped.py; here also the launch count, empty and one-row experts,
repeated tokens, bf16 input and output, the full 4096-token workload, and the
tile-contiguous weight copies.

nvfp4_moe_mlp_static (given global scales) likewise against
nvfp4_quantize_act with NVFP4_GS_GIVEN + nvfp4_grouped_gemm (SiLU*up
quantised with the given scale) + nvfp4_grouped_gemm (store): four launches,
its gate/up epilogue also writing the f16 copy of H~ the down projection
stages.
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import moe as omoe
from synthetic import WORKLOADS, bf16_normal, expert_seeds, router_logits
from tests.gpu_util import announce, dev_bf16, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


def _experts(e, k, i, seed0):
    import mlp_prefill_amd as m
    mats = [[], [], []]
    for x in range(e):
        for j, (s, shp) in enumerate(zip(expert_seeds(seed0, x), [(i, k), (i, k), (k, i)])):
            w = m.bf16_from_bits(bf16_normal(s, shp, sigma=0.02))
            q = m.NVFP4.empty(*shp)
            m.nvfp4_quantize_act(w, q)
            mats[j].append(q)
    return [m.NVFP4.stack(v) for v in mats]


def _separate(x, rows, offs, w, m_slots, y_dtype):
    import mlp_prefill_amd as m
    t, k = x.shape
    i = w[0].rows
    xq = m.NVFP4.empty(t, k)
    m.nvfp4_quantize_act(x, xq)
    hq = m.NVFP4.empty(m_slots, i)
    m.nvfp4_grouped_gemm(xq, rows, offs, w[0], w[1], out_q=hq, epilogue=m.EPI_SILU_MUL_REQUANT, m=m_slots)
    y = torch.empty((m_slots, k), dtype=y_dtype, device="cuda")
    m.nvfp4_grouped_gemm(hq, None, offs, w[2], out=y, epilogue=m.EPI_STORE)
    torch.cuda.synchronize()
    return xq, hq, y


def _fused(x, rows, offs, w, m_slots, y_dtype):
    import mlp_prefill_amd as m
    t, k = x.shape
    i = w[0].rows
    xq, hq = m.NVFP4.empty(t, k), m.NVFP4.empty(m_slots, i)
    y = torch.empty((m_slots, k), dtype=y_dtype, device="cuda")
    ws = torch.empty(m.moe_mlp_ws_bytes(t, k, i, w[0].gscale.numel(), m_slots), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    before = m.launch_count()
    m.nvfp4_moe_mlp(x, rows, offs, w[0], w[1], w[2], xq, hq, y, ws=ws)
    launches = m.launch_count() - before
    torch.cuda.synchronize()
    return xq, hq, y, launches


def _same(a, b, what):
    assert torch.equal(a, b), f"{what}: the one-call expert MLP differs from the separate calls"


def _check(x, a_rows, offsets, w, y_dtype=torch.float32):
    rows = torch.from_numpy(np.ascontiguousarray(a_rows, dtype=np.int32)).cuda()
    offs = torch.from_numpy(np.ascontiguousarray(offsets, dtype=np.int32)).cuda()
    m_slots = len(a_rows)
    xq0, hq0, y0 = _separate(x, rows, offs, w, m_slots, y_dtype)
    xq1, hq1, y1, launches = _fused(x, rows, offs, w, m_slots, y_dtype)
    for f in ("codes", "scales", "gscale"):
        _same(getattr(xq0, f), getattr(xq1, f), f"x~ {f}")
        _same(getattr(hq0, f), getattr(hq1, f), f"H~ {f}")
    _same(y0, y1, "y_slots")
    # quantise (one launch up to 8192 blocks of 16, else amax pass + quantise),
    # gate/up, requantise, down, split reduction
    assert launches == (5 if x.shape[0] * x.shape[1] // 16 <= 8192 else 6), launches


def test_moe_mlp_routed_top2():
    announce("one-call expert MLP: 96 tokens, top-2 of 8 experts")
    r = omoe.route(router_logits(55, 96, 8), 2)
    w = _experts(8, 256, 384, 156)
    _check(dev_bf16(bf16_normal(56, (96, 256))), r.a_rows, r.group_offsets, w)


def test_moe_mlp_edge_groups_bf16():
    """Empty experts, a one-row expert, repeated tokens; bf16 y and float32 x."""
    announce("one-call expert MLP: empty / one-row / ragged groups, bf16 out")
    rng = np.random.default_rng(9)
    offsets = np.array([0, 0, 1, 40, 57, 57], dtype=np.int32)
    a_rows = rng.integers(0, 30, size=57).astype(np.int32)
    w = _experts(5, 256, 256, 177)
    x = dev_bf16(bf16_normal(77, (30, 256))).float()
    _check(x, a_rows, offsets, w, torch.bfloat16)


def test_moe_mlp_workload_full_size_tiled():
    """T=4096 routed top-8 over 64 experts, hidden 4096, expert width 2048,
    with the weights' tile-contiguous copies in the one-call path only."""
    import mlp_prefill_amd as m
    p = WORKLOADS["moe_4096_top8_of_64"].params
    t, e, top, k, i = p["T"], p["E"], p["topk"], p["K"], p["I"]
    announce("one-call expert MLP: MoE workload full size, tiled weights")
    r = omoe.route(router_logits(p["router_seed"], t, e), top)
    w = _experts(e, k, i, p["expert_seed0"])
    wt = []
    for q in w:
        c = dataclasses.replace(q, tiled=None)
        c.tile()
        wt.append(c)
    x = dev_bf16(bf16_normal(p["x_seed"], (t, k)))
    rows = torch.from_numpy(np.ascontiguousarray(r.a_rows, dtype=np.int32)).cuda()
    offs = torch.from_numpy(np.ascontiguousarray(r.group_offsets, dtype=np.int32)).cuda()
    m_slots = t * top
    xq0, hq0, y0 = _separate(x, rows, offs, w, m_slots, torch.bfloat16)
    xq1, hq1, y1, launches = _fused(x, rows, offs, wt, m_slots, torch.bfloat16)
    for f in ("codes", "scales", "gscale"):
        _same(getattr(xq0, f), getattr(xq1, f), f"x~ {f}")
        _same(getattr(hq0, f), getattr(hq1, f), f"H~ {f}")
    _same(y0, y1, "y_slots")
    assert launches == 6, launches
    # no workspace word is read before the call writes it: a call on a
    # workspace filled with 0xA5 bytes gives the same bits
    ws = torch.full((m.moe_mlp_ws_bytes(t, k, i, e, m_slots),), 0xA5, dtype=torch.uint8, device="cuda")
    y2 = torch.empty_like(y1)
    xq2, hq2 = m.NVFP4.empty(t, k), m.NVFP4.empty(m_slots, i)
    m.nvfp4_moe_mlp(x, rows, offs, wt[0], wt[1], wt[2], xq2, hq2, y2, ws=ws)
    torch.cuda.synchronize()
    _same(y1, y2, "y_slots on a dirty workspace")


# ---- static global scales: nvfp4_moe_mlp_static ---------------------------------------


def _separate_static(x, rows, offs, w, m_slots, y_dtype, gx, gh):
    import mlp_prefill_amd as m
    t, k = x.shape
    i = w[0].rows
    xq = m.NVFP4.empty(t, k)
    xq.gscale.fill_(gx)
    m.nvfp4_quantize_act(x, xq, gs_mode=m.GS_GIVEN)
    hq = m.NVFP4.empty(m_slots, i)
    hq.gscale.fill_(gh)
    m.nvfp4_grouped_gemm(xq, rows, offs, w[0], w[1], out_q=hq, epilogue=m.EPI_SILU_MUL_QUANT_GIVEN, m=m_slots)
    y = torch.empty((m_slots, k), dtype=y_dtype, device="cuda")
    m.nvfp4_grouped_gemm(hq, None, offs, w[2], out=y, epilogue=m.EPI_STORE)
    torch.cuda.synchronize()
    return xq, hq, y


def _fused_static(x, rows, offs, w, m_slots, y_dtype, gx, gh, ws=None):
    import mlp_prefill_amd as m
    t, k = x.shape
    i = w[0].rows
    xq, hq = m.NVFP4.empty(t, k), m.NVFP4.empty(m_slots, i)
    xq.gscale.fill_(gx)
    hq.gscale.fill_(gh)
    y = torch.empty((m_slots, k), dtype=y_dtype, device="cuda")
    if ws is None:
        ws = torch.empty(m.moe_mlp_ws_bytes(t, k, i, w[0].gscale.numel(), m_slots, static=True), dtype=torch.uint8,
                         device="cuda")
    torch.cuda.synchronize()
    before = m.launch_count()
    m.nvfp4_moe_mlp_static(x, rows, offs, w[0], w[1], w[2], xq, hq, y, ws=ws)
    launches = m.launch_count() - before
    torch.cuda.synchronize()
    return xq, hq, y, launches


def _check_static(x, a_rows, offsets, w, y_dtype=torch.float32, gx=0.002, gh=0.003):
    rows = torch.from_numpy(np.ascontiguousarray(a_rows, dtype=np.int32)).cuda()
    offs = torch.from_numpy(np.ascontiguousarray(offsets, dtype=np.int32)).cuda()
    m_slots = len(a_rows)
    xq0, hq0, y0 = _separate_static(x, rows, offs, w, m_slots, y_dtype, gx, gh)
    xq1, hq1, y1, launches = _fused_static(x, rows, offs, w, m_slots, y_dtype, gx, gh)
    for f in ("codes", "scales", "gscale"):
        _same(getattr(xq0, f), getattr(xq1, f), f"static x~ {f}")
        _same(getattr(hq0, f), getattr(hq1, f), f"static H~ {f}")
    _same(y0, y1, "static y_slots")
    # quantise x with its given scale, gate/up with the quantising epilogue, down, split reduction
    assert launches == 4, launches
    return xq1, hq1, y1


def test_moe_mlp_static_routed_top2():
    announce("one-call expert MLP, static scales: 96 tokens, top-2 of 8 experts")
    r = omoe.route(router_logits(57, 96, 8), 2)
    w = _experts(8, 256, 384, 158)
    _check_static(dev_bf16(bf16_normal(58, (96, 256))), r.a_rows, r.group_offsets, w)


def test_moe_mlp_static_edge_groups_bf16():
    """Empty experts, a one-row expert, repeated tokens; bf16 y and float32 x."""
    announce("one-call expert MLP, static scales: empty / one-row / ragged groups, bf16 out")
    rng = np.random.default_rng(11)
    offsets = np.array([0, 0, 1, 40, 57, 57], dtype=np.int32)
    a_rows = rng.integers(0, 30, size=57).astype(np.int32)
    w = _experts(5, 256, 256, 179)
    x = dev_bf16(bf16_normal(79, (30, 256))).float()
    _check_static(x, a_rows, offsets, w, torch.bfloat16, gx=0.0015, gh=0.0005)


def test_moe_mlp_static_workload_full_size_tiled():
    """T=4096 routed top-8 over 64 experts with the weights' tile-contiguous
    copies in the one-call path only, scales from a dynamic pass; a second
    call on a workspace filled with 0xA5 bytes gives the same bits."""
    import mlp_prefill_amd as m
    p = WORKLOADS["moe_4096_top8_of_64"].params
    t, e, top, k, i = p["T"], p["E"], p["topk"], p["K"], p["I"]
    announce("one-call expert MLP, static scales: MoE workload full size, tiled weights")
    r = omoe.route(router_logits(p["router_seed"], t, e), top)
    w = _experts(e, k, i, p["expert_seed0"])
    wt = []
    for q in w:
        c = dataclasses.replace(q, tiled=None)
        c.tile()
        wt.append(c)
    x = dev_bf16(bf16_normal(p["x_seed"], (t, k)))
    rows = torch.from_numpy(np.ascontiguousarray(r.a_rows, dtype=np.int32)).cuda()
    offs = torch.from_numpy(np.ascontiguousarray(r.group_offsets, dtype=np.int32)).cuda()
    m_slots = t * top
    # the scales a calibration (dynamic) pass measures
    xd, hd, _, _ = _fused(x, rows, offs, w, m_slots, torch.bfloat16)
    gx, gh = float(xd.gscale.item()), float(hd.gscale.item())
    xq0, hq0, y0 = _separate_static(x, rows, offs, w, m_slots, torch.bfloat16, gx, gh)
    xq1, hq1, y1, launches = _fused_static(x, rows, offs, wt, m_slots, torch.bfloat16, gx, gh)
    for f in ("codes", "scales", "gscale"):
        _same(getattr(xq0, f), getattr(xq1, f), f"static x~ {f}")
        _same(getattr(hq0, f), getattr(hq1, f), f"static H~ {f}")
    _same(y0, y1, "static y_slots")
    assert launches == 4, launches
    ws = torch.full((m.moe_mlp_ws_bytes(t, k, i, e, m_slots, static=True),), 0xA5, dtype=torch.uint8, device="cuda")
    _, _, y2, _ = _fused_static(x, rows, offs, wt, m_slots, torch.bfloat16, gx, gh, ws=ws)
    _same(y1, y2, "static y_slots on a dirty workspace")
