"""Expert-grouped NVFP4 GEMMs (one launch per GEMM, offsets on the device) vs the oracle."""
import numpy as np
import pytest
import torch

from oracle import gemm as ogemm
from oracle import mlp as omlp
from oracle import moe as omoe
from oracle import quant
from synthetic import WORKLOADS, bf16_bits_to_f32, bf16_normal, expert_seeds, router_logits
from tests.gpu_util import (TOL, announce, assert_bf16_rounding_close, assert_nvfp4_equal, bf16_tensor_to_f32,
                            dev_quantize, legit_requant_flips, max_norm_err, require_gpu, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


def _experts(e, k, i, seed0, with_ref=True):
    import mlp_prefill_amd as m
    dev = [[], [], []]
    ref = [[], [], []]
    for x in range(e):
        for j, (s, shp) in enumerate(zip(expert_seeds(seed0, x), [(i, k), (i, k), (k, i)])):
            bits = bf16_normal(s, shp, sigma=0.02)
            dev[j].append(dev_quantize(bits))
            if with_ref:
                ref[j].append(quant.quantize(bf16_bits_to_f32(bits)))
    return [m.NVFP4.stack(d) for d in dev], ref


def _run_grouped_mlp(xq, a_rows, offsets, wdev, m_slots, k, i):
    import mlp_prefill_amd as m
    rows = torch.from_numpy(np.ascontiguousarray(a_rows, dtype=np.int32)).cuda()
    offs = torch.from_numpy(np.ascontiguousarray(offsets, dtype=np.int32)).cuda()
    hq = m.NVFP4.empty(m_slots, i)
    ws = m.nvfp4_grouped_gemm(xq, rows, offs, wdev[0], wdev[1], out_q=hq, epilogue=m.EPI_SILU_MUL_REQUANT,
                              m=m_slots)
    y = torch.empty((m_slots, k), dtype=torch.float32, device="cuda")
    m.nvfp4_grouped_gemm(hq, None, offs, wdev[2], out=y, epilogue=m.EPI_STORE)
    torch.cuda.synchronize()
    h = ws[: m_slots * i * 4].view(torch.float32).view(m_slots, i).cpu().numpy()
    return h, to_host(hq), y.cpu().numpy()


def _check_small(t, e, k, i, a_rows, offsets, seed):
    xb = bf16_normal(seed, (t, k))
    xq = dev_quantize(xb)
    wdev, wref = _experts(e, k, i, seed + 100)
    m_slots = len(a_rows)
    h, hq, y = _run_grouped_mlp(xq, a_rows, offsets, wdev, m_slots, k, i)
    xq_ref = quant.quantize(bf16_bits_to_f32(xb))
    assert_nvfp4_equal(to_host(xq), xq_ref, "x~")
    ref = omlp.grouped_mlp(xq_ref, a_rows, offsets, *wref)
    eh = max_norm_err(h, ref["h"])
    nflip, nsflip = legit_requant_flips(ref["h"].astype(np.float32), hq, ref["hq"])
    corr = ref["y"] + omlp.grouped_gemm(hq, None, offsets, wref[2]) - omlp.grouped_gemm(ref["hq"], None, offsets, wref[2])
    ey, ecorr = max_norm_err(y, ref["y"]), max_norm_err(y, corr)
    print(f"grouped T={t} E={e}: H err {eh:.2e}  flips {nflip}/{nsflip}  Y err {ey:.2e}  corrected {ecorr:.2e}")
    assert eh <= 1e-4
    assert abs(float(hq.gs) / float(ref["hq"].gs) - 1.0) <= 2.0 ** -16
    assert ecorr <= TOL


def test_grouped_mlp_routed_top2():
    announce("grouped mlp: 96 tokens, top-2 of 8 experts")
    r = omoe.route(router_logits(55, 96, 8), 2)
    _check_small(96, 8, 256, 384, r.a_rows, r.group_offsets, 56)


def test_grouped_mlp_edge_groups():
    # empty expert, one-row expert, ragged experts, repeated tokens
    announce("grouped mlp: empty / one-row / ragged groups")
    rng = np.random.default_rng(9)
    offsets = np.array([0, 0, 1, 40, 57, 57], dtype=np.int32)
    a_rows = rng.integers(0, 30, size=57).astype(np.int32)
    _check_small(30, 5, 256, 256, a_rows, offsets, 77)


def test_grouped_store_gemm_matches_per_expert_gemm():
    import mlp_prefill_amd as m
    announce("grouped store gemm: 3 experts")
    t, k, n = 40, 384, 256
    xb = bf16_normal(3, (t, k))
    xq = dev_quantize(xb)
    xq_ref = quant.quantize(bf16_bits_to_f32(xb))
    wbits = [bf16_normal(10 + x, (n, k), sigma=0.02) for x in range(3)]
    wdev = m.NVFP4.stack([dev_quantize(b) for b in wbits])
    wref = [quant.quantize(bf16_bits_to_f32(b)) for b in wbits]
    a_rows = np.array(list(range(0, 40, 2)) + list(range(1, 40, 2)) + [5, 6, 7], dtype=np.int32)
    offsets = np.array([0, 20, 40, 43], dtype=np.int32)
    out = torch.empty((43, n), dtype=torch.float32, device="cuda")
    m.nvfp4_grouped_gemm(xq, torch.from_numpy(a_rows).cuda(), torch.from_numpy(offsets).cuda(), wdev, out=out)
    torch.cuda.synchronize()
    err = max_norm_err(out.cpu().numpy(), omlp.grouped_gemm(xq_ref, a_rows, offsets, wref))
    print(f"grouped store gemm error {err:.2e}")
    assert err <= 1e-5


@pytest.mark.parametrize("offsets", [[0, 20, 20, 43], [0, 0, 43, 43], [0, 13, 30, 43]],
                         ids=["empty_middle", "one_nonempty", "three"])
def test_grouped_store_gemm_split_k(offsets):
    """Few tiles and a long K: the store contraction splits K and the fixed-order
    reduction scales each slot by its expert's weight scale (the expert found from
    the offsets, with empty experts sharing an offset); bf16 output."""
    import mlp_prefill_amd as m
    announce(f"grouped store gemm, split K, offsets {offsets}")
    t, k, n, e = 40, 4096, 256, 3
    assert m.grouped_ws_bytes(43, n, k, e, m.EPI_STORE) > 43 * k * 2 + 43 * n * 4   # more than one split
    xb = bf16_normal(31, (t, k))
    xq = dev_quantize(xb)
    xq_ref = quant.quantize(bf16_bits_to_f32(xb))
    # weight scales differ by expert (sigma 0.02, 0.05, 0.1), so a wrong expert shows
    wbits = [bf16_normal(40 + x, (n, k), sigma=(0.02, 0.05, 0.1)[x]) for x in range(e)]
    wdev = m.NVFP4.stack([dev_quantize(b) for b in wbits])
    wref = [quant.quantize(bf16_bits_to_f32(b)) for b in wbits]
    a_rows = np.array([(7 * s) % t for s in range(43)], dtype=np.int32)
    offs = np.array(offsets, dtype=np.int32)
    out = torch.empty((43, n), dtype=torch.bfloat16, device="cuda")
    m.nvfp4_grouped_gemm(xq, torch.from_numpy(a_rows).cuda(), torch.from_numpy(offs).cuda(), wdev, out=out)
    ref = omlp.grouped_gemm(xq_ref, a_rows, offs, wref)
    assert_bf16_rounding_close(bf16_tensor_to_f32(out), ref)


def test_grouped_mlp_moe_workload_full_size_sampled():
    """T=4096 routed top-8 over 64 experts, hidden 4096, expert width 2048.

    The device runs every expert (one grouped launch per GEMM).  Checked on a
    sample of experts: H against the oracle (independent of the global scale
    of H), the requantisation of the device's H (global scale and codes,
    bit-exact), and the down projection of the device's H~.
    """
    import mlp_prefill_amd as m
    p = WORKLOADS["moe_4096_top8_of_64"].params
    t, e, top, k, i = p["T"], p["E"], p["topk"], p["K"], p["I"]
    announce("grouped mlp: MoE workload full size (sampled experts)")
    r = omoe.route(router_logits(p["router_seed"], t, e), top)
    xb = bf16_normal(p["x_seed"], (t, k))
    xq = dev_quantize(xb)
    wdev, _ = _experts(e, k, i, p["expert_seed0"], with_ref=False)
    m_slots = t * top
    h, hq, y = _run_grouped_mlp(xq, r.a_rows, r.group_offsets, wdev, m_slots, k, i)
    xq_ref = quant.quantize(bf16_bits_to_f32(xb))
    assert_nvfp4_equal(to_host(xq), xq_ref, "x~")
    # the global scale of H~ is the device H's amax / 2688, rounded once
    assert hq.gs == quant.global_scale(h)
    sample = [0, 17, 63]
    for x in sample:
        s0, s1 = int(r.group_offsets[x]), int(r.group_offsets[x + 1])
        wg, wu, wd = [quant.quantize(bf16_bits_to_f32(bf16_normal(s, shp, sigma=0.02)))
                      for s, shp in zip(expert_seeds(p["expert_seed0"], x), [(i, k), (i, k), (k, i)])]
        href, _ = omlp.mlp_gu_act(xq_ref.take_rows(r.a_rows[s0:s1]), wg, wu)
        eh = max_norm_err(h[s0:s1], href)
        got = quant.NVFP4(hq.codes[s0:s1], hq.scales[s0:s1], hq.gs, s1 - s0, i)
        assert_nvfp4_equal(got, quant.quantize(h[s0:s1], gs=hq.gs), f"expert {x} requant")
        ey = max_norm_err(y[s0:s1], ogemm.gemm(got, wd))
        print(f"expert {x}: {s1 - s0} slots, H err {eh:.2e}, down err {ey:.2e}")
        assert eh <= 1e-4
        assert ey <= 1e-5
