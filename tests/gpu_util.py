"""Helpers for the GPU parity tests: device setup, host<->device NVFP4, metrics."""
import json
import os
import sys

import numpy as np
import pytest
import torch

from oracle import formats, quant
from synthetic import bf16_bits_to_f32

TOL = 2e-3   # max |y - y_ref| / max |y_ref|: the agreement bar for GEMM/MLP outputs


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test on a host without a GPU")
    import mlp_prefill_amd  # noqa: F401  (fails loudly when the library is missing)


def record(case, **stats):
    """Append one JSON line of parity statistics to the file named by the
    environment variable NVFP4_PARITY_LOG (nothing when it is unset)."""
    path = os.environ.get("NVFP4_PARITY_LOG")
    if not path:
        return
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "a") as f:
        f.write(json.dumps({"case": case, **{k: (float(v) if isinstance(v, (np.floating, float)) else v)
                                               for k, v in stats.items()}}) + "\n")


def announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev_bf16(bits):
    import mlp_prefill_amd as m
    return m.bf16_from_bits(np.ascontiguousarray(bits))


def dev_quantize(bits_or_f32, gs_mode=0, gs=None):
    """Quantise a host bf16 (uint16 bits) or float32 matrix on the device."""
    import mlp_prefill_amd as m
    if bits_or_f32.dtype == np.uint16:
        x = dev_bf16(bits_or_f32)
    else:
        x = torch.from_numpy(np.ascontiguousarray(bits_or_f32)).cuda()
    rows, cols = x.shape
    q = m.NVFP4.empty(rows, cols)
    if gs is not None:
        q.gscale.fill_(float(gs))
    m.nvfp4_quantize_act(x, q, gs_mode=gs_mode)
    return q


def to_host(q, rows=None):
    """Device NVFP4 -> oracle NVFP4 (host)."""
    torch.cuda.synchronize()
    codes = q.codes.cpu().numpy().reshape(-1, q.cols // 2)
    scales = q.scales.cpu().numpy().reshape(-1, q.cols // 16)
    gs = np.float32(q.gscale.cpu().numpy()[0])
    n = codes.shape[0] if rows is None else rows
    return quant.NVFP4(codes[:n], scales[:n], gs, n, q.cols)


def assert_nvfp4_equal(got, ref, what):
    assert got.gs.view(np.uint32) == np.float32(ref.gs).view(np.uint32), \
        f"{what}: gscale {got.gs!r} != {ref.gs!r}"
    bad_s = np.argwhere(got.scales != ref.scales)
    assert bad_s.size == 0, f"{what}: {len(bad_s)} scale mismatches, first {bad_s[:5].tolist()}"
    bad_c = np.argwhere(got.codes != ref.codes)
    assert bad_c.size == 0, f"{what}: {len(bad_c)} code-byte mismatches, first {bad_c[:5].tolist()}"


def max_norm_err(y, ref):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(y - ref)) / den) if den > 0 else float(np.max(np.abs(y)))


def assert_bf16_rounding_close(got, ref, fp32_tol=1e-5):
    """bf16 outputs: each element within bf16 rounding (at most 2^-8 of |value|,
    half a unit in the last of 8 significant bits) of the reference, plus the
    float32 accumulation noise `fp32_tol` * max|ref|."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    bound = 2.0 ** -8 * np.abs(ref) * (1 + 1e-6) + fp32_tol * np.max(np.abs(ref))
    bad = np.abs(got - ref) > bound
    assert not bad.any(), f"{int(bad.sum())} bf16 outputs beyond rounding, first {np.argwhere(bad)[:5].tolist()}"


def bf16_tensor_to_f32(t):
    torch.cuda.synchronize()
    return bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))


def legit_requant_flips(h32, hq_gpu, hq_ref, rel=2.0 ** -14):
    """Check that every place where two NVFP4 encodings of (nearly) the same
    float32 matrix differ is a rounding decision the oracle takes within
    `rel` (relative) of a boundary.  h32 is the oracle's RN32(H).

    Returns (number of differing elements, number of differing blocks).
    Raises AssertionError on a difference that is not near a boundary.
    """
    gs = np.float64(hq_ref.gs)
    rows, cols = h32.shape
    nb = cols // 16
    xb = np.abs(h32.astype(np.float64)).reshape(rows, nb, 16)
    amax_b = xb.max(-1)
    # block scales: the ratio amax_b / (6 gs) must sit near an E4M3 midpoint
    sdiff = hq_gpu.scales != hq_ref.scales
    if sdiff.any():
        r = amax_b[sdiff] / (6.0 * gs)
        mids = formats.E4M3_MIDS
        near = np.min(np.abs(r[:, None] - mids[None, :]) / mids[None, :], axis=1) <= rel
        assert np.all(near), f"{int((~near).sum())} block-scale differences away from any boundary"
    cg = quant.unpack_codes(hq_gpu.codes).reshape(rows, nb, 16)
    cr = quant.unpack_codes(hq_ref.codes).reshape(rows, nb, 16)
    # compare values, so that +0 and -0 (a sign disagreement at magnitude 0) agree
    cdiff = (formats.E2M1_TABLE[cg] != formats.E2M1_TABLE[cr]) & ~sdiff[..., None]
    if cdiff.any():
        d = formats.E4M3_TABLE[hq_ref.scales.astype(int)][..., None] * gs
        qv = (xb / np.where(d == 0, 1, d))[cdiff]
        mids = formats.E2M1_MIDS
        near = np.min(np.abs(qv[:, None] - mids[None, :]) / mids[None, :], axis=1) <= rel
        assert np.all(near), f"{int((~near).sum())} code differences away from any boundary"
    return int(cdiff.sum()), int(sdiff.sum())
