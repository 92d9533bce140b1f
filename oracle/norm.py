"""Oracle for RMSNorm fused into the NVFP4 activation quantiser.  TEST INFRASTRUCTURE ONLY.

The DSV4 audit page suggests folding the RMSNorm in front of an NVFP4 linear
into the linear's activation quantisation, since the quantiser already does an
amax-based normalisation (nvfp4-megamoe-kernel performance audit, P8 item 2;
the llama.cpp discussion lists a batched-row rms_norm among its fusions).  The
pages give no formula; the plainest reading is the usual RMSNorm with a
per-channel gain:

    y[r, c] = x[r, c] * gamma[c] / sqrt(mean_c x[r, c]^2 + eps)

computed here in float64.  The fused kernel forms y in float32 and quantises
it with a global scale over the whole call, exactly as the plain quantiser
does for x (amax, then block scales and codes).
"""
import numpy as np

from . import quant


def inv_rms(x, eps):
    """1 / sqrt(mean over the row of x^2 + eps), float64 [rows]."""
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / np.sqrt(np.mean(x * x, axis=1) + float(eps))


def rmsnorm(x, gamma, eps):
    """y = x * gamma / sqrt(mean(x^2) + eps) per row, float64."""
    x = np.asarray(x, dtype=np.float64)
    return x * inv_rms(x, eps)[:, None] * np.asarray(gamma, dtype=np.float64)[None, :]


def rmsnorm_quantize(x, gamma, eps):
    """NVFP4 of RN32(rmsnorm(x)) with a per-call global scale."""
    return quant.quantize(rmsnorm(x, gamma, eps).astype(np.float32))
