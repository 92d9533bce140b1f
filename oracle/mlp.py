"""The NVFP4 W4A4 MLP: gate/up, SiLU(gate)*up, requantisation, down projection.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Steps, in the order the pages give them:

1. The activation x (bf16, read exactly as float32) is quantised once on the
   device with a per-call global scale (DSV4 audit page, section P0; vllm.cpp
   issue, "Fix directions" 3) and that one quantised activation feeds both the
   gate and the up projection (llama.cpp discussion, "What the patch does").
2. G = x~ . Wg~^T and U = x~ . Wu~^T (exact, `gemm`), computed for the whole
   batch of T tokens at once (vllm.cpp issue, "Fix directions" 1).
3. H = SiLU(G) * U with SiLU(g) = g / (1 + e^-g), in float64.  Which projection
   is the gate is not stated on the pages; the gate is the operand under SiLU.
4. H is quantised straight into the down projection's NVFP4 input format,
   with no wider intermediate tensor in between (the llama.cpp discussion's
   patch fuses the GLU with the quantisation of the next matrix product's
   activation), with a per-call global scale over the whole [T, I] tensor.  The float64 H is first
   rounded to float32 (RN32), the precision a device epilogue holds it in; it
   is not rounded to bf16.
5. Y = H~ . Wd~^T (exact), reported in float64; a device emits it as float32
   (parity) or bf16 (the next layer's input).

Stacked layers (vllm.cpp issue, "Fix directions" 2: activations stay on the
device): each layer's output becomes the next layer's input as
bf16(RN32(Y)), round-to-nearest-even.  No residual and no norm sit between the
layers -- the pages do not describe any around the MLP.  Each call (one ubatch
through one layer) computes its own activation global scales.

Static global scales (DSV4 audit page, section P0, fix 1): the activation
global scales are measured once, by a warm-up forward pass, kept on the
device, and used as given by every later call.  With the scale of H known in
advance, the GLU output can be quantised by the producer itself, and the down
projection can emit the next layer's NVFP4 input directly (same page, section
P8, item 1: quantise in the producer's epilogue instead of writing a
wide-precision tensor for the consumer to re-read).  Reading taken: the
warm-up scales are the ones the dynamic path computes on the warm-up batch,
unchanged (no margin); later inputs beyond 6 * 448 * gs saturate (block scale
448, codes +-6); the down output that is quantised is RN32 of Y (float32, no
bf16 step in between).

Grouped (expert) variant: slots are token rows gathered by `a_rows`, grouped by
expert through `group_offsets`; each expert applies its own weights (with their
own global scales) to its slots; the GLU output of all slots shares one global
scale (one requantisation per call).
"""
import numpy as np

from . import quant
from .gemm import gemm


def silu(g):
    """g / (1 + exp(-g)) in float64 (exp overflow for g << 0 gives -0.0, the limit)."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def glu(gate, up):
    """H = SiLU(gate) * up, float64."""
    return silu(gate) * np.asarray(up, dtype=np.float64)


def requantize(h):
    """Quantise the GLU output: RN32 first, then NVFP4 with its own global scale."""
    return quant.quantize(np.asarray(h, dtype=np.float64).astype(np.float32))


def mlp_gu_act(xq, w_gate, w_up):
    """Gate/up on one shared quantised activation; returns H (float64) and H~."""
    h = glu(gemm(xq, w_gate), gemm(xq, w_up))
    return h, requantize(h)


def mlp_down(hq, w_down):
    """Y = H~ . Wd~^T, float64."""
    return gemm(hq, w_down)


def mlp(x, w_gate, w_up, w_down):
    """One MLP call on float32 activations x [T, K]; returns every stage."""
    xq = quant.quantize(x)
    h, hq = mlp_gu_act(xq, w_gate, w_up)
    y = mlp_down(hq, w_down)
    return {"xq": xq, "h": h, "hq": hq, "y": y}


def warmup_scales(x_warm, w_gate, w_up):
    """Global scales (gs_x, gs_h) that the dynamic path computes on a warm-up batch."""
    xq = quant.quantize(np.asarray(x_warm, dtype=np.float32))
    _, hq = mlp_gu_act(xq, w_gate, w_up)
    return np.float32(xq.gs), np.float32(hq.gs)


def mlp_gu_act_static(xq, w_gate, w_up, gs_h):
    """Gate/up with the given global scale for H~; returns H (float64) and H~."""
    h = glu(gemm(xq, w_gate), gemm(xq, w_up))
    return h, quant.quantize(h.astype(np.float32), gs=gs_h)


def mlp_down_quant(hq, w_down, gs_y):
    """Down projection emitting NVFP4 with the given global scale: NVFP4(RN32(Y))."""
    return quant.quantize(gemm(hq, w_down).astype(np.float32), gs=gs_y)


def mlp_static(x, w_gate, w_up, w_down, gs_x, gs_h):
    """One MLP call with static global scales for x~ and H~; returns every stage."""
    xq = quant.quantize(np.asarray(x, dtype=np.float32), gs=gs_x)
    h, hq = mlp_gu_act_static(xq, w_gate, w_up, gs_h)
    y = mlp_down(hq, w_down)
    return {"xq": xq, "h": h, "hq": hq, "y": y}


def bf16_round(x):
    """Round float32 values to bf16 (nearest, ties to even) and return them as float32."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def stacked_mlp(x, layers, ubatch):
    """x [T, K] float32 through `layers` [(Wg~, Wu~, Wd~), ...] in ubatches of `ubatch` rows.

    Returns the last layer's float64 output Y [T, K] and the list of each
    layer's bf16 (as float32) outputs, which are the inputs of the next layer.
    """
    x = np.asarray(x, dtype=np.float32)
    t = x.shape[0]
    y_last = np.zeros((t, layers[-1][2].rows), dtype=np.float64)
    chained = [np.zeros((t, layer[2].rows), dtype=np.float32) for layer in layers]
    for u0 in range(0, t, ubatch):
        cur = x[u0:u0 + ubatch]
        for li, (wg, wu, wd) in enumerate(layers):
            y = mlp(cur, wg, wu, wd)["y"]
            cur = bf16_round(y.astype(np.float32))
            chained[li][u0:u0 + ubatch] = cur
            if li == len(layers) - 1:
                y_last[u0:u0 + ubatch] = y
    return y_last, chained


def _groups(group_offsets):
    off = np.asarray(group_offsets, dtype=np.int64)
    return [(e, int(off[e]), int(off[e + 1])) for e in range(len(off) - 1)]


def grouped_gemm(aq, a_rows, group_offsets, w_list):
    """Per-expert C[slots of e] = gather(A~, a_rows)[slots of e] . W~_e^T (float64)."""
    a_rows = np.arange(aq.rows) if a_rows is None else np.asarray(a_rows, dtype=np.int64)
    out = np.zeros((len(a_rows), w_list[0].rows), dtype=np.float64)
    for e, s0, s1 in _groups(group_offsets):
        if s1 > s0:
            out[s0:s1] = gemm(aq.take_rows(a_rows[s0:s1]), w_list[e])
    return out


def grouped_mlp(xq, a_rows, group_offsets, wg_list, wu_list, wd_list):
    """Expert-grouped MLP on the shared quantised activation xq.

    Returns H (float64, [slots, I]), H~ (one global scale over all slots) and
    Y (float64, [slots, K]) in slot order.
    """
    g = grouped_gemm(xq, a_rows, group_offsets, wg_list)
    u = grouped_gemm(xq, a_rows, group_offsets, wu_list)
    h = glu(g, u)
    hq = requantize(h)
    y = grouped_gemm(hq, None, group_offsets, wd_list)
    return {"h": h, "hq": hq, "y": y}
