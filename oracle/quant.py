"""NVFP4 quantisation, written out from its definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is quantised and how (readings of the pages, which leave most of the
format unstated):

* Global scale.  gs = amax / (6 * 448) with amax = max|x| over the whole tensor
  of this call, clamped below at 1e-8; this is the runtime activation global
  scale of the DSV4 audit page (section P0, "Per-call .item() D2H sync inside
  every NVFP4 linear"), there evaluated in Python float64 and stored as a
  float32.  Rounding the float64 quotient of two float32 operands to float32
  gives the correctly rounded float32 quotient (53 >= 2*24 + 2), so
  gs = RN32(max(amax, RN32(1e-8)) / 2688).
* Block scale.  One E4M3 scale per 16 consecutive elements along a row (the
  K direction).  S = RNE_E4M3(amax_b / (6 * gs)) in exact real arithmetic,
  saturating at 448, subnormals kept, exact ties to the even code.
* Element codes.  q = RNE_E2M1(x / (dec(S) * gs)) in exact real arithmetic,
  saturating at magnitude 6, exact ties to the even code; the sign bit is the
  sign bit of x (so -0.0 and tiny negatives give code 0x8); a block whose scale
  decodes to 0 gets magnitude 0 everywhere.
* Packing.  Row-major, K contiguous; byte j of a row holds element 2j in bits
  3:0 and element 2j+1 in bits 7:4; scales are a separate [rows][cols/16] byte
  array.  The llama.cpp discussion ("What the patch does") traces a stall to a
  36-byte block of 32 code bytes and 4 scale bytes that is only 4-byte aligned;
  keeping codes and scales apart keeps both arrays 16-byte aligned.

Exactness.  Every rounding decision compares |x| (a float32, exact in float64)
against a threshold mid * dec(S) * gs or 6 * mid * gs, where mid is the
midpoint between two neighbouring codes.  The midpoint has at most 5
significant bits, dec(S) at most 4, 6 has 2 and gs 24, so each threshold has at
most 31 significant bits and its float64 product is exact.  The comparisons are
therefore decisions in exact real arithmetic.
"""
from dataclasses import dataclass

import numpy as np

from . import formats

BLOCK = 16
GS_DIVISOR = formats.E2M1_MAX * formats.E4M3_MAX          # 6 * 448 = 2688
AMAX_FLOOR = np.float32(1e-8)


@dataclass
class NVFP4:
    """An NVFP4 matrix [rows][cols]: packed E2M1 codes, E4M3 scales, fp32 global scale."""
    codes: np.ndarray      # uint8 [rows, cols // 2]
    scales: np.ndarray     # uint8 [rows, cols // 16]
    gs: np.float32
    rows: int
    cols: int

    def take_rows(self, idx):
        """The rows `idx` (gather), keeping the global scale."""
        idx = np.asarray(idx, dtype=np.int64)
        return NVFP4(self.codes[idx], self.scales[idx], self.gs, len(idx), self.cols)


def global_scale(x):
    """gs = RN32(max(max|x|, 1e-8) / (6*448)) over the whole float32 tensor `x`.

    DSV4 audit page, section P0: amax of |x|, clamped at 1e-8, divided by
    6.0 * 448.0.  An empty tensor has amax 0.
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    amax = max(amax, AMAX_FLOOR)
    return np.float32(np.float64(amax) / GS_DIVISOR)


def block_scale_codes(block_amax, gs):
    """E4M3 code of each block scale: RNE_E4M3(block_amax / (6*gs)), saturating at 448.

    thr[c] = 6 * mid_c * gs is the exact decision threshold between codes c
    and c+1 (increasing in c).  The code is the number of thresholds strictly
    below the value, plus one when the value sits exactly on thr[c] with c
    odd (between c and c+1 the even code wins).  Values above the last
    threshold get code 0x7E (448): saturation.
    """
    thr = (6.0 * formats.E4M3_MIDS) * np.float64(gs)          # exact, <= 31 significant bits
    a = np.asarray(block_amax, dtype=np.float64)
    below = np.searchsorted(thr, a, side="left")             # number of thresholds < a
    on = below < len(thr)
    tie = np.zeros(a.shape, dtype=bool)
    tie[on] = thr[below[on]] == a[on]
    code = below + (tie & (below % 2 == 1))
    return code.astype(np.uint8)


def element_codes(x_blocks, scale_codes, gs):
    """E2M1 codes of x_blocks [..., nb, 16] given each block's E4M3 scale code [..., nb].

    The decision threshold between magnitudes i and i+1 is mid_i * d * gs
    (exact).  On an exact tie the even index wins: at even i the value must
    exceed the threshold to round up, at odd i it rounds up when equal too.
    """
    d = formats.E4M3_TABLE[scale_codes.astype(np.int64)]    # exact decoded block scale
    dgs = (d * np.float64(gs))[..., None]                    # [..., nb, 1], exact
    mag = np.abs(x_blocks.astype(np.float64))
    idx = np.zeros(mag.shape, dtype=np.int8)
    for i, mid in enumerate(formats.E2M1_MIDS):
        thr = mid * dgs                                      # exact, <= 31 significant bits
        idx += (mag > thr) if i % 2 == 0 else (mag >= thr)
    idx = np.where((d == 0.0)[..., None], 0, idx)            # zero scale: magnitude 0
    sign = np.signbit(x_blocks).astype(np.int8)
    return (sign * 8 + idx).astype(np.uint8)


def pack_codes(codes):
    """[rows, cols] 4-bit codes -> [rows, cols/2] bytes, element 2j in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed):
    """[rows, cols/2] bytes -> [rows, cols] 4-bit codes."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


def quantize(x, gs=None):
    """NVFP4-quantise a float32 matrix x [rows, cols] (cols a multiple of 16).

    gs=None computes the per-call global scale from x (`global_scale`);
    otherwise the given float32 global scale is used as is.
    """
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] % BLOCK:
        raise ValueError("x must be [rows, cols] with cols % 16 == 0")
    if not np.all(np.isfinite(x)):
        raise ValueError("x must be finite")
    rows, cols = x.shape
    gs = global_scale(x) if gs is None else np.float32(gs)
    nb = cols // BLOCK
    row_chunk = max(1, (1 << 23) // max(cols, 1))         # bounds the temporaries
    codes = np.empty((rows, cols // 2), dtype=np.uint8)
    scales = np.empty((rows, nb), dtype=np.uint8)
    if rows == 0 or cols == 0:
        return NVFP4(codes, scales, gs, rows, cols)
    for r0 in range(0, rows, row_chunk):
        xb = x[r0:r0 + row_chunk].reshape(-1, nb, BLOCK)
        s = block_scale_codes(np.max(np.abs(xb), axis=-1), gs)
        c = element_codes(xb, s, gs)
        scales[r0:r0 + row_chunk] = s
        codes[r0:r0 + row_chunk] = pack_codes(c.reshape(-1, cols))
    return NVFP4(codes, scales, gs, rows, cols)


def expand(q):
    """code value * block scale value, float64 [rows, cols]; multiples of 2^-10, exact."""
    c = unpack_codes(q.codes)
    vals = formats.E2M1_TABLE[c.astype(np.int64)]
    s = formats.E4M3_TABLE[q.scales.astype(np.int64)]
    return vals * np.repeat(s, BLOCK, axis=1)


def dequantize(q):
    """x_hat = code * scale * gs, float64 [rows, cols] (exact: <= 30 significant bits)."""
    return expand(q) * np.float64(q.gs)
