"""NVFP4 x NVFP4 contraction with exact accumulation.

TEST INFRASTRUCTURE ONLY (see the package docstring).

y[t, n] = gs_a * gs_b * sum_k (q_a[t,k] * S_a[t, k/16]) * (q_b[n,k] * S_b[n, k/16])

i.e. C = A . B^T with both operands stored K-contiguous, the shape of a linear
layer's activation [T, K] times its weight [N, K] (the MUL_MAT of the llama.cpp
discussion, "Verified").  Each factor q*S is a multiple of 2^-10 with at most
6 significant bits, so each product is a multiple of 2^-20; any partial sum of
such products is exact in float64 while sum_k |a_k||b_k| < 2^33.  The float64
matrix product below is therefore exact whatever order or blocking the BLAS
uses; a Cauchy-Schwarz bound checks the condition and an int64 product takes
over when it cannot be shown.  The result is then multiplied by the exact
float64 product gs_a * gs_b (one float64 rounding).
"""
import numpy as np

from . import quant

_EXACT_LIMIT = 2.0 ** 33


def _exact_dot(a, b):
    """a [M,K] . b [N,K]^T for float64 matrices of multiples of 2^-10, exactly."""
    if a.shape[0] == 0 or b.shape[0] == 0:
        return np.zeros((a.shape[0], b.shape[0]), dtype=np.float64)
    # sum_k |a_k||b_k| <= ||a|| ||b||; the norms carry rounding of ~1e-16 relative,
    # far below the factor-of-two margin kept here.
    bound = np.sqrt(np.max(np.einsum("ij,ij->i", a, a))) * np.sqrt(np.max(np.einsum("ij,ij->i", b, b)))
    if bound < _EXACT_LIMIT / 2:
        return a @ b.T
    if np.max(np.abs(a) @ np.abs(b).T) < _EXACT_LIMIT / 2:
        return a @ b.T
    ai = np.rint(a * 1024.0).astype(np.int64)
    bi = np.rint(b * 1024.0).astype(np.int64)
    return (ai @ bi.T).astype(np.float64) * 2.0 ** -20


def gemm_acc(a, b):
    """sum_k (q*S)_a (q*S)_b, exact (float64), without the global scales."""
    if a.cols != b.cols:
        raise ValueError("K mismatch")
    return _exact_dot(quant.expand(a), quant.expand(b))


def gemm(a, b):
    """C[M, N] = dequant(A) . dequant(B)^T in float64 (exact up to one final rounding)."""
    return gemm_acc(a, b) * (np.float64(a.gs) * np.float64(b.gs))
