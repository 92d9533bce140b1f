"""Seeded synthetic inputs shared by the oracle-side tests and the device path.

This module only draws random numbers and lays them out; it holds none of the
NVFP4 method's arithmetic.  Both sides (the HIP library through its binding,
and the CPU oracle) receive the same host arrays from here.

The pages' workloads -- a 27B NVFP4 checkpoint prefilled by llama-bench with a
16384-token prompt in 1024-token ubatches (llama.cpp discussion, setup line and
results table), T=1 and T=5 MLP launches in a tp=2 trace (vllm.cpp issue,
"Problem") -- need trained weights that are not available; these generators
stand in for them with the same shapes: hidden 5120, intermediate 17408,
activations ~ N(0,1) in bf16 (optionally with a few outlier channels),
weights ~ N(0, 0.02) in bf16.

bf16 values are carried on the host as uint16 bit patterns (numpy has no bf16).
"""
from dataclasses import dataclass

import numpy as np


def _round_f32_to_bf16_bits(x):
    """float32 -> bf16 bit patterns (uint16), nearest with ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b):
    """bf16 bit patterns (uint16) -> float32 values (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def outlier_channels(seed, k, frac=0.001):
    """round(frac * k) distinct channel indices, drawn with their own seed."""
    rng = np.random.default_rng(seed)
    n = int(round(frac * k))
    return np.sort(rng.choice(k, n, replace=False)) if n else np.zeros(0, dtype=np.int64)


def bf16_normal(seed, shape, sigma=1.0, outliers=None, outlier_gain=50.0):
    """N(0, sigma^2) float32 draws (PCG64 `seed`), optional channel outliers, rounded to bf16 bits.

    `outliers` is a list of column indices whose values are multiplied by
    `outlier_gain` (in float32) before the rounding to bf16.
    """
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    if outliers is not None and len(outliers):
        x[..., np.asarray(outliers)] *= np.float32(outlier_gain)
    return _round_f32_to_bf16_bits(x)


def router_logits(seed, t, e):
    """Router logits ~ N(0, 1), float32 [t, e] (PCG64 `seed`)."""
    return np.random.default_rng(seed).standard_normal((t, e), dtype=np.float32)


@dataclass
class Workload:
    name: str
    desc: str
    params: dict


# The five workloads: sizes, distributions and seeds.
WORKLOADS = {
    "gemm_16x256x512": Workload(
        "gemm_16x256x512", "single NVFP4 GEMM, T=16 K=256 N=512",
        dict(T=16, K=256, N=512, x_seed=1001, w_seed=1002, w_sigma=0.02)),
    "mlp_decode_5120x17408": Workload(
        "mlp_decode_5120x17408", "decode-shaped MLP at T=1 and T=5",
        dict(Ts=(1, 5), K=5120, I=17408, x_seed=2001, wg_seed=2002, wu_seed=2003, wd_seed=2004,
             w_sigma=0.02)),
    "mlp_prefill_1024x5120x17408": Workload(
        "mlp_prefill_1024x5120x17408", "prefill ubatch MLP, T=1024, 0.1% outlier channels x50",
        dict(T=1024, K=5120, I=17408, x_seed=3001, outlier_seed=3005, wg_seed=3002, wu_seed=3003,
             wd_seed=3004, w_sigma=0.02)),
    "mlp_long_prefill_16x1024_4layers": Workload(
        "mlp_long_prefill_16x1024_4layers", "T=16384 as 16 ubatches of 1024 through 4 stacked MLPs",
        dict(T=16384, ubatch=1024, layers=4, K=5120, I=17408, x_seed=4001, layer_seed0=4002,
             w_sigma=0.02)),
    "moe_4096_top8_of_64": Workload(
        "moe_4096_top8_of_64", "expert-grouped MLP, T=4096 top-8 of 64, hidden 4096, expert width 2048",
        dict(T=4096, E=64, topk=8, K=4096, I=2048, x_seed=5001, router_seed=5005, expert_seed0=5100,
             w_sigma=0.02)),
}


def layer_seeds(seed0, layer):
    """(gate, up, down) weight seeds of stacked layer `layer`."""
    return seed0 + 3 * layer, seed0 + 3 * layer + 1, seed0 + 3 * layer + 2


def expert_seeds(seed0, expert):
    """(gate, up, down) weight seeds of expert `expert`."""
    return seed0 + 3 * expert, seed0 + 3 * expert + 1, seed0 + 3 * expert + 2
