"""Benchmark of the batched NVFP4 W4A4 MLP on one MI355X.

Default workload: a 16384-token prefill processed as 16 ubatches of 1024
tokens through 4 stacked MLP layers (hidden 5120, intermediate 17408), bf16
activations kept on the device between layers.  One step = the whole pass
(64 whole-MLP calls: quantise x, gate/up + SiLU*up + requantise, down -> bf16,
each layer's output amax handed to the next layer's quantiser).
Inputs are seeded synthetic draws (N(0,1) activations, N(0,0.02) weights),
resident in HBM before the timed region; weights are quantised on the device
beforehand (cold path).

Prints one JSON line.  Extra fields: the 1024-token MLP, the decode-shaped
T=1 / T=5 MLP (weight-streaming GB/s, cold and hot MALL), the 4-layer decode
stack eager and replayed from a HIP graph, the expert-grouped MLP, the
roofline of the dominant kernel and the CPU oracle timed on a bounded sample.
"""
import argparse
import dataclasses
import json
import os
import sys
import time
import types

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "NVFP4 MLP effective TFLOPS & tokens/s at T=1024/16384; % MFMA peak; T=1 HBM GB/s"
PEAK_F16_TFLOPS = 2500.0          # MI355X dense f16 MFMA
PEAK_HBM_GBS = 8000.0             # MI355X HBM3E
PEAK_FP4_TFLOPS = 10100.0         # MI355X dense fp4 MFMA (not the arithmetic used here)
K_HID, I_INT = 5120, 17408
COPY_BYTES = 256 << 20            # elementwise pass used to calibrate byte counters
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gate_up_gemm_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "mlp_prefill_amd", "csrc", f) for f in ("gemm.hip", "device_common.h")]


def kernel_source_hash():
    """SHA-256 of the dominant kernel's sources with // comments and blank lines removed."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        for line in open(f, encoding="utf-8"):
            code = line.split("//", 1)[0].strip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()


def traffic_bytes():
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None when the kernel sources changed since it was taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def mlp_flops(t, k=K_HID, i=I_INT):
    return 6.0 * t * k * i


# Weight preparation at set-up (not timed, like the weights' quantisation):
# the tile-contiguous copy the large-batch contractions stage from.
TILED_WEIGHTS = True


class Layer:
    """Quantised weights of one MLP layer on the device (with their
    tile-contiguous copies unless --row-major-weights)."""

    def __init__(self, m, seeds, k=K_HID, i=I_INT):
        from synthetic import bf16_normal
        self.w = []
        for seed, shp in zip(seeds, [(i, k), (i, k), (k, i)]):
            bits = bf16_normal(seed, shp, sigma=0.02)
            x = m.bf16_from_bits(bits)
            q = m.NVFP4.empty(*shp)
            m.nvfp4_quantize_act(x, q)
            del x
            if TILED_WEIGHTS:
                q.tile()
            self.w.append(q)


class MlpRunner:
    """Preallocated buffers for one MLP call shape (T tokens).

    chained=True: the down projection also writes max|y| (its output-amax
    epilogue), and a call marked `from_amax` quantises its input with the
    global scale formed from the amax the previous call wrote (one launch
    instead of the amax pass + quantise)."""

    def __init__(self, m, t, k=K_HID, i=I_INT):
        self.m, self.t, self.k, self.i = m, t, k, i
        self.xq = m.NVFP4.empty(t, k)
        self.hq = m.NVFP4.empty(t, i)
        self.ws_q = torch.empty(m.ws_bytes_quantize(t, k), dtype=torch.uint8, device="cuda")
        self.ws_gu = torch.empty(max(m.mlp_gu_act_ws_bytes(t, k, i), 256), dtype=torch.uint8, device="cuda")
        self.ws_dn = torch.empty(max(m.mlp_down_ws_bytes(t, i, k), 256), dtype=torch.uint8, device="cuda")
        self.amax = m.amax_buffer()

    def __call__(self, x, layer, y, chained=False, from_amax=False):
        m = self.m
        if from_amax:
            m.nvfp4_quantize_act(x, self.xq, gs_mode=m.GS_FROM_AMAX, ws=self.amax)
        else:
            m.nvfp4_quantize_act(x, self.xq, ws=self.ws_q)
        m.nvfp4_mlp_gu_act(self.xq, layer.w[0], layer.w[1], self.hq, ws=self.ws_gu)
        m.nvfp4_mlp_down(self.hq, layer.w[2], y, ws=self.ws_dn, amax=self.amax if chained else None)


class WholeRunner:
    """The whole-MLP call (nvfp4_mlp) for one shape: the quantisers write the f16
    operand copies (no expansion launches), and chained layers hand max|y| to the
    next layer through two alternating amax buffers."""

    def __init__(self, m, t, k=K_HID, i=I_INT):
        self.m = m
        self.xq = m.NVFP4.empty(t, k)
        self.hq = m.NVFP4.empty(t, i)
        self.ws = torch.empty(m.mlp_ws_bytes(t, k, i), dtype=torch.uint8, device="cuda")
        self.amax = [m.amax_buffer(), m.amax_buffer()]

    def __call__(self, x, layer, y, li, chained):
        """Layer li of a chain: x_amax from layer li-1, y_amax for layer li+1 when chained."""
        x_amax = self.amax[(li - 1) % 2] if li > 0 else None
        y_amax = self.amax[li % 2] if chained else None
        self.m.nvfp4_mlp(x, layer.w[0], layer.w[1], layer.w[2], self.xq, self.hq, y, x_amax=x_amax, y_amax=y_amax,
                         ws=self.ws)


def time_events(fn, reps, warm=2, scrub=None):
    """Per-repetition device durations (ms) with HIP events on the current stream."""
    for _ in range(warm):
        fn()
    out = []
    for _ in range(reps):
        if scrub is not None:
            scrub()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        e.synchronize()
        out.append(s.elapsed_time(e))
    return out


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(n_ubatch):
    """The oracle on the first `n_ubatch` 1024-token ubatches of the stacked workload through layer 0."""
    from threadpoolctl import threadpool_info

    from oracle import mlp as omlp
    from oracle import quant
    from synthetic import WORKLOADS, bf16_bits_to_f32, bf16_normal, layer_seeds
    p = WORKLOADS["mlp_long_prefill_16x1024_4layers"].params
    ub = p["ubatch"]
    x = bf16_bits_to_f32(bf16_normal(p["x_seed"], (p["T"], p["K"])))[:n_ubatch * ub]
    log("cpu baseline: quantising layer-0 weights with the oracle (cold, untimed)")
    w = [quant.quantize(bf16_bits_to_f32(bf16_normal(s, shp, sigma=p["w_sigma"])))
         for s, shp in zip(layer_seeds(p["layer_seed0"], 0), [(p["I"], p["K"]), (p["I"], p["K"]), (p["K"], p["I"])])]
    log(f"cpu baseline: oracle MLP on {n_ubatch} ubatches of {ub} tokens (timed)")
    t0 = time.perf_counter()
    for u in range(n_ubatch):
        omlp.mlp(x[u * ub:(u + 1) * ub], *w)
    dt = time.perf_counter() - t0
    t_sample = n_ubatch * ub
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    return {"value": mlp_flops(t_sample) / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(), "host_cores_available": len(os.sched_getaffinity(0)),
            "sample": f"the first {n_ubatch} ubatches ({t_sample} tokens) of the long-prefill input through "
                      f"layer 0 (quantise x, gate/up, SiLU*up, requantise, down; float64 numpy); {dt:.2f} s, "
                      f"{t_sample / dt:.1f} tokens/s; weight quantisation excluded",
            "seconds": dt}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the 1024-token, decode and expert-grouped lines")
    ap.add_argument("--cpu-ubatches", type=int, default=8, help="ubatches the CPU oracle runs (about 10-15 s)")
    ap.add_argument("--row-major-weights", action="store_true",
                    help="no tile-contiguous weight copies: the contractions stage the row-major weights")
    ap.add_argument("--decode-only", action="store_true",
                    help="print only the decode-shaped MLP line (T = 1 and T = 5) and exit")
    ap.add_argument("--moe-only", action="store_true",
                    help="print only the expert-grouped MLP line (4096 tokens, top-8 of 64 experts) and exit")
    args = ap.parse_args()
    global TILED_WEIGHTS
    TILED_WEIGHTS = not args.row_major_weights
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path is built and measured "
              f"on a single MI355X)", file=sys.stderr)
        return 2

    import mlp_prefill_amd as m
    from synthetic import WORKLOADS, bf16_normal, layer_seeds
    torch.cuda.set_device(0)
    if args.decode_only:
        print(json.dumps({"decode": decode_line(m)}), flush=True)
        return 0
    if args.moe_only:
        print(json.dumps({"moe": moe_line(m)}), flush=True)
        return 0
    p = WORKLOADS["mlp_long_prefill_16x1024_4layers"].params
    T, UB, L = p["T"], p["ubatch"], p["layers"]

    log("generating inputs and quantising weights on the device")
    x_all = m.bf16_from_bits(bf16_normal(p["x_seed"], (T, K_HID)))
    layers = [Layer(m, layer_seeds(p["layer_seed0"], li)) for li in range(L)]
    run = WholeRunner(m, UB)
    y_buf = [torch.empty((UB, K_HID), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    out = torch.empty((T, K_HID), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()

    def step():
        # one whole-MLP call per (ubatch, layer); each layer's down projection
        # hands max|y| to the next layer's quantiser
        for u in range(T // UB):
            cur = x_all[u * UB:(u + 1) * UB]
            for li, layer in enumerate(layers):
                dst = out[u * UB:(u + 1) * UB] if li == L - 1 else y_buf[li % 2]
                run(cur, layer, dst, li, chained=li < L - 1)
                cur = dst

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    n_calls = (T // UB) * L
    # The dominant kernel (gate/up contraction) is bracketed by HIP events on
    # its own stream inside the library, throughout the timed region.
    m.nvfp4_timing_begin(m.KC_GEMM_GLU, n_calls * args.steps)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(args.steps):
        step()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / args.steps
    n_gemm, dropped, gemm_total_ms = m.nvfp4_timing_end()
    assert n_gemm == n_calls * args.steps and dropped == 0, (n_gemm, dropped)
    flops = mlp_flops(T) * L
    tflops = flops / (ms * 1e-3) / 1e12
    tokens_s = T / (ms * 1e-3)
    log(f"{ms:.3f} ms/step, {tflops:.1f} TFLOP/s, {tokens_s:.0f} tokens/s")

    # ---- dominant kernel: the gate/up contraction with the SiLU*up epilogue ------------
    gemm_ms = gemm_total_ms / n_gemm
    gemm_flops = 4.0 * UB * K_HID * I_INT
    achieved = gemm_flops / (gemm_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_F16_TFLOPS, "traffic": traffic_bytes(),
                "kernel": "nvfp4::gemm_kernel<4, 2, 1, true, false, 1, 2, 2> (gate/up contraction, SiLU*up epilogue, "
                          "1024-token ubatch)",
                "flops_per_launch": gemm_flops, "avg_launch_ms": gemm_ms, "launches_timed": n_gemm,
                "arith": "f16 MFMA 32x32x16, fp32 accumulate (NVFP4 operands expanded exactly)",
                "peak_kind": "dense f16 MFMA: the instruction the exact NVFP4 contraction runs on gfx950 (frac is "
                             "against it); the fp4 peak is quoted in frac_of_fp4_dense_peak",
                "frac_of_fp4_dense_peak": achieved / PEAK_FP4_TFLOPS}
    log(f"dominant kernel {gemm_ms:.3f} ms -> {achieved:.1f} TFLOP/s ({100 * achieved / PEAK_F16_TFLOPS:.1f}% of f16 peak)")

    # Per-class breakdown of one further step (each class timed in its own window).
    breakdown = {}
    for name, kc in (("quantize", m.KC_QUANTIZE), ("expand", m.KC_EXPAND), ("gemm_glu", m.KC_GEMM_GLU),
                     ("gemm_store", m.KC_GEMM_STORE), ("reduce", m.KC_REDUCE)):
        m.nvfp4_timing_begin(kc, 8 * n_calls)
        step()
        n_k, _, tot = m.nvfp4_timing_end()
        breakdown[name] = {"launches_per_step": n_k, "ms_per_step": tot}
    roofline["breakdown_one_step"] = breakdown

    # A plain elementwise kernel of known traffic (reads and writes COPY_BYTES),
    # so that profiler byte counters taken on this same command can be
    # calibrated against it.
    src = torch.zeros(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst

    extra = {}
    if not args.no_extra:
        extra = extra_lines(m)
        log("extra: long prefill with the ubatches over two streams")
        extra["two_streams"] = two_stream_line(m, layers, x_all, out, args.steps)
        log("extra: long prefill with static global scales")
        extra["static_gs"] = static_line(m, layers, x_all, args.steps)
        extra["decode_stack"] = decode_stack_line(m, layers)
        extra["quantize"] = quantize_line(m)

    result = {
        "metric": METRIC, "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "mlp_long_prefill_16x1024_4layers", "tokens": T, "ubatch": UB, "layers": L,
                   "hidden": K_HID, "intermediate": I_INT, "storage": "nvfp4 (e2m1 codes, e4m3 block-16 scales, "
                   "fp32 global scale)", "accumulate": "fp32",
                   "weights": ("row-major, plus tile-contiguous copies written at set-up (untimed, like the weight "
                               "quantisation)") if TILED_WEIGHTS else "row-major"},
        "tokens_per_s": tokens_s, "flops_per_step": flops,
        "roofline": roofline,
    }
    result.update(extra)
    if not args.no_cpu_baseline:
        cb = cpu_baseline(args.cpu_ubatches)
        result["cpu_baseline"] = cb
        log(f"cpu baseline {cb['value'] * 1e3:.2f} GFLOP/s on {cb['cores']} threads")
    print(json.dumps(result), flush=True)
    return 0


def two_stream_line(m, layers, x_all, ref_out, steps, ub=1024, n_streams=2):
    """The long-prefill workload with its ubatches dealt in turn to two streams
    (default priority), each stream running its ubatches' 4-layer chains with
    its own workspace and buffers.  The 16 ubatches are independent through an
    MLP stack, so one chain's memory-bound launches (quantisers, split-K
    reduction) can run beside the other chain's contractions.  The headline
    value keeps the sequential order (one ubatch after another, as a model
    with attention between the MLPs must); this line reports the overlap, and
    its output is compared bit for bit with the sequential pass's."""
    t_all, k = x_all.shape
    n_l = len(layers)
    runs = [WholeRunner(m, ub) for _ in range(n_streams)]
    ybufs = [[torch.empty((ub, k), dtype=torch.bfloat16, device="cuda") for _ in range(2)] for _ in range(n_streams)]
    out = torch.empty_like(ref_out)
    streams = [torch.cuda.Stream() for _ in range(n_streams)]

    def step():
        main = torch.cuda.current_stream()
        for st in streams:
            st.wait_stream(main)
        for u in range(t_all // ub):
            j = u % n_streams
            run, y_buf = runs[j], ybufs[j]
            cur = x_all[u * ub:(u + 1) * ub]
            for li, layer in enumerate(layers):
                dst = out[u * ub:(u + 1) * ub] if li == n_l - 1 else y_buf[li % 2]
                x_amax = run.amax[(li - 1) % 2] if li > 0 else None
                y_amax = run.amax[li % 2] if li < n_l - 1 else None
                m.nvfp4_mlp(cur, layer.w[0], layer.w[1], layer.w[2], run.xq, run.hq, dst, x_amax=x_amax,
                            y_amax=y_amax, ws=run.ws, stream=streams[j])
                cur = dst
        for st in streams:
            main.wait_stream(st)

    ms = sorted(time_events(step, steps, warm=2))
    med = ms[len(ms) // 2]
    torch.cuda.synchronize()
    flops = mlp_flops(t_all, k, layers[0].w[0].rows) * n_l
    return {"workload": "mlp_long_prefill_16x1024_4layers, ubatches alternating over two streams",
            "streams": n_streams, "ms_per_step": med, "TFLOP/s": flops / (med * 1e-3) / 1e12,
            "tokens_per_s": t_all / (med * 1e-3), "output_equals_sequential": bool(torch.equal(out, ref_out))}


def static_line(m, layers, x_all, steps, ub=1024):
    """The long-prefill workload with static global scales: one dynamic
    warm-up ubatch records every layer's input and GLU-output scales on the
    device; the timed passes quantise the first layer's input with its given
    scale, quantise each GLU output in the gate/up epilogue and let each down
    projection but the last emit the next layer's NVFP4 input directly."""
    t_all, k = x_all.shape
    i = layers[0].w[0].rows
    n_l = len(layers)
    xq = [m.NVFP4.empty(ub, k) for _ in range(n_l)]
    hq = [m.NVFP4.empty(ub, i) for _ in range(n_l)]
    ws_q = torch.empty(m.ws_bytes_quantize(ub, k), dtype=torch.uint8, device="cuda")
    ws_gu = torch.empty(max(m.mlp_gu_act_ws_bytes(ub, k, i), 256), dtype=torch.uint8, device="cuda")
    ws_dn = torch.empty(max(m.mlp_down_ws_bytes(ub, i, k), 256), dtype=torch.uint8, device="cuda")
    ybf = torch.empty((ub, k), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((t_all, k), dtype=torch.bfloat16, device="cuda")
    # warm-up: the dynamic path on ubatch 0 writes each scale into the tensors kept for the static passes
    cur = x_all[:ub]
    for li, layer in enumerate(layers):
        m.nvfp4_quantize_act(cur, xq[li], ws=ws_q)
        m.nvfp4_mlp_gu_act(xq[li], layer.w[0], layer.w[1], hq[li], ws=ws_gu)
        m.nvfp4_mlp_down(hq[li], layer.w[2], ybf, ws=ws_dn)
        cur = ybf
    torch.cuda.synchronize()

    def step():
        for u in range(t_all // ub):
            m.nvfp4_quantize_act(x_all[u * ub:(u + 1) * ub], xq[0], gs_mode=m.GS_GIVEN, ws=ws_q)
            for li, layer in enumerate(layers):
                m.nvfp4_mlp_gu_act_static(xq[li], layer.w[0], layer.w[1], hq[li], ws=ws_gu)
                if li + 1 < n_l:
                    m.nvfp4_mlp_down_quant(hq[li], layer.w[2], xq[li + 1], ws=ws_dn)
                else:
                    m.nvfp4_mlp_down(hq[li], layer.w[2], out[u * ub:(u + 1) * ub], ws=ws_dn)

    step()
    torch.cuda.synchronize()
    b0 = m.launch_count()
    step()
    launches = (m.launch_count() - b0) // (t_all // ub)
    ms = sorted(time_events(step, steps, warm=1))
    med = ms[len(ms) // 2]
    flops = mlp_flops(t_all, k, i) * n_l
    return {"workload": "mlp_long_prefill_16x1024_4layers, static global scales (warm-up on ubatch 0)",
            "ms_per_step": med, "TFLOP/s": flops / (med * 1e-3) / 1e12, "tokens_per_s": t_all / (med * 1e-3),
            "launches_per_ubatch": launches,
            "path": "quantise(given gs) -> [gate/up with quantising epilogue -> down emitting the next "
                    "layer's NVFP4 input] x 3 -> gate/up -> down (bf16)"}


def decode_line(m):
    """Decode-shaped MLP (5120/17408) at T = 1 and T = 5: weight-streaming GB/s cold and hot; the
    whole-MLP call at 8, 12 and 16 tokens (cold)."""
    from synthetic import WORKLOADS, bf16_normal
    p2 = WORKLOADS["mlp_decode_5120x17408"].params
    log("extra: decode-shaped MLP T=1, T=5")
    lay = Layer(m, (p2["wg_seed"], p2["wu_seed"], p2["wd_seed"]))
    wbytes = sum(w.codes.numel() + w.scales.numel() + 4 for w in lay.w)
    scrub_buf = torch.ones(1 << 27, dtype=torch.int64, device="cuda")
    dec = {"workload": "mlp_decode_5120x17408", "weight_bytes": wbytes}
    launches = {}
    for tt in p2["Ts"]:
        x = m.bf16_from_bits(bf16_normal(p2["x_seed"], (tt, K_HID)))
        run = MlpRunner(m, tt)
        y = torch.empty((tt, K_HID), dtype=torch.float32, device="cuda")
        before = m.launch_count()
        run(x, lay, y)
        launches[tt] = m.launch_count() - before
        hot = float(np.median(time_events(lambda: run(x, lay, y), 50)))
        # cold: reading a 1 GiB buffer between reps evicts the 150 MB of weights
        # from the 256 MB MALL and the L2s (a read leaves no dirty lines whose
        # write-back would compete with the timed call)
        cold = float(np.median(time_events(lambda: run(x, lay, y), 20, scrub=lambda: scrub_buf.sum())))
        # static global scales (warm-up = this call's own scales): quantise with
        # the given scale (1 launch), gate/up with the quantising epilogue (2),
        # down (3)
        xq_s, hq_s = m.NVFP4.empty(tt, K_HID), m.NVFP4.empty(tt, lay.w[0].rows)
        xq_s.gscale.copy_(run.xq.gscale)
        hq_s.gscale.copy_(run.hq.gscale)
        ws_s = torch.empty(max(m.mlp_gu_act_static_ws_bytes(tt, K_HID, lay.w[0].rows), 256), dtype=torch.uint8,
                           device="cuda")

        def run_static():
            m.nvfp4_quantize_act(x, xq_s, gs_mode=m.GS_GIVEN, ws=run.ws_q)
            m.nvfp4_mlp_gu_act_static(xq_s, lay.w[0], lay.w[1], hq_s, ws=ws_s)
            m.nvfp4_mlp_down(hq_s, lay.w[2], y, ws=run.ws_dn)
        run_static()
        b0 = m.launch_count()
        run_static()
        static_launches = m.launch_count() - b0
        cold_s = float(np.median(time_events(run_static, 20, scrub=lambda: scrub_buf.sum())))
        # the whole-MLP call (one entry point, the decode path's four launches)
        ws_f = torch.empty(m.mlp_ws_bytes(tt, K_HID, lay.w[0].rows), dtype=torch.uint8, device="cuda")

        def run_fused():
            m.nvfp4_mlp(x, lay.w[0], lay.w[1], lay.w[2], run.xq, run.hq, y, ws=ws_f)
        run_fused()
        b0 = m.launch_count()
        run_fused()
        fused_launches = m.launch_count() - b0
        cold_f = float(np.median(time_events(run_fused, 20, scrub=lambda: scrub_buf.sum())))
        hot_f = float(np.median(time_events(run_fused, 50)))
        dec[f"T{tt}"] = {"ms_hot": hot, "ms_cold": cold, "hbm_gbs_cold": wbytes / (cold * 1e-3) / 1e9,
                         "hbm_gbs_hot": wbytes / (hot * 1e-3) / 1e9,
                         "frac_hbm_peak_cold": wbytes / (cold * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "whole_mlp_ms_cold": cold_f, "whole_mlp_ms_hot": hot_f,
                         "whole_mlp_hbm_gbs_cold": wbytes / (cold_f * 1e-3) / 1e9,
                         "whole_mlp_frac_hbm_peak_cold": wbytes / (cold_f * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "whole_mlp_launches": fused_launches,
                         "static_gs_ms_cold": cold_s, "static_gs_hbm_gbs_cold": wbytes / (cold_s * 1e-3) / 1e9,
                         "static_gs_launches": static_launches}
    dec["launches_per_call"] = launches
    dec["t5_over_t1_cold"] = dec["T5"]["ms_cold"] / dec["T1"]["ms_cold"]
    dec["whole_mlp_t5_over_t1_cold"] = dec["T5"]["whole_mlp_ms_cold"] / dec["T1"]["whole_mlp_ms_cold"]
    # medium batches on the same weights: the whole-MLP call, cold
    med = {}
    for tt in (8, 12, 16):
        x = m.bf16_from_bits(bf16_normal(p2["x_seed"] + tt, (tt, K_HID)))
        xq, hq = m.NVFP4.empty(tt, K_HID), m.NVFP4.empty(tt, lay.w[0].rows)
        y = torch.empty((tt, K_HID), dtype=torch.float32, device="cuda")
        ws_f = torch.empty(m.mlp_ws_bytes(tt, K_HID, lay.w[0].rows), dtype=torch.uint8, device="cuda")

        def run_fused():
            m.nvfp4_mlp(x, lay.w[0], lay.w[1], lay.w[2], xq, hq, y, ws=ws_f)
        run_fused()
        b0 = m.launch_count()
        run_fused()
        nl = m.launch_count() - b0
        cold_f = float(np.median(time_events(run_fused, 20, scrub=lambda: scrub_buf.sum())))
        med[f"T{tt}"] = {"whole_mlp_ms_cold": cold_f, "whole_mlp_hbm_gbs_cold": wbytes / (cold_f * 1e-3) / 1e9,
                         "whole_mlp_launches": nl}
    dec["medium_batches"] = med
    del lay, scrub_buf
    return dec


def gemm_small_line(m):
    """The single 16 x 256 x 512 NVFP4 GEMM workload: activation quantisation on
    the device plus the contraction (float32 out), launch-latency bound."""
    from synthetic import WORKLOADS, bf16_normal
    p = WORKLOADS["gemm_16x256x512"].params
    log("extra: single GEMM 16x256x512")
    x = m.bf16_from_bits(bf16_normal(p["x_seed"], (p["T"], p["K"])))
    w = m.NVFP4.empty(p["N"], p["K"])
    m.nvfp4_quantize_act(m.bf16_from_bits(bf16_normal(p["w_seed"], (p["N"], p["K"]), sigma=0.02)), w)
    xq = m.NVFP4.empty(p["T"], p["K"])
    c = torch.empty((p["T"], p["N"]), dtype=torch.float32, device="cuda")
    ws_q = torch.empty(m.ws_bytes_quantize(p["T"], p["K"]), dtype=torch.uint8, device="cuda")
    ws_g = torch.empty(max(m.gemm_ws_bytes(p["T"], p["N"], p["K"]), 256), dtype=torch.uint8, device="cuda")

    def call():
        m.nvfp4_quantize_act(x, xq, ws=ws_q)
        m.nvfp4_gemm(xq, w, c, ws=ws_g)
    b0 = m.launch_count()
    call()
    launches = m.launch_count() - b0
    ts = sorted(time_events(call, 50, warm=5))
    med = ts[len(ts) // 2]
    flops = 2.0 * p["T"] * p["K"] * p["N"]
    return {"workload": "gemm_16x256x512", "ms": med, "ms_min": ts[0], "ms_p90": ts[int(0.9 * (len(ts) - 1))],
            "gflops": flops / (med * 1e-3) / 1e9, "launches_per_call": launches,
            "note": "quantise x (device global scale) + contraction; a few microseconds of launch latency dominate"}


def extra_lines(m):
    """1024-token MLP and decode-shaped T=1/T=5 MLP (separate weights, as their workloads define)."""
    from synthetic import WORKLOADS, bf16_normal, outlier_channels
    out = {"gemm_16x256x512": gemm_small_line(m)}
    p3 = WORKLOADS["mlp_prefill_1024x5120x17408"].params
    log("extra: 1024-token MLP")
    lay = Layer(m, (p3["wg_seed"], p3["wu_seed"], p3["wd_seed"]))
    x = m.bf16_from_bits(bf16_normal(p3["x_seed"], (p3["T"], K_HID),
                                     outliers=outlier_channels(p3["outlier_seed"], K_HID)))
    whole = WholeRunner(m, p3["T"])
    y = torch.empty((p3["T"], K_HID), dtype=torch.float32, device="cuda")
    before = m.launch_count()
    whole(x, lay, y, 0, False)
    launches = m.launch_count() - before
    ms = float(np.median(time_events(lambda: whole(x, lay, y, 0, False), 20)))
    # ten calls between one pair of events: the per-call time without the host's
    # launch latency in front of each call (the one-call figure above includes it)
    ms_b2b = float(np.median(time_events(lambda: [whole(x, lay, y, 0, False) for _ in range(10)], 5))) / 10
    out["prefill_1024"] = {"workload": "mlp_prefill_1024x5120x17408", "ms": ms,
                           "tflops": mlp_flops(p3["T"]) / (ms * 1e-3) / 1e12,
                           "tokens_per_s": p3["T"] / (ms * 1e-3),
                           "frac_f16_peak": mlp_flops(p3["T"]) / (ms * 1e-3) / 1e12 / PEAK_F16_TFLOPS,
                           "launches": launches, "call": "nvfp4_mlp (whole MLP; global scales computed on the device)",
                           "back_to_back": {"ms_per_call": ms_b2b,
                                            "tflops": mlp_flops(p3["T"]) / (ms_b2b * 1e-3) / 1e12}}
    # the separate calls (quantise, gate/up + requantise, down), and the
    # whole-MLP call on the row-major weights alone (no tile-contiguous copies)
    run = MlpRunner(m, p3["T"])
    before = m.launch_count()
    run(x, lay, y)
    launches_sep = m.launch_count() - before
    ms_sep = float(np.median(time_events(lambda: run(x, lay, y), 20)))
    out["prefill_1024"]["separate_calls"] = {"ms": ms_sep, "tflops": mlp_flops(p3["T"]) / (ms_sep * 1e-3) / 1e12,
                                             "launches": launches_sep}
    if TILED_WEIGHTS:
        rm = [dataclasses.replace(w, tiled=None) for w in lay.w]
        lay_rm = types.SimpleNamespace(w=rm)
        ms_rm = float(np.median(time_events(lambda: whole(x, lay_rm, y, 0, False), 20)))
        out["prefill_1024"]["row_major_weights"] = {"ms": ms_rm, "tflops": mlp_flops(p3["T"]) / (ms_rm * 1e-3) / 1e12}
    del lay, run, whole, x, y
    out["decode"] = decode_line(m)
    # the tensor-parallel (tp = 2) shard on one GPU: intermediate 8704
    log("extra: tp=2 shard MLP (5120 -> 2 x 8704 -> 5120), T = 1024 and T = 1")
    scrub_buf = torch.ones(1 << 27, dtype=torch.int64, device="cuda")
    ih = I_INT // 2

    lay = Layer(m, (6001, 6002, 6003), i=ih)
    shard = {"workload": "mlp_prefill_1024x5120x17408 tp=2 shard (intermediate 8704)"}
    for tt in (1024, 1):
        x = m.bf16_from_bits(bf16_normal(6004, (tt, K_HID)))
        run = MlpRunner(m, tt, i=ih)
        y = torch.empty((tt, K_HID), dtype=torch.bfloat16, device="cuda")
        if tt == 1:
            ms = float(np.median(time_events(lambda: run(x, lay, y), 20, scrub=lambda: scrub_buf.sum())))
            wb = sum(w.codes.numel() + w.scales.numel() + 4 for w in lay.w)
            shard["T1"] = {"ms_cold": ms, "hbm_gbs_cold": wb / (ms * 1e-3) / 1e9}
        else:
            ms = float(np.median(time_events(lambda: run(x, lay, y), 20)))
            tf = mlp_flops(tt, i=ih) / (ms * 1e-3) / 1e12
            shard["T1024"] = {"ms": ms, "tflops": tf, "frac_f16_peak": tf / PEAK_F16_TFLOPS,
                              "tokens_per_s": tt / (ms * 1e-3)}
    out["tp2_shard"] = shard
    del lay, scrub_buf
    out["moe"] = moe_line(m)
    return out


def quantize_line(m):
    """Activation quantisation (A1+A2, two launches), the same with a given
    (static) global scale (one launch) and the fused RMSNorm variant (N2), bf16
    input: GB/s of the algorithmic traffic, 2 B read + 0.5625 B written per
    element, at the 1024-token shape and on a 65536 x 5120 probe."""
    from synthetic import bf16_normal
    log("extra: quantisation kernels (plain and RMSNorm-fused)")
    out = {"unit_bytes_per_element": 2.5625}
    g = torch.ones(K_HID, dtype=torch.float32, device="cuda")
    for rows in (1024, 65536):
        x = m.bf16_from_bits(bf16_normal(777, (1024, K_HID))).repeat(rows // 1024, 1)
        q = m.NVFP4.empty(rows, K_HID)
        ws = torch.empty(max(m.ws_bytes_quantize(rows, K_HID), m.rmsnorm_quantize_ws_bytes(rows, K_HID)),
                         dtype=torch.uint8, device="cuda")
        nbytes = rows * K_HID * 2.5625
        tq = float(np.median(time_events(lambda: m.nvfp4_quantize_act(x, q, ws=ws), 20)))
        tg = float(np.median(time_events(lambda: m.nvfp4_quantize_act(x, q, gs_mode=m.GS_GIVEN, ws=ws), 20)))
        tn = float(np.median(time_events(lambda: m.nvfp4_rmsnorm_quantize_act(x, g, 1e-6, q, ws=ws), 20)))
        out[f"rows{rows}"] = {"quantize_ms": tq, "quantize_gbs": nbytes / (tq * 1e-3) / 1e9,
                              "quantize_frac_hbm": nbytes / (tq * 1e-3) / 1e9 / PEAK_HBM_GBS,
                              "given_gs_quantize_ms": tg, "given_gs_quantize_gbs": nbytes / (tg * 1e-3) / 1e9,
                              "rmsnorm_quantize_ms": tn, "rmsnorm_quantize_gbs": nbytes / (tn * 1e-3) / 1e9}
        del x, q, ws
    return out


def decode_stack_line(m, layers):
    """One token (T = 1) and five (T = 5) through the 4 stacked full-size layers,
    eager and replayed from a HIP graph.  The 601.6 MB of weights exceed the
    256 MB MALL, so every pass streams them from HBM."""
    log("extra: 4-layer decode stack, eager and HIP graph")
    wbytes = sum(w.codes.numel() + w.scales.numel() + 4 for lay in layers for w in lay.w)
    out = {"workload": "mlp_long_prefill_16x1024_4layers weights, T = 1 and T = 5 per pass", "weight_bytes": wbytes}
    for t in (1, 5):
        from synthetic import bf16_normal
        x = m.bf16_from_bits(bf16_normal(99, (t, K_HID)))
        run = MlpRunner(m, t)
        ys = [torch.empty((t, K_HID), dtype=torch.bfloat16, device="cuda") for _ in range(2)]

        def stack():
            cur = x
            for li, lay in enumerate(layers):
                run(cur, lay, ys[li % 2])
                cur = ys[li % 2]
        eager = float(np.median(time_events(stack, 20)))
        b0 = m.launch_count()
        stack()
        launches = m.launch_count() - b0
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                stack()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = float(np.median(time_events(g.replay, 20)))
        del g
        # the same stack through the whole-MLP call (4 launches per layer)
        ws_f = torch.empty(m.mlp_ws_bytes(t, K_HID, layers[0].w[0].rows), dtype=torch.uint8, device="cuda")

        def stack_whole():
            cur = x
            for li, lay in enumerate(layers):
                m.nvfp4_mlp(cur, lay.w[0], lay.w[1], lay.w[2], run.xq, run.hq, ys[li % 2], ws=ws_f)
                cur = ys[li % 2]
        eager_w = float(np.median(time_events(stack_whole, 20)))
        b0 = m.launch_count()
        stack_whole()
        launches_w = m.launch_count() - b0
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                stack_whole()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph_w = float(np.median(time_events(g.replay, 20)))
        del g
        out[f"T{t}"] = {"ms_eager": eager, "ms_graph": graph, "ms_per_layer_graph": graph / len(layers),
                        "hbm_gbs_graph": wbytes / (graph * 1e-3) / 1e9,
                        "frac_hbm_peak_graph": wbytes / (graph * 1e-3) / 1e9 / PEAK_HBM_GBS,
                        "launches_per_pass": launches,
                        "whole_mlp_ms_eager": eager_w, "whole_mlp_ms_graph": graph_w,
                        "whole_mlp_hbm_gbs_graph": wbytes / (graph_w * 1e-3) / 1e9,
                        "whole_mlp_frac_hbm_peak_graph": wbytes / (graph_w * 1e-3) / 1e9 / PEAK_HBM_GBS,
                        "whole_mlp_launches_per_pass": launches_w}
    return out


def moe_line(m):
    """Expert-grouped MoE layer on the device: 4096 tokens routed top-8 over 64
    experts (hidden 4096, expert width 2048): route, the expert MLP in one call
    (quantise, grouped gate/up + SiLU*up + requantise, grouped down), combine;
    also timed with the separate quantise and grouped-GEMM calls."""
    from synthetic import WORKLOADS, bf16_normal, expert_seeds, router_logits
    p = WORKLOADS["moe_4096_top8_of_64"].params
    t, e, top, k, i = p["T"], p["E"], p["topk"], p["K"], p["I"]
    log("extra: expert-grouped MoE layer (64 experts, top-8), device routing and combine")
    mats = [[], [], []]
    for x in range(e):
        for j, (sd, shp) in enumerate(zip(expert_seeds(p["expert_seed0"], x), [(i, k), (i, k), (k, i)])):
            w = m.bf16_from_bits(bf16_normal(sd, shp, sigma=0.02))
            q = m.NVFP4.empty(*shp)
            m.nvfp4_quantize_act(w, q)
            mats[j].append(q)
    wg, wu, wd = (m.NVFP4.stack(v) for v in mats)
    del mats
    if TILED_WEIGHTS:
        for w in (wg, wu, wd):
            w.tile()
    x = m.bf16_from_bits(bf16_normal(p["x_seed"], (t, k)))
    logits = torch.from_numpy(router_logits(p["router_seed"], t, e)).cuda()
    slots = t * top
    offs = torch.empty(e + 1, dtype=torch.int32, device="cuda")
    rows = torch.empty(slots, dtype=torch.int32, device="cuda")
    slot_of = torch.empty((t, top), dtype=torch.int32, device="cuda")
    cw = torch.empty((t, top), dtype=torch.float32, device="cuda")
    ws_r = torch.empty(max(m.moe_route_ws_bytes(t, e, top), 256), dtype=torch.uint8, device="cuda")
    xq = m.NVFP4.empty(t, k)
    hq = m.NVFP4.empty(slots, i)
    ys = torch.empty((slots, k), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((t, k), dtype=torch.bfloat16, device="cuda")
    ws_q = torch.empty(m.ws_bytes_quantize(t, k), dtype=torch.uint8, device="cuda")
    ws_g = torch.empty(max(m.grouped_ws_bytes(slots, i, k, e, m.EPI_SILU_MUL_REQUANT), 256), dtype=torch.uint8,
                       device="cuda")
    ws_d = torch.empty(max(m.grouped_ws_bytes(slots, k, i, e, m.EPI_STORE), 256), dtype=torch.uint8, device="cuda")
    ws_m = torch.empty(m.moe_mlp_ws_bytes(t, k, i, e, slots), dtype=torch.uint8, device="cuda")

    def layer():
        m.nvfp4_moe_route(logits, top, offs, rows, slot_of, cw, ws=ws_r)
        m.nvfp4_moe_mlp(x, rows, offs, wg, wu, wd, xq, hq, ys, ws=ws_m)
        m.nvfp4_moe_combine(ys, slot_of, cw, y)

    def layer_separate():
        m.nvfp4_moe_route(logits, top, offs, rows, slot_of, cw, ws=ws_r)
        m.nvfp4_quantize_act(x, xq, ws=ws_q)
        m.nvfp4_grouped_gemm(xq, rows, offs, wg, wu, out_q=hq, epilogue=m.EPI_SILU_MUL_REQUANT, m=slots, ws=ws_g)
        m.nvfp4_grouped_gemm(hq, None, offs, wd, out=ys, epilogue=m.EPI_STORE, ws=ws_d)
        m.nvfp4_moe_combine(ys, slot_of, cw, y)

    before = m.launch_count()
    layer()
    launches = m.launch_count() - before
    # the variants are timed one after another: warm the GPU up first so that
    # the first one timed does not run in a lower clock state than the others
    for _ in range(20):
        layer()
    ms = float(np.median(time_events(layer, 10)))
    before = m.launch_count()
    layer_separate()
    parts = {"separate_calls_launches": m.launch_count() - before,
             "separate_calls_ms": float(np.median(time_events(layer_separate, 10)))}
    for name, kc in (("route", m.KC_ROUTE), ("combine", m.KC_COMBINE)):
        m.nvfp4_timing_begin(kc, 64)
        for _ in range(5):
            layer()
        n, _, tot = m.nvfp4_timing_end()
        parts[f"{name}_ms"] = tot / 5
    # static global scales (warm-up = the dynamic layer just run): quantise with
    # the given scale, gate/up with the quantising epilogue (no float32 H, no
    # requantisation)
    xq_s, hq_s = m.NVFP4.empty(t, k), m.NVFP4.empty(slots, i)
    xq_s.gscale.copy_(xq.gscale)
    hq_s.gscale.copy_(hq.gscale)
    ws_gs = torch.empty(max(m.grouped_ws_bytes(slots, i, k, e, m.EPI_SILU_MUL_QUANT_GIVEN), 256), dtype=torch.uint8,
                        device="cuda")

    ws_ms = torch.empty(m.moe_mlp_ws_bytes(t, k, i, e, slots, static=True), dtype=torch.uint8, device="cuda")

    def layer_static():
        # one call: quantise x with its given scale (and its f16 copy), gate/up
        # quantising H~ in its epilogue (and H~'s f16 copy), down, reduction
        m.nvfp4_moe_route(logits, top, offs, rows, slot_of, cw, ws=ws_r)
        m.nvfp4_moe_mlp_static(x, rows, offs, wg, wu, wd, xq_s, hq_s, ys, ws=ws_ms)
        m.nvfp4_moe_combine(ys, slot_of, cw, y)

    def layer_static_separate():
        m.nvfp4_moe_route(logits, top, offs, rows, slot_of, cw, ws=ws_r)
        m.nvfp4_quantize_act(x, xq_s, gs_mode=m.GS_GIVEN, ws=ws_q)
        m.nvfp4_grouped_gemm(xq_s, rows, offs, wg, wu, out_q=hq_s, epilogue=m.EPI_SILU_MUL_QUANT_GIVEN, m=slots,
                             ws=ws_gs)
        m.nvfp4_grouped_gemm(hq_s, None, offs, wd, out=ys, epilogue=m.EPI_STORE, ws=ws_d)
        m.nvfp4_moe_combine(ys, slot_of, cw, y)

    before = m.launch_count()
    layer_static()
    launches_s = m.launch_count() - before
    ms_s = float(np.median(time_events(layer_static, 10)))
    parts["static_gs_ms"] = ms_s
    parts["static_gs_launches_per_call"] = launches_s
    before = m.launch_count()
    layer_static_separate()
    parts["static_gs_separate_calls_launches"] = m.launch_count() - before
    parts["static_gs_separate_calls_ms"] = float(np.median(time_events(layer_static_separate, 10)))
    flops = mlp_flops(slots, k, i)
    parts["static_gs_tflops"] = flops / (ms_s * 1e-3) / 1e12
    tf = flops / (ms * 1e-3) / 1e12
    comb_bytes = slots * k * 2 + t * k * 2 + t * top * 8
    return {"workload": "moe_4096_top8_of_64", "ms": ms, "tflops": tf, "frac_f16_peak": tf / PEAK_F16_TFLOPS,
            "tokens_per_s": t / (ms * 1e-3), "slots": slots, "launches_per_call": launches, **parts,
            "combine_gbs": comb_bytes / (parts["combine_ms"] * 1e-3) / 1e9,
            "note": "ms covers routing, the expert MLP call (quantisation, both grouped GEMMs) and the combine; "
                    "TFLOP/s counts the 6*slots*K*I of the expert MLPs"}


if __name__ == "__main__":
    sys.exit(main())
