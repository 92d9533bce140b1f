"""Plain CPU oracle for the batched T-token NVFP4 W4A4 MLP.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding) imports, calls or links this package; only the tests, the
``smoke()`` self-check and the CPU-baseline leg of the benchmark use it.  It
shares no code with the HIP path.

It computes, slowly and in float64 numpy, exactly what the pages describe:

* ``formats``   -- E2M1 element codes and E4M3 block-scale codes, decoded from
                   their bit definitions (OCP MX v1.0 for E2M1, OCP OFP8 for
                   E4M3 "FN"; the largest values 6 and 448 are the ones the
                   global-scale formula of the DSV4 audit page divides by).
* ``quant``     -- NVFP4 quantisation: device-style global scale
                   amax/(6*448) with the amax clamp at 1e-8 (audit page,
                   section P0), one E4M3 scale per 16-element K-block, E2M1
                   codes packed two per byte.
* ``gemm``      -- dequantised contraction with exact float64 accumulation.
* ``mlp``       -- gate/up sharing one quantised activation, SiLU(gate)*up,
                   requantisation of the GLU output straight into the
                   down-projection's NVFP4 input (llama.cpp discussion,
                   "What the patch does"), the down projection, stacked layers
                   with device-resident bf16 activations (vllm.cpp issue,
                   "Fix directions" 1-2) and the expert-grouped variant.
* ``moe``       -- top-k routing into expert-grouped slots and the weighted
                   combine of the per-slot outputs (readings in its docstring).
* ``norm``      -- RMSNorm fused into the activation quantisation.

Every rounding decision is taken in exact arithmetic (float64 products that are
provably exact); see each function's docstring for the reading it follows.
"""
from . import formats, quant, gemm, mlp, moe, norm  # noqa: F401
