"""CPU oracle for Speculative Pipeline Decoding (SPD): TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package. The GPU path (the HIP library and its Python binding)
never imports, calls or links anything here, and this package never imports
the GPU path: the only code both sides share is the seeded input generator in
``spd_inputs``.

What it computes, and from which passage:
  * the target model: a dense pre-norm decoder (RMSNorm, RoPE, GQA softmax
    attention, SwiGLU) and the hybrid variant with linear-attention layers
    (model.py);
  * SPD itself, step by step, in the pages' notation (spd.py): n pipeline
    stages of L/n layers, n tokens of one sequence in flight, the Pipeline
    Draft Module (PDM) reading the pipeline's input states with multi-depth
    anchor aggregation, streaming verification by greedy match or rejection
    sampling, and KV truncation, pipeline flush and reseed on rejection
    (pith.science review of arXiv 2605.30852, "What carries the argument" and
    "Core claim"; rejection sampling per Leviathan et al. 2023, cited there
    as the paper's section 3.5 assumption);
  * plain autoregressive decoding (spd.ar_decode), the plain definition of
    the result at temperature 0;
  * the output-state variant of the PDM schedule, the ablation the review
    sets against the early start (spd.py, speculate_from="output");
  * sampling rules, top-p sets and their near-tie envelope, and the
    counter-based RNG (sampling.py);
  * stage planning by per-layer cost (plan.py).

Arithmetic is float64 (numpy), with float32 available for the oracle's own
error check. The one storage rounding the precision contract fixes, the bf16
KV cache, is applied explicitly.

Parity pins live in tests/test_oracle_*.py. Every function here is pinned by
at least one of them; none is "parity unpinned" except the pages' printed
speedups, which need trained models and cannot be reproduced. The PDM's draft
path (anchor aggregation, projection, the speculation layers over the window,
its own final norm and the tied head) and the PDM prefill are pinned against a
route that steps no pipeline: one causal forward of the target for every
position's depths, one causal forward of the PDM over the step's feature rows
(tests/test_oracle_pdm.py, which also plants three mistakes in copies of the
PDM pass and requires each to fail).
"""
