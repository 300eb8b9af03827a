"""Plain fp64 CPU oracle of the quantized MoE layer -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package's smoke check and the benchmark's CPU-baseline
leg may import this package.  The product path never calls it and it calls
nothing of the product path: the two share no code, only the seeded input
buffers from ``synth``.

What it computes, per token (pages cited by title and section):
  * router logits over 512 experts and a softmax over them, the 10 largest
    selected with gates renormalised over the selected ten, plus one always-on
    shared expert (page "Strata Runs 125B Qwen3.8-Flash-Next on a 12GB Gaming
    GPU", section "What it is"; page "Strata: a 125B AI model on your gaming
    PC", model spec table, row "Experts");
  * each selected expert's SwiGLU FFN at hidden size 2,560 (same spec table,
    row "Hidden dimension") from 2-bit block-quantized weights (the Q2_0 build
    named in section "The numbers, measured by the author" of the first page);
  * the gate-weighted combine plus the shared expert;
  * a stack of 48 such layers joined by a residual add (spec table, row "Layers");
  * an expert-cache mode in which only the cached experts are computed and the
    misses are listed (first page, section "How a 125B model fits in 12 GB").

Everything is float64 with library primitives (numpy matmul, sort) as steps; no
blocking, fusion or reordering beyond what the definitions state.

Readings where the pages are silent (softmax router, renormalised gates, lowest
index wins ties, SwiGLU without biases, intermediate size 640, the bit layouts,
fp32 layer output) are listed with the workloads they come from in the design
notes at the repository root.  Every function is pinned by the CPU tests in
``tests/test_oracle_pins.py`` against closed forms, brute force, invariants or
textbook routines; no function here is parity-unpinned.
"""
from . import formats, layer  # noqa: F401
