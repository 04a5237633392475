"""CPU oracle for the routed top-k experts forward -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct fp64 reference of what the GPU library computes.
Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
it; the product (the HIP library and its Python binding) never does, and the two
share no code.

Sources (Hugging Face Transformers docs, "Experts backends" page, read in its
es/fr/id/ru translations):
  * introduction: per token a router picks k experts; the hidden state is
    projected through the chosen experts and aggregated with the routing weights;
  * backend table, "eager" row: the reference implementation loops over the
    selected experts and applies the projections to their tokens (fast mode);
  * backend table, "grouped_mm" row: tokens are sorted by selected expert before
    one grouped GEMM (the routing bookkeeping);
  * backend table, "deepgemm_megamoe" row, and the "SonicMoE" section: the expert
    is a gated MLP -- up projection, SwiGLU, down projection; silu maps to SwiGLU;
  * "FP8 and FP4 quantized experts" section and its note: block scales in float32
    or UE8M0 consumed directly, dynamic per-row activation scales, dequantisation
    is code times scale.

Pins (tests/test_oracle_*.py): library routines (argsort/bincount/torch casts),
dense brute force over all experts, the k=1 dense-MLP special case, a hand-reduced
closed-form instance, the OCP e4m3 anchor codes, invariants under relabelling,
and literal-vs-fast cross-checks.  Parity unpinned: none of the functions here.
"""

from . import numerics, moe  # noqa: F401
