"""CPU oracle for inference-native zeroth-order scoring (test infrastructure).

Only tests/, the smoke check and the bench's CPU-baseline leg may import,
call, link or execute anything in this package.  The product path never
does, and the two share no code: only the seeded input generators in
`synth/` serve both.

What it computes, in fp64, is the plain definition of the method on the
pages ("Zeroth-Order Fine-Tuning Was an Inference Workload All Along",
section "Why ZO Fine-Tuning Is Really Scoring", the equations for L+, L-, c
and the update; section "The System Reorganization", the lazy U-accumulation
equations; and the arXiv abstract of "Inference-Native Zeroth-Order
Optimization", which states candidate-state queries, ProbePlan, factorized
side states and LoRA banks): forward passes of a decoder at the candidate
parameter states theta +/- eps*z, summed label log-probs, the two-point
coefficient and the lazy low-rank update.

Modules:
  rng     - Philox4x32-10 and the exact-operation Gaussian stream (C, via ctypes)
  params  - the weight-initialisation spec (logical tensors, tags, rounding)
  model   - the decoder forward (OPT-style and Qwen3-style), plain numpy
  zo      - ProbePlan, packing, score, estimate, update, bank

Every function is pinned by a `-m "not gpu"` test in tests/; the absolute
log-prob values have no worked example on the pages, so they are pinned by
an independent library implementation of the same architectures
(transformers, fp64) and by closed forms, not by printed numbers.
"""
