"""CPU oracle for the routed-expert MoE feed-forward layer.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain, obviously-correct
reference that the GPU library is checked against.  Only the test suite, the
smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py``
may import it.  The product path (``quantized_routed_expert_amd``) never imports,
calls or falls back to anything in here, and nothing in here imports the product.

Arithmetic is numpy float64 throughout.  Every function cites the passage of the
source pages (or the workload definition) that it follows:

* "Qwen3.8-Flash-Next UD-IQ2_XS (L4 fix) for Basalt", section "What was
  changed": the routed experts go through a device-planned MoE tail and grouped
  kernels; the down-projection formats covered include IQ4_NL, NVFP4 and Q8_0;
  IQ4_NL costs 4.5 bits per weight.
* "The fastest inference engine for Qwen3.8-Flash-Next on Blackwell" (model
  card), section "Sources": tensors are GGUF tensors copied unchanged, so GGUF
  block conventions hold (blocks run along a row's reduction dimension).
* "Basalt at 665 tok/s? Qwen3.8 Flash-Next Setup and GPU Requirements",
  section "RAM and VRAM Hold Different Parts of the Expert Weights": each token
  uses only its selected experts.
* The workload definition of the routed-expert layer (router GEMV, softmax over
  the top-k with renormalised weights and lower-index tie-break, per-expert
  plan, SwiGLU experts, an always-on shared expert, deterministic combine, and
  the Q8_0 / IQ4_NL / NVFP4-style block formats with the IQ4_NL codebook).

Parity status of each function is stated in its docstring; every function here
is pinned by a CPU test (tests/test_oracle_*.py) against closed forms, library
routines, brute force or invariants.
"""

from . import formats, moe  # noqa: F401
