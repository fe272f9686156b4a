"""CPU oracle for the FP8 small-GEMM + LayerNorm block.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only the test suite, the smoke check and
the CPU-baseline leg of the benchmark use it.  It shares no code with the HIP
library (no common helpers, tables or constants) and imports nothing from it.

Everything here is plain NumPy in float64 (float32 only where the method
itself fixes an fp32 step, e.g. the scale division and the x*r product that
decides an FP8 code).  It is slow and written to be checked by eye against:

  [LoKA]  "LoKA: Low-precision Kernel Applications for Recommendation Models
          At Scale" (Meta, arXiv 2605.10886)
  [GEM]   "GEM Training: How Meta Doubled the Efficiency of Its LLM-Scale Ads
          Foundation Model" (Meta engineering blog)
  [OCP]   the OCP 8-bit floating point (e4m3fn / e5m2) and MX v1.0 formats,
          which [LoKA] names through its MX reference [63] and [GEM] through
          "MXFP8"; the pages print no encoding table, so the format
          definitions themselves are the source.

Modules:
  codec     FP8 / E8M0 / bf16 encode and decode (exact, integer-checked)
  quant     amax, scales and saturating RNE casts for every scaling mode
  forward   quantize -> fp64 GEMM -> dequant + bias -> LayerNorm -> bf16
  backward  LayerNorm backward, e5m2 dZ, dgrad and wgrad in fp64
  grouped   the grouped forward as a list of independent forwards
  mere      mean element-wise relative error ([LoKA] section II-C)
  report    per-layer MERE of every workload against the bf16 reference
  dispatch  the Dispatch runtime's recipe selection rule ([LoKA] section III-C)
  probe     the Probe's input/weight statistics and sampler ([LoKA] section III-A1)

Parity unpinned: nothing.  Every function is pinned by tests/test_oracle_*.py
against hand-worked encodings, closed forms, invariants or brute force.
"""

from . import codec, quant, forward, backward, grouped, mere, dispatch, probe, report  # noqa: F401
