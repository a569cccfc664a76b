"""CPU oracle for the per-tensor-scaled FP8 GEMM path — TEST INFRASTRUCTURE ONLY.

This package is the slow, plain, obviously-correct definition that the HIP
library is checked against.  It is never part of the product path: only the
test-suite, the smoke check and the benchmark's CPU-baseline leg may import
it.  It shares no code with the HIP library and imports nothing from it.

Modules
-------
codec    OCP FP8 E4M3 / E5M2 decode and encode (round to nearest even,
         saturating), three independent encoders.
scaling  amax, the per-tensor scale rule, the delayed-scaling amax-history
         ring, the scaled cast, and per-block (current) scaling.
gemm     dequantised GEMM in fp64, exact integer dot products, the error
         bound, and the fine-grained grouped GEMM.
linear   one FP8 linear-layer step (forward, data and weight gradients)
         under the HYBRID recipe with delayed scaling.

Sources (the pages this follows)
--------------------------------
* "4.2 Hopper I — Transformer Engine·FP8" (aegloslab.com): §4.2.3 the two
  formats and their roles, §4.2.4 amax-based scale, scaled cast, FP32
  accumulation and the ×(1/scale) restore, delayed scaling from an amax
  history, §4.2.5 worked example A, §4.2.6 the recipe (HYBRID, history 16,
  "max"), §4.2.8 the OCP FP8 standard, §4.2.10 exercise 2.
* "FP8 and low-precision formats" (aiunderstanding.org): "Deep dive" — bit
  splits, per-tensor or per-block scale factors; "Technical insight" —
  scale, FP8 multiply-accumulate, divide back, partial sums in FP32.
* "#fp8" tag page (discuss.pytorch.kr), DeepGEMM entry: MoE grouped GEMM and
  two-level accumulation (promotion) of FP8 partial sums.

Parity status per function is listed in each module's header.
"""

from . import codec, scaling, gemm, linear  # noqa: F401
