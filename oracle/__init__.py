"""CPU oracle for the causal block-scaled MXFP8 attention training call.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this package:
only the test suite, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` use it.  It shares no code with the HIP library, and it
imports nothing from the product package.

The oracle is written for a reader holding the pages that describe the method.
Page titles used in citations throughout this package:

* [Summary]  "FLAMIA: FLAsh MIcroscaling Attention for Fast and Causally Safe
  Training on Blackwell" -- the Chinese summary page whose bullets are tagged
  with the paper's sections (§3.1 Token-Block Scaling, §3.2 Causally Safe
  Scales, §3.3 Forward-Backward Numerical Consistency, §3.6.2 Load-Balanced
  Scheduling, §4.3 Ablation Study, §4.5 Causality and Training Stability).
* [Reading]  "因果安全的低精度注意力——FLAMIA Blackwell 训练内核精读" -- the
  close reading; its part 四 has sub-sections 4.1 (token-block scaling),
  4.2 (causally safe scaling), 4.3 (forward/backward consistency) and
  4.4 (kernel engineering).
* [News]     "FLAMIA Brings Causally Safe Low-Precision Attention to
  Blackwell" -- section "Key design choices".

Floating point is fp64 unless the method fixes a precision (fp32 scores and
probabilities, E4M3 / E2M1 / E8M0 codes, bf16 outputs).
"""

from . import formats, hadamard, quant, attention, worklist, nvfp4  # noqa: F401
