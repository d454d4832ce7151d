"""CPU oracle for the blockwise-FP8 MoE FFN forward: TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct numpy implementation of what the layer
computes.  Floating point is fp64 except where the method fixes a storage
precision (fp32 activation/weight scales, fp32 quotients before encoding,
fp32 routing arithmetic, the bf16 output).  It shares no code with the HIP
library and imports nothing from it; only ``synth`` (seeded draws, no
arithmetic of the method) is common to both.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path never calls it.

Sources, cited by page title and section:
  [R1 card]      llm-architectures-explained, "DeepSeek-R1", sections "Facts and
                 where they come from", "Modelled costs", "Every architecture field".
  [aguasto]      aguasto, "DeepSeek-R1" record, section "Quantization".
  [arch blog]    onlylabs, "DeepSeek v3 and R1 Model Architecture: Why it's
                 powerful and economical", sections "Architecture Overview",
                 "More Aggressive Mixture-of-Expert", "Structural change",
                 "Local Balanced Routing to Experts", and the FP8 table-of-contents
                 headings "Fine granularity quantization", "More Mantissa bits of
                 fp8", "Better Accumulation Precision", "Online Quantization",
                 "More customized data format and scaling factor".

Where the pages are silent the oracle takes one stated reading (sigmoid
scoring, group-limited top-k with a top-2-sum group score, e4m3 = OCP E4M3FN,
1x128 / 128x128 scale tiles, fp32 scales); each reading is named in the
docstring of the function that applies it.

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
something other than itself (closed forms, brute force, library routines,
invariants).  One part has no such pin and is marked "parity unpinned": the
fidelity of the FP8 layer to unquantised math (the pages' claim is cut off).
"""
from . import e4m3, quant, route, permute, gemm, ffn, calibrate, backward  # noqa: F401
