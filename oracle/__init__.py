"""Float64 CPU oracle of the GBLA and LION-s layers.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or run
anything in this package: only the tests, the smoke check and the CPU-baseline
leg of the benchmark use it. It shares no code with the HIP library and its
Python binding; both sides are fed from the seeded input generator, which holds
none of the method's arithmetic.

Modules:
  gbla  -- Eqs. (2)-(6) of "Gated Bidirectional Linear Attention for Generative
           Retrieval" (core method, sections 2 and 3), forward, a quadratic
           brute-force forward, and the hand-derived backward.
  lion  -- the selective-decay mask, the full masked linear-attention form and
           the corrected bidirectional RNN of "Linear Attention for Efficient
           Bidirectional Sequence Modeling" (method details, key designs 1-2),
           forward and backward of the full form.
"""
from . import gbla, lion  # noqa: F401
