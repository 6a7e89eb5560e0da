"""CPU oracle for the stochastically rounded INT8 backward of a linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: it is used by ``tests/``, by the smoke
check in ``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of
``bench.py``, and by nothing else.  It shares no code with the HIP library.

It is written from the page "Efficient Quantization Training with Stochastic
Rounding via Structured Subspace Randomness" (cited below as "S3R page",
with its section names) and from the "Stochastic Rounding" explainer page
(cited as "SR explainer").  The display equations (1)-(6) of the S3R page
were lost from the text; each function states which surrounding sentences it
follows and which reading it takes.

Precision: the quantizer decides integers, so it runs in the precision the
GPU kernel uses for that decision (IEEE fp32, one rounding per operation, no
contraction), as numpy float32 element-wise arithmetic.  Everything else
(rounding errors, error-correction statistics, dequantised gradients) is
float64.  Integer GEMMs are exact.

Modules:
  philox    -- Philox4x32-10 counter-based generator and the threshold maps
  quantize  -- fold, step, RTNE / SR / S3R codes, forward-operand prep
  ec        -- S3R-EC error statistics and the structured projection
  backward  -- exact integer GEMMs, dequantised and corrected dX and dW
  swiglu    -- the SwiGLU FFN block's backward glue between the down and the
               gate / up projections (fp32 in a fixed order, bf16 results)

Parity status: every function here is pinned by a test in
``tests/test_oracle_pins.py`` or ``tests/test_oracle_swiglu_pins.py`` (against torch's Philox header, exact rational
arithmetic, closed forms, library routines or brute force); none is marked
"parity unpinned".
"""
from . import philox, quantize, ec, backward  # noqa: F401
