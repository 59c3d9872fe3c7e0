"""Plain CPU oracle for the Direct-P FP4 attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) may import, call or link this package.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use
it.

The oracle is written from the method's description on the pages
"Hardware-Aware FP4 FlashAttention-4" (summary page, section "What the paper
found"; arXiv listing 2609.04105v1, abstract): NVFP4 Q and K, scores mapped
straight to MXFP4 E2M1 probability codes with one E8M0 scale per 32 keys, the
softmax denominator summed from the same rounded probabilities that feed P.V,
FP8 or MXFP4 V, and an FP8 P/V variant for causal training.  Where the pages
leave a step open, the reading chosen is stated in the docstring of the
function that implements it.

Numerics: quantization runs in numpy float32 (IEEE round-to-nearest-even),
following the stated operation order; attention runs in float64.

Modules:
  formats    -- E2M1, E4M3 (fn) and E8M0 codecs
  quant      -- NVFP4 (Q, K), FP8 E4M3 per-tensor and MXFP4 (V) quantizers
  attention  -- Direct-P and FP8-P/V tiled forward, exact softmax attention
  loglin     -- exp-free log-linear probability casts (E4M3, E2M1) of the
                related methods listed beside the arXiv entry
  backward   -- causal-training backward: probabilities rebuilt from the
                saved quantized Q/K and LSE, FP8 gradient operands (E5M2 dO)

Parity status: every function is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py`` (closed forms, exhaustive codec checks against
torch's float8 dtypes, invariants, and an exact-attention special case).
"""

from . import formats, quant, attention, loglin, backward  # noqa: F401
