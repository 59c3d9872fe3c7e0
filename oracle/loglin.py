"""Exp-free (log-linear) probability encoders of the oracle.  TEST INFRASTRUCTURE ONLY.

Two related methods listed on the arXiv listing of "Hardware-Aware FP4
FlashAttention-4" (2609.04105v1), section "Related papers", turn a log2-domain
score into a low-precision probability code without evaluating 2**x:

* "VC-Attention: Value Smoothing and Softmax Casting for Low-bit Attention":
  the shifted log-domain score becomes an E4M3 probability code through one
  fused multiply-add, with neither the FP32 exponential nor a format
  conversion.
* "EFQ-Softmax: Exp-Free Quantization for Softmax": shifted scores become
  block-scaled E2M1 operands directly, with no exponential.

Only the abstracts are on the pages.  Reading taken for both (the plainest one
that an FMA alone can realise): a minifloat with M mantissa bits and exponent
bias b stores, for a normal value 2**n * (1 + j / 2**M), the integer code
2**M * (n + b) + j, so the code read as an integer is a fixed-point log2 of
the value.  The cast therefore takes

    code = clamp(RNE(2**M * (y + b)), 0, top)

with y the log2 of the wanted probability (y = t - m' for FP8 E4M3 with unit
scale, M = 3, b = 7; y = t - m' - e for E2M1 under the same E8M0 block exponent
e as Direct-P, M = 1, b = 1), RNE = round half to even, and top the largest
finite code (0x7E for E4M3, 7 for E2M1).  y = -inf (a masked key) gives 0.
The value that a code decodes to is Mitchell's piecewise-linear 2**y with its
fraction rounded to M bits in the normal range, and the subnormal value of the
code below it (codes under 2**M).  The denominator and P.V both use the
decoded codes, as in Direct-P.
"""

import numpy as np

# format -> (mantissa bits M, exponent bias b, largest finite code)
LOGLIN_FORMATS = {
    "e4m3": (3, 7, 0x7E),
    "e2m1": (1, 1, 7),
}


def loglin_position(y, fmt):
    """The unrounded code position 2**M * (y + b) of log2-domain values ``y``
    (float64; -inf stays -inf)."""
    mbits, bias, _ = LOGLIN_FORMATS[fmt]
    return np.ldexp(np.asarray(y, dtype=np.float64) + bias, mbits)


def loglin_round(z, fmt):
    """Code of an unrounded position z: clamp(RNE(z), 0, top); -inf -> 0."""
    top = LOGLIN_FORMATS[fmt][2]
    z = np.asarray(z, dtype=np.float64)
    z = np.where(np.isfinite(z), z, -1.0)      # -inf (masked key) -> code 0
    return np.clip(np.rint(z), 0, top).astype(np.uint8)


def loglin_encode(y, fmt):
    """Log-linear cast of log2-domain values ``y`` (float64, -inf allowed) to
    unsigned minifloat codes (uint8): clamp(RNE(2**M * (y + b)), 0, top)."""
    return loglin_round(loglin_position(y, fmt), fmt)
