"""FP8 (E4M3) KV-cache values in fp64 — oracle (test infrastructure only).

The pages name FP8 among the KV-cache / attention precisions ([Tool]
"FlashInfer", section "What it does": low-precision compute for attention;
[Windows] "flashinfer-windows" README, feature list: FP8 quantization for
attention) and give GEMM FP8 a per-tensor scale ([Guide] "Features (from the
repository README)"). They fix neither the 8-bit format nor where the scale
sits. Reading taken:

* the format is OCP 8-bit floating point E4M3 (the "fn" variant without
  infinities): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
  exponent field 0 is subnormal (``m/8 * 2^-6``); the code with every
  exponent and mantissa bit set is NaN; the largest finite value is 448;
* one float scale per tensor (one for all of K, one for all of V): the stored
  code ``c`` stands for ``scale * e4m3(c)``.

The decoding below is the format's definition written out, not a table.
"""
from __future__ import annotations

import numpy as np

E4M3_BIAS = 7
E4M3_MAX = 448.0


def e4m3_value(codes: np.ndarray) -> np.ndarray:
    """Value of each E4M3 byte code as float64 (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - E4M3_BIAS)
    subnormal = (m / 8.0) * np.exp2(1.0 - E4M3_BIAS)
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where((e == 15) & ((c & 0x7) == 7), np.nan, mag)
    return sign * mag
