"""fp4 KV-cache values for the oracle -- test infrastructure.

The decode section of the page "Ascend Sparse Attention Forward
算法与优化技术简析" names an FP4 KV cache beside the FP8 one, both dequantised
to bf16 for the products.  The fp4 decode workload stores every KV element as
an E2M1 code with one float32 scale per group of 128 consecutive columns
(five groups for 576 columns, as for fp8).  The value of an element is
code_value * scale.

E2M1 is the 4-bit floating point element format of the OCP Microscaling (MX)
specification: 1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit; the
exponent field 0 encodes the subnormals m * 0.5; there are no infinities and
no NaN; the largest value is 1.5 * 2^2 = 6.  Bit 3 of the 4-bit code is the
sign, bits 2..1 the exponent, bit 0 the mantissa.
"""
from __future__ import annotations

import numpy as np

FP4_GROUP = 128


def e2m1_decode(codes) -> np.ndarray:
    """Exact float64 values of E2M1 4-bit codes (integers 0..15)."""
    c = np.asarray(codes).astype(np.int64)
    if np.any((c < 0) | (c > 15)):
        raise ValueError("E2M1 codes are 4-bit")
    sign = np.where(c >> 3, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    normal = (1.0 + m / 2.0) * np.exp2(e.astype(np.float64) - 1.0)
    subnormal = m * 0.5
    return sign * np.where(e == 0, subnormal, normal)


def dequant_fp4_rows(codes, scales, group: int = FP4_GROUP) -> np.ndarray:
    """Exact float64 KV rows from E2M1 codes [rows, d] (one code per entry)
    and float32 group scales [rows, ceil(d / group)]:
    value[r, c] = e2m1(codes[r, c]) * scales[r, c // group]; the product of a
    2-bit and a 24-bit significand is exact in float64."""
    codes = np.asarray(codes)
    scales = np.asarray(scales, dtype=np.float32).astype(np.float64)
    rows, d = codes.shape
    ng = -(-d // group)
    assert scales.shape == (rows, ng)
    return e2m1_decode(codes) * scales[:, np.arange(d) // group]
