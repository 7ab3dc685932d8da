"""fp8 KV-cache values for the oracle -- test infrastructure.

The decode page section "Decoding KV Cache Layout 优化" stores each token's
quantised data next to its scales; the fp8 decode workload quantises every KV
row to FP8 E4M3 with one float32 scale per group of 128 consecutive columns
(576 columns give five groups, the last one 64 wide).  The value of an element
is code_value * scale, where code_value is the E4M3 number the byte encodes.

E4M3 here is the OCP 8-bit floating point format, "fn" variant
(OCP Microscaling / OFP8 specification): 1 sign bit, 4 exponent bits with
bias 7, 3 mantissa bits; exponent field 0 encodes subnormals m * 2^-9; there
are no infinities; S.1111.111 is NaN; the largest finite value is
1.75 * 2^8 = 448.

The decode is written from that definition (no lookup in any library); the
tests check it against torch's float8_e4m3fn conversion.
"""
from __future__ import annotations

import numpy as np

FP8_GROUP = 128


def e4m3fn_decode(codes) -> np.ndarray:
    """Exact float64 values of E4M3 (fn) byte codes; NaN for the NaN codes."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = m * 2.0 ** -9
    v = np.where(e == 0, subnormal, normal)
    v = np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, v)
    return sign * v


def dequant_fp8_rows(codes, scales, group: int = FP8_GROUP) -> np.ndarray:
    """Exact float64 KV rows from fp8 codes [rows, d] and float32 group scales
    [rows, ceil(d / group)]: value[r, c] = e4m3(codes[r, c]) * scales[r, c // group].
    Both factors are exact in float64 and their product (4 + 24 significant
    bits) is exact too."""
    codes = np.asarray(codes)
    scales = np.asarray(scales, dtype=np.float32).astype(np.float64)
    rows, d = codes.shape
    ng = -(-d // group)
    assert scales.shape == (rows, ng)
    col_group = np.arange(d) // group
    return e4m3fn_decode(codes) * scales[:, col_group]
