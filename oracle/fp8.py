"""FP8 KV cache values for the oracle (test infrastructure).

The pages count an FP8 cache at one byte per value ([CH] §挑战 2, the KV-size
equation's b, FP8 = 1) and leave FP8 KV outside their study ([CPEV] §限制与待校准项).
The format used is OCP FP8 E4M3 ("fn"): bit 7 sign, bits 6..3 exponent with bias
7, bits 2..0 mantissa; exponent field 0 encodes subnormals m/8 * 2^-6; the codes
0x7f and 0xff are NaN and there are no infinities. A cached value is its
dequantisation scale times the decoded code.
"""
from __future__ import annotations

import numpy as np


def e4m3_to_float(codes) -> np.ndarray:
    """Exact fp64 value of each E4M3 code (uint8 array)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    return np.where((c & 0x7F) == 0x7F, np.nan, sign * mag)


def dequantize(codes, scale: float) -> np.ndarray:
    """scale * value(code), fp64."""
    return float(scale) * e4m3_to_float(codes)
