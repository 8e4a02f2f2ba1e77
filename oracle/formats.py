"""Exact decoding of the storage formats into float64.  Test infrastructure only.

bf16: the upper 16 bits of an IEEE binary32.
FP8: the pages state that the KV cache is FP8 (GLM-5.3 report, aisoku.org, the
"Configuration and numbers" table: "1M-token FP8 KV"); the flavour is read as OCP
E4M3FN (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no infinities; only
S.1111.111 is NaN; largest finite 448; subnormals m * 2^-9).
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def _e4m3_value(code: int) -> float:
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9           # subnormal: 0.m * 2^(1-7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3FN bytes -> float64 values (exact)."""
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]
