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


# --------------------------------------------------------------------------- MXFP4
# The vLLM AgentX article (news.ainew.jp), "Hybrid KV cache management", names an FP4
# indexer (with Figure 5's packed per-block layout), and its "DeepSeek V4" kernel notes name
# MXFP4.  The FP4 keys are read as OCP Microscaling MXFP4: elements are FP4 E2M1 (1 sign, 2
# exponent bits with bias 1, 1 mantissa bit; no infinities or NaN; largest value 6) and
# every 32 consecutive elements share one E8M0 scale (an 8-bit biased exponent: 2^(e-127);
# 0xFF is NaN).


def _e2m1_value(code: int) -> float:
    s = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return s * m * 0.5                    # subnormal: 0.m * 2^(1-1)
    return s * (1.0 + m / 2.0) * 2.0 ** (e - 1)


_E2M1_TABLE = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """FP4 E2M1 codes (0..15) -> float64 values (exact)."""
    return _E2M1_TABLE[np.asarray(codes, dtype=np.uint8) & 0xF]


def e8m0_decode(codes: np.ndarray) -> np.ndarray:
    """E8M0 scale codes -> 2^(code - 127) as float64 (exact); 0xFF -> NaN."""
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


def mxfp4_decode(packed: np.ndarray, scales: np.ndarray, group: int = 32) -> np.ndarray:
    """MXFP4 vectors -> float64.  packed [..., D/2] bytes hold two elements each, element
    2j in the low nibble of byte j and element 2j+1 in the high nibble; scales [..., D/32]
    are the E8M0 codes of the groups of 32 consecutive elements."""
    packed = np.asarray(packed, dtype=np.uint8)
    el = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.float64)
    el[..., 0::2] = e2m1_decode(packed & 0xF)
    el[..., 1::2] = e2m1_decode(packed >> 4)
    return el * np.repeat(e8m0_decode(scales), group, axis=-1)
