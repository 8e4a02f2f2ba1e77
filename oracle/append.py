"""Paged KV append with per-token FP8 quantisation.  TEST INFRASTRUCTURE ONLY (see the
package docstring).

[AgentX] "Hybrid KV cache management": one shared block pool; a sequence's logical
token t lives in physical block block_table[s][t // bs], row t % bs, so appending the
new tokens of a step is a scatter through the block table.  [GLM] "Configuration and
numbers" (FP8 KV) and "What's new" (the latent KV): the cache stores FP8.  The pages
give no quantiser; the plain reading used here (and stated in the library header) is
per token: amax = max |x|, scale = amax / 448 in float32 (1 when amax = 0), code =
the OCP E4M3FN value nearest to x / scale (float32 division), ties to the even code,
magnitudes beyond 448 clamped to 448.  Both divisions are IEEE float32 so that the
decision of each code is taken in the same precision as in the kernel.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64, e4m3_decode

# the 127 non-negative finite E4M3FN values, code 0x00 .. 0x7E, increasing
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALUES = e4m3_decode(_POS_CODES)


def e4m3_nearest(y: np.ndarray) -> np.ndarray:
    """float32 values -> E4M3FN codes: the nearest representable value, ties to the even
    code (mantissa bit 0 clear), |y| > 448 -> +-448.  Written as a nearest-value search
    over the decoded code table, independent of any bit-level encoder."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))
    a = np.minimum(a, 448.0)
    hi = np.searchsorted(_POS_VALUES, a, side="left")          # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    # the sign bit follows the sign of y (a negative value that rounds to zero is -0, 0x80)
    return code | np.where(np.signbit(y), np.uint8(0x80), np.uint8(0))


def quantize_token_fp8(x_bits: np.ndarray) -> tuple[np.ndarray, np.float32]:
    """One token's bf16 values [D] -> (E4M3 codes [D], float32 scale)."""
    x = bf16_to_f64(x_bits).astype(np.float32)     # exact: bf16 is a subset of float32
    amax = np.float32(np.max(np.abs(x)))
    scale = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
    y = (x / scale).astype(np.float32)
    return e4m3_nearest(y), scale


def token_positions(cached_len, new_len, q_start, n_tokens: int):
    """For each new-token row i: (sequence, logical position), or (-1, -1) for rows that
    belong to no sequence."""
    seq = np.full(n_tokens, -1, dtype=np.int64)
    pos = np.full(n_tokens, -1, dtype=np.int64)
    for s in range(len(new_len)):
        for j in range(int(new_len[s])):
            i = int(q_start[s]) + j
            if 0 <= i < n_tokens:
                seq[i] = s
                pos[i] = int(cached_len[s]) + j
    return seq, pos


def append_gqa(k_pool, v_pool, block_table, cached_len, new_len, q_start, k_new, v_new,
               num_blocks: int | None = None):
    """bf16 pools [NB][Hkv][bs][d] updated with the new rows k_new/v_new [n][Hkv][d]
    (bit patterns copied).  Rows whose block id is out of range are not written."""
    k_pool = k_pool.copy()
    v_pool = v_pool.copy()
    nb, _, bs, _ = k_pool.shape
    seq, pos = token_positions(cached_len, new_len, q_start, k_new.shape[0])
    for i in range(k_new.shape[0]):
        if seq[i] < 0:
            continue
        b = int(block_table[seq[i], pos[i] // bs])
        if not (0 <= b < nb):
            continue
        k_pool[b, :, pos[i] % bs, :] = k_new[i]
        v_pool[b, :, pos[i] % bs, :] = v_new[i]
    return k_pool, v_pool


def append_fp8(pool, scale, block_table, cached_len, new_len, q_start, x_new):
    """FP8 pool [NB][bs][D] (uint8) and scales [NB][bs] updated with the new bf16 rows
    x_new [n][D], each quantised per token."""
    pool = pool.copy()
    scale = scale.copy()
    nb, bs, _ = pool.shape
    seq, pos = token_positions(cached_len, new_len, q_start, x_new.shape[0])
    for i in range(x_new.shape[0]):
        if seq[i] < 0:
            continue
        b = int(block_table[seq[i], pos[i] // bs])
        if not (0 <= b < nb):
            continue
        codes, sc = quantize_token_fp8(x_new[i])
        pool[b, pos[i] % bs, :] = codes
        scale[b, pos[i] % bs] = sc
    return pool, scale
