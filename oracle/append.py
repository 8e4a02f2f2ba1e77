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

from .formats import bf16_to_f64, e2m1_decode, e4m3_decode

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


# --------------------------------------------------------------------------- MXFP4 keys
# The 8 non-negative E2M1 values, code 0 .. 7, increasing.
_FP4_POS_CODES = np.arange(8, dtype=np.uint8)
_FP4_POS_VALUES = e2m1_decode(_FP4_POS_CODES)
FP4_EMAX = 2            # exponent of the largest E2M1 value (6 = 1.5 * 2^2)


def e2m1_nearest(y: np.ndarray) -> np.ndarray:
    """float values -> E2M1 codes: the nearest representable value, ties to the even code
    (mantissa bit clear), |y| > 6 -> +-6; the sign bit follows the sign of y (a negative
    value that rounds to zero is -0, code 0x8).  A nearest-value search over the table."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), 6.0)
    hi = np.minimum(np.searchsorted(_FP4_POS_VALUES, a, side="left"), 7)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _FP4_POS_VALUES[lo]
    d_hi = _FP4_POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_FP4_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _FP4_POS_CODES[hi], _FP4_POS_CODES[lo]).astype(np.uint8)
    return code | np.where(np.signbit(y), np.uint8(0x8), np.uint8(0))


def mx_shared_exponent(amax: float) -> int:
    """E8M0 code of a group whose largest magnitude is amax: the OCP MX conversion takes
    X = 2^(floor(log2 amax) - emax) with emax = 2 for E2M1, so the group's largest element
    lands in [4, 8) before rounding.  An all-zero group takes scale 1 (code 127); codes
    are kept in [2, 252], where every element times the scale is a normal bfloat16 (the
    kernels' staging format) -- the lower clamp acts only for amax < 2^-123."""
    if amax == 0.0:
        return 127
    m, p = np.frexp(np.float64(amax))          # amax = m 2^p, m in [0.5, 1): floor(log2) = p - 1
    return int(min(max(int(p) - 1 - FP4_EMAX + 127, 2), 252))


def quantize_token_mxfp4(x_bits: np.ndarray, group: int = 32) -> tuple[np.ndarray, np.ndarray]:
    """One token's bf16 values [D] -> (packed E2M1 bytes [D/2], E8M0 scale codes [D/32]).
    Each group of 32: code = nearest E2M1 to x / 2^(e-127) (exact division by a power of
    two), element 2j in the low nibble of byte j."""
    x = bf16_to_f64(x_bits)
    d = x.shape[0]
    codes = np.empty(d, dtype=np.uint8)
    scales = np.empty(d // group, dtype=np.uint8)
    for g in range(d // group):
        xs = x[g * group:(g + 1) * group]
        e = mx_shared_exponent(float(np.max(np.abs(xs))))
        scales[g] = e
        codes[g * group:(g + 1) * group] = e2m1_nearest(xs / np.ldexp(1.0, e - 127))
    return (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8), scales


# --------------------------------------------------------------------------- packed blocks
# One allocation per 64-token block holds every cache group of the MLA layer
# ([AgentX] "Hybrid KV cache management", Figure 5: the packed KV cache layout):
#   [0, 36864)       FP8 E4M3 latent   [64][576]
#   [36864, 37120)   fp32 latent scale [64]
#   [37120, 41216)   MXFP4 index keys  [64][64]   (128 elements, two per byte)
#   [41216, 41472)   E8M0 key scales   [64][4]
PACKED_BS = 64
PACKED_LATENT = 0
PACKED_LATENT_SCALE = 64 * 576
PACKED_KEYS = PACKED_LATENT_SCALE + 64 * 4
PACKED_KEY_SCALES = PACKED_KEYS + 64 * 64
PACKED_BLOCK_BYTES = PACKED_KEY_SCALES + 64 * 4


def packed_fields(pool: np.ndarray):
    """Views of a packed pool [NB][41472] bytes: (latent [NB][64][576] u8, latent scale
    [NB][64] f32, keys [NB][64][64] u8, key scales [NB][64][4] u8)."""
    nb = pool.shape[0]
    assert pool.shape[1] == PACKED_BLOCK_BYTES and pool.dtype == np.uint8
    lat = pool[:, PACKED_LATENT:PACKED_LATENT_SCALE].reshape(nb, 64, 576)
    lsc = np.ascontiguousarray(pool[:, PACKED_LATENT_SCALE:PACKED_KEYS]).view(np.float32).reshape(nb, 64)
    keys = pool[:, PACKED_KEYS:PACKED_KEY_SCALES].reshape(nb, 64, 64)
    ksc = pool[:, PACKED_KEY_SCALES:].reshape(nb, 64, 4)
    return lat, lsc, keys, ksc


def append_packed(pool, block_table, cached_len, new_len, q_start, x_new, part: str):
    """Packed pool [NB][41472] bytes updated with the new bf16 rows: part "latent" takes
    x_new [n][576] (FP8 per token, as append_fp8), part "keys" takes x_new [n][128]
    (MXFP4).  Rows whose block id is out of range are not written."""
    pool = pool.copy()
    nb = pool.shape[0]
    seq, pos = token_positions(cached_len, new_len, q_start, x_new.shape[0])
    for i in range(x_new.shape[0]):
        if seq[i] < 0:
            continue
        b = int(block_table[seq[i], pos[i] // PACKED_BS])
        if not (0 <= b < nb):
            continue
        r = int(pos[i] % PACKED_BS)
        if part == "latent":
            codes, sc = quantize_token_fp8(x_new[i])
            pool[b, PACKED_LATENT + 576 * r:PACKED_LATENT + 576 * (r + 1)] = codes
            pool[b, PACKED_LATENT_SCALE + 4 * r:PACKED_LATENT_SCALE + 4 * (r + 1)] = \
                np.array([sc], np.float32).view(np.uint8)
        else:
            packed, scales = quantize_token_mxfp4(x_new[i])
            pool[b, PACKED_KEYS + 64 * r:PACKED_KEYS + 64 * (r + 1)] = packed
            pool[b, PACKED_KEY_SCALES + 4 * r:PACKED_KEY_SCALES + 4 * (r + 1)] = scales
    return pool
