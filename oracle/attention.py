"""Plain float64 attention, indexer scores and top-k over contiguous K/V.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Citations name the page and the
section; the pages print no formulas, so each definition is the textbook form of the
operation the passage names:

  [AgentX]  vLLM AgentX article (news.ainew.jp)
  [GLM]     GLM-5.3 on 16xH200 report (aisoku.org)

Conventions (the pages are silent; these are the plain readings):
  * key t is visible to a query at logical position p iff t <= p (inclusive causal);
  * GQA: query head h reads KV head h // (Hq / Hkv);
  * softmax is computed exactly in two passes (max, then exp/sum), never online;
  * the contractions are plain float64 matrix products (numpy matmul, BLAS).
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64, e4m3_decode, mxfp4_decode

_ROW_CHUNK_BYTES = 1 << 28     # bound the size of one score matrix (rows x keys x 8 B)


# --------------------------------------------------------------------------- paging
def gather_paged(pool: np.ndarray, block_row: np.ndarray, n_tokens: int) -> np.ndarray:
    """The oracle's own host gather from a paged pool.

    [AgentX] "Hybrid KV cache management": the page is the single allocation unit and
    one shared block pool serves every sequence through its block table.  Logical token
    t lives in physical block block_row[t // bs], row t % bs.

    pool: [num_blocks][bs][...] (MLA / indexer) or [num_blocks][Hkv][bs][d] (GQA; pass
    it transposed to [num_blocks][bs][Hkv][d]).  Returns [n_tokens][...].
    """
    bs = pool.shape[1]
    out = np.empty((n_tokens,) + pool.shape[2:], dtype=pool.dtype)
    for t0 in range(0, n_tokens, bs):
        b = int(block_row[t0 // bs])
        if b < 0:
            raise ValueError(f"block table has no block for logical token {t0}")
        n = min(bs, n_tokens - t0)
        out[t0:t0 + n] = pool[b, :n]
    return out


# --------------------------------------------------------------------------- attention
def _softmax_rows(s: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Exact two-pass softmax of each row (masked entries are -inf).  Returns P and lse.
    A row with no visible key gets P = 0 and lse = -inf (it carries no weight in a merge)."""
    m = np.max(s, axis=-1, keepdims=True)
    empty = ~np.isfinite(m)
    m = np.where(empty, 0.0, m)
    e = np.exp(s - m)
    z = np.sum(e, axis=-1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(empty, 0.0, e / np.where(empty, 1.0, z))
        lse = np.where(empty, -np.inf, m + np.log(np.where(empty, 1.0, z)))[..., 0]
    return p, lse


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: np.ndarray, scale: float):
    """Causal multi-head / grouped-query softmax attention in float64.

    q [n][Hq][d_qk], k [L][Hkv][d_qk], v [L][Hkv][d_v] (float64), q_pos [n] logical
    positions.  For query i, head h, g = h // (Hq/Hkv):
        s_t = scale * <q[i,h], k[t,g]>  for t <= q_pos[i];  P = softmax(s);  o = sum_t P_t v[t,g]
        lse = log sum_t exp(s_t)
    Returns (o [n][Hq][d_v], lse [n][Hq]).
    The pages name paged attention over a shared pool ([AgentX] "Hybrid KV cache
    management") and MLA with one latent head ([AgentX] "Kimi K3"); GQA grouping is the
    plain reading for the 32-query / 8-KV-head workloads.
    """
    n, Hq, _ = q.shape
    L, Hkv, _ = k.shape
    dv = v.shape[2]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    q_pos = np.asarray(q_pos, dtype=np.int64)
    o = np.empty((n, Hq, dv), dtype=np.float64)
    lse = np.empty((n, Hq), dtype=np.float64)
    rows = max(1, _ROW_CHUNK_BYTES // (8 * max(1, L) * G))
    t = np.arange(L)
    for g in range(Hkv):
        kg = k[:, g, :]
        vg = v[:, g, :]
        for i0 in range(0, n, rows):
            i1 = min(n, i0 + rows)
            qs = q[i0:i1, g * G:(g + 1) * G, :]                     # [r][G][d]
            s = np.matmul(qs, kg.T) * scale                          # [r][G][L]
            mask = t[None, None, :] > q_pos[i0:i1, None, None]
            s = np.where(mask, -np.inf, s)
            p, l_ = _softmax_rows(s)
            o[i0:i1, g * G:(g + 1) * G, :] = np.matmul(p, vg)
            lse[i0:i1, g * G:(g + 1) * G] = l_
    return o, lse


def attention_probs(q, k, q_pos, scale):
    """The probability matrix P [n][Hq][L] of `attention` (for the row-sum and mask pins)."""
    n, Hq, _ = q.shape
    L, Hkv, _ = k.shape
    G = Hq // Hkv
    kk = np.repeat(k, G, axis=1)                                    # [L][Hq][d]
    s = np.einsum("nhd,thd->nht", q, kk) * scale
    s = np.where(np.arange(L)[None, None, :] > np.asarray(q_pos)[:, None, None], -np.inf, s)
    return _softmax_rows(s)[0]


def lse_merge(parts):
    """Merge partial attention results over disjoint key ranges.

    [AgentX] "Kimi K3": each rank writes its partial attention output and its
    log-sum-exp, and the partials are combined locally with online softmax.  For parts
    (o_j, lse_j) (o_j normalised over its own key range):
        M = max_j lse_j;  w_j = exp(lse_j - M);  o = sum_j w_j o_j / sum_j w_j;
        lse = M + log sum_j w_j.
    Parts whose key range is empty carry lse = -inf and weight 0.
    """
    lses = np.stack([p[1] for p in parts])                   # [J][...]
    M = np.max(lses, axis=0)
    w = np.exp(lses - M)
    z = np.sum(w, axis=0)
    o = sum(w[j][..., None] * parts[j][0] for j in range(len(parts))) / z[..., None]
    return o, M + np.log(z)


def paged_gqa_attention(wl, s: int):
    """Attention of sequence s of a paged GQA workload, through the oracle's own gather
    of the pool (bf16 K/V [num_blocks][Hkv][bs][d])."""
    L = int(wl.total_len[s])
    row = wl.block_table[s]
    kp = np.swapaxes(wl.k_pool, 1, 2)                        # [NB][bs][Hkv][d] view
    vp = np.swapaxes(wl.v_pool, 1, 2)
    k = bf16_to_f64(gather_paged(kp, row, L))
    v = bf16_to_f64(gather_paged(vp, row, L))
    q = bf16_to_f64(wl.q_rows(s))
    return attention(q, k, v, wl.q_pos(s), wl.scale)


# --------------------------------------------------------------------------- MLA
def mla_dequant(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """K_t = scale_t * e4m3(codes_t): the FP8 latent KV ([GLM] table: FP8 KV) as float64."""
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]


def mla_attention(q_bits: np.ndarray, kv_codes: np.ndarray, kv_scale: np.ndarray,
                  q_pos: np.ndarray, scale: float, d_v: int = 512):
    """MLA in its shared-latent (MQA) form.

    [GLM] "What's new": the MLA latent KV is shared by all 64 heads; [AgentX] "Kimi K3":
    MLA compresses KV into one latent with a single head.  So Hkv = 1, keys are the whole
    576-wide latent (512 latent + 64 rope dims) and values are its first 512 dims.
    q_bits [n][Hq][576] bf16, kv_codes [L][576] e4m3, kv_scale [L] fp32.
    """
    kk = mla_dequant(kv_codes, kv_scale)                      # [L][576]
    k = kk[:, None, :]
    v = kk[:, None, :d_v]
    return attention(bf16_to_f64(q_bits), k, v, q_pos, scale)


def indexer_scores(q_bits: np.ndarray, w: np.ndarray, k_codes: np.ndarray, k_scale: np.ndarray,
                   q_pos: np.ndarray) -> np.ndarray:
    """Indexer scores I[i, t] = sum_h w[i,h] * max(0, <q[i,h], k_t>), t <= pos(i), else -inf.

    [AgentX] "DeepSeek V4": the indexer has 64 heads but yields one global top-k per
    token; [GLM] "What's new": the indexer picks 2,048 tokens and its cost is quadratic
    in the prompt.  k_t = scale_t * e4m3(k_codes_t) is one 128-wide key per token shared
    by every indexer head.  q_bits [n][H][d] bf16, w [n][H] fp32.
    """
    return indexer_scores_from_keys(q_bits, w, mla_dequant(k_codes, k_scale), q_pos)


def indexer_scores_mxfp4(q_bits: np.ndarray, w: np.ndarray, k_packed: np.ndarray, k_scales: np.ndarray,
                         q_pos: np.ndarray) -> np.ndarray:
    """indexer_scores with MXFP4 keys ([AgentX] "Hybrid KV cache management": the FP4
    indexer): k_t = the decoded MXFP4 vector of token t (k_packed [L][d/2] bytes, k_scales
    [L][d/32] E8M0 codes)."""
    return indexer_scores_from_keys(q_bits, w, mxfp4_decode(k_packed, k_scales), q_pos)


def indexer_scores_from_keys(q_bits: np.ndarray, w: np.ndarray, k: np.ndarray, q_pos: np.ndarray) -> np.ndarray:
    """I[i, t] = sum_h w[i,h] * max(0, <q[i,h], k[t]>) for t <= pos(i), else -inf, with the
    keys already decoded to float64 k [L][d]."""
    q = bf16_to_f64(q_bits)                                   # [n][H][d]
    wf = np.asarray(w, dtype=np.float64)
    n, L = q.shape[0], k.shape[0]
    out = np.empty((n, L), dtype=np.float64)
    t = np.arange(L)
    rows = max(1, _ROW_CHUNK_BYTES // (8 * max(1, L) * q.shape[1]))
    for i0 in range(0, n, rows):
        i1 = min(n, i0 + rows)
        s = np.matmul(q[i0:i1], k.T)                          # [r][H][L]
        sc = np.matmul(wf[i0:i1, None, :], np.maximum(s, 0.0))[:, 0, :]   # sum over heads
        out[i0:i1] = np.where(t[None, :] > np.asarray(q_pos[i0:i1])[:, None], -np.inf, sc)
    return out


def topk_indices(scores: np.ndarray, valid_len: int, k: int) -> np.ndarray:
    """The k highest-scoring of tokens 0..valid_len-1, ties to the lower token index,
    returned in ascending token order and padded with -1 to length k.

    [GLM] "What's new" and "How to try": the indexer selects 2,048 tokens per query
    token.  Order and padding are not stated; ascending order with -1 padding is the
    reading chosen.  Selection is a full stable sort by (-score, index).
    """
    valid_len = int(valid_len)
    s = np.asarray(scores[:valid_len], dtype=np.float64)
    order = np.lexsort((np.arange(valid_len), -s))           # last key is primary
    take = np.sort(order[:min(k, valid_len)])
    out = np.full(k, -1, dtype=np.int32)
    out[:take.shape[0]] = take
    return out


def sparse_mla_attention(q_bits: np.ndarray, kv_codes: np.ndarray, kv_scale: np.ndarray,
                         topk: np.ndarray, scale: float, d_v: int = 512):
    """Sparse MLA: each query token attends only to its selected tokens.

    [AgentX] "DeepSeek V4": sparse MLA scans and gathers the top-k KV entries, then
    attends; [GLM] "How to try": prompts that fit inside the 2,048-token top-k still go
    through the same sparse (MQA) kernel.  q_bits [n][Hq][576]; kv_codes [L][576] and
    kv_scale [L] are the sequence's contiguous latent cache; topk [n][k] logical
    positions, -1 = skip.  The causal mask is implied by the selection.
    """
    q = bf16_to_f64(q_bits)
    n, Hq, _ = q.shape
    o = np.empty((n, Hq, d_v), dtype=np.float64)
    lse = np.empty((n, Hq), dtype=np.float64)
    for i in range(n):
        sel = topk[i][topk[i] >= 0]
        if sel.size == 0:
            o[i], lse[i] = 0.0, -np.inf
            continue
        kk = mla_dequant(kv_codes[sel], kv_scale[sel])       # [m][576]
        s = (q[i] @ kk.T) * scale                             # [Hq][m]
        p, l_ = _softmax_rows(s)
        o[i] = p @ kk[:, :d_v]
        lse[i] = l_
    return o, lse
