"""GPU parity at the benchmarked sizes: the suffix prefill (8 x (142,000 + 2,048)), the
MLA MTP3 decode (64 sequences, contexts 32K-256K) and the indexer -> top-2,048 -> sparse
MLA chain at 131,072 cached + 4,096 new tokens, plus a multi-chunk indexer case whose
query positions sit on the 8,192-key chunk edges.

Each call runs at its real shape and launch configuration; the oracle (fp64, contiguous
K/V gathered by its own host loop) checks sampled rows.  Top-k is compared bit-exactly
against the oracle's selection on the GPU's own scores (identical scores); against the
oracle's fp64 scores, any index that differs must be a near-tie at the k-th score.
"""
import time

import numpy as np
import pytest

import oracle
import workloads as W
from workloads.device import GqaOnDevice, MlaOnDevice
from gpu_util import BF16_L1, BF16_MAX_ABS, FP8_L1, FP8_MAX_ABS, LSE_ABS, assert_close, bf16_out

pytestmark = pytest.mark.gpu


def _log(msg):
    print(f"[full-size] {msg}", flush=True)


def test_suffix_prefill_full_size_sampled(pa_lib):
    """8 sequences x (142,000 cached + 2,048 new), 32q/8kv, d128: the first and last new
    token, both sides of a 64-token tile edge and one middle token of sequences 0 and 7,
    all 32 heads, against the oracle over each row's visible keys."""
    import torch
    t0 = time.time()
    wl = W.make_prefix_prefill(3)
    dev = GqaOnDevice(wl)
    _log(f"suffix prefill workload ready in {time.time() - t0:.1f}s")
    lse = torch.empty((wl.q.shape[0], wl.num_q_heads), dtype=torch.float32, device="cuda")
    out = pa_lib.paged_attn_prefill(dev.q, dev.pool, dev.bt, dev.cached, dev.n_new, dev.q_start,
                                    num_q_heads=wl.num_q_heads, max_new_len=dev.max_new,
                                    max_total_len=dev.max_total, scale=wl.scale, lse=lse)
    torch.cuda.synchronize()
    got, lg = bf16_out(out), lse.cpu().numpy()
    del dev, out, lse
    torch.cuda.empty_cache()
    kp, vp = np.swapaxes(wl.k_pool, 1, 2), np.swapaxes(wl.v_pool, 1, 2)
    toks = np.array([0, 63, 64, 1000, 2047])
    for s in (0, 7):
        L = int(wl.total_len[s])
        k = oracle.bf16_to_f64(oracle.gather_paged(kp, wl.block_table[s], L))
        v = oracle.bf16_to_f64(oracle.gather_paged(vp, wl.block_table[s], L))
        rows = wl.q_start[s] + toks
        ro, rl = oracle.attention(oracle.bf16_to_f64(wl.q[rows]), k, v, wl.q_pos(s)[toks], wl.scale)
        assert_close(got[rows], ro, BF16_MAX_ABS, BF16_L1, f"suffix prefill seq={s} tokens={list(toks)}")
        np.testing.assert_allclose(lg[rows], rl, atol=LSE_ABS)


def test_mla_mtp3_decode_full_size_sampled(pa_lib):
    """64 sequences x 4 MTP tokens, 64 heads, FP8 latent, contexts U[32768, 262144]: the
    shortest, median and longest sequences (all 4 tokens x 64 heads, up to 43 splits)."""
    import torch
    t0 = time.time()
    mla = W.make_mla_decode(4)
    dev = MlaOnDevice(mla)
    _log(f"MLA decode workload ready in {time.time() - t0:.1f}s")
    S, T, H = mla.num_seqs, 4, mla.num_q_heads
    lse = torch.empty((S, T, H), dtype=torch.float32, device="cuda")
    out = pa_lib.paged_attn_decode(dev.q.view(S, T, H, 576), dev.pool, dev.bt, dev.total_len, q_per_seq=T,
                                   num_q_heads=H, max_context_len=dev.max_total, scale=mla.scale, lse=lse)
    torch.cuda.synchronize()
    got = bf16_out(out).reshape(S * T, H, 512)
    lg = lse.cpu().numpy().reshape(S * T, H)
    del dev, out, lse
    torch.cuda.empty_cache()
    order = np.argsort(mla.total_len, kind="stable")
    for s in (int(order[0]), int(order[S // 2]), int(order[-1])):
        L = int(mla.total_len[s])
        codes = oracle.gather_paged(mla.kv_pool, mla.block_table[s], L)
        sc = oracle.gather_paged(mla.kv_scale[..., None], mla.block_table[s], L)[:, 0]
        ro, rl = oracle.mla_attention(mla.q_rows(s), codes, sc, mla.q_pos(s), mla.scale)
        assert_close(got[s * T:(s + 1) * T], ro, FP8_MAX_ABS, FP8_L1, f"MLA MTP3 full seq={s} L={L}")
        np.testing.assert_allclose(lg[s * T:(s + 1) * T], rl, atol=LSE_ABS)


def _indexer_chain(pa, dev, k):
    import torch
    n_q = dev.q_idx.shape[0]
    scores = torch.empty((n_q, dev.max_total), dtype=torch.float32, device="cuda")
    topk = pa.mla_indexer_topk(dev.q_idx, dev.w, dev.idx_pool, dev.bt, dev.cached, dev.n_new, dev.q_start,
                               max_new_len=dev.max_new, max_total_len=dev.max_total, k=k, scores_out=scores)
    torch.cuda.synchronize()
    return topk, scores


def _check_scores_and_topk(mla, idx, s, rows, sc_rows, topk_rows, k, what):
    """Scores of the given query rows (global row ids) of sequence s against the oracle,
    and their top-k against the oracle's selection on those same (GPU) scores."""
    L = int(mla.total_len[s])
    kc = oracle.gather_paged(idx.idx_pool, mla.block_table[s], L)
    ks = oracle.gather_paged(idx.idx_scale[..., None], mla.block_table[s], L)[:, 0]
    pos = mla.q_pos(s)[rows - mla.q_start[s]]
    ref = oracle.indexer_scores(idx.q_idx[rows], idx.w[rows], kc, ks, pos)
    got = sc_rows[:, :L].astype(np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got)), f"{what}: -inf pattern differs"
    assert np.all(np.isneginf(sc_rows[:, L:])), f"{what}: scores past the context must be -inf"
    err = np.abs(got[fin] - ref[fin])
    scale_ref = np.abs(ref[fin]).max()
    print(f"{what}: indexer max_abs={err.max():.3e} (ref max {scale_ref:.2f})", flush=True)
    assert err.max() <= 2e-3 * scale_ref
    for r in range(len(rows)):
        exact = oracle.topk_indices(got[r], pos[r] + 1, k)
        assert np.array_equal(topk_rows[r], exact), (what, int(rows[r]))
        oref = oracle.topk_indices(ref[r], pos[r] + 1, k)
        diff = np.setxor1d(oref[oref >= 0], topk_rows[r][topk_rows[r] >= 0])
        if diff.size:
            kth = np.sort(ref[r][:pos[r] + 1])[::-1][min(k, pos[r] + 1) - 1]
            assert np.all(np.abs(ref[r][diff] - kth) <= 2 * err.max() + 1e-12), (what, int(rows[r]))
    return kc, ks


def test_indexer_multi_chunk_edges(pa_lib):
    """Keys in 8,192-key chunks: query positions 8,190-8,193 and 16,382-16,385 straddle the
    first two chunk edges, 19,991-19,999 sit in the last (partial) chunk; rows of three
    sequences share workgroups.  Full score rows and the top-2,048 of every row."""
    lengths, n_new = [8194, 16386, 20000], [4, 4, 9]
    mla, idx = W.make_sparse_mla(94, lengths=lengths, n_new=n_new, num_q_heads=16)
    dev = MlaOnDevice(mla, idx)
    k = 2048
    topk, scores = _indexer_chain(pa_lib, dev, k)
    tk, sc = topk.cpu().numpy(), scores.cpu().numpy()
    for s in range(3):
        rows = np.arange(mla.q_start[s], mla.q_start[s + 1])
        _check_scores_and_topk(mla, idx, s, rows, sc[rows], tk[rows], k, f"multi-chunk seq={s}")


def test_indexer_topk_sparse_mla_full_size(pa_lib):
    """The whole sparse-MLA chain at 131,072 cached + 4,096 new tokens (17 indexer chunks):
    scores of 32 sampled rows against the oracle, top-2,048 of 256 rows bit-exact on the
    GPU's scores, and sparse MLA (64 heads, FP8 latent) on the GPU's selections for 32
    rows against the oracle on the same index sets."""
    import torch
    t0 = time.time()
    mla, idx = W.make_sparse_mla(5)
    dev = MlaOnDevice(mla, idx)
    _log(f"sparse MLA workload ready in {time.time() - t0:.1f}s")
    n_q, k = dev.q_idx.shape[0], 2048
    topk, scores = _indexer_chain(pa_lib, dev, k)
    lse = torch.empty((n_q, mla.num_q_heads), dtype=torch.float32, device="cuda")
    out = pa_lib.sparse_mla_attn(dev.q, dev.pool, dev.bt, dev.q_seq, topk, scale=mla.scale, lse=lse)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    top_rows = np.unique(np.concatenate([[0, 1, 2047, 2048, n_q - 2, n_q - 1],
                                         rng.choice(n_q, 250, replace=False)]))
    rows_t = torch.from_numpy(top_rows).cuda()
    sc = scores.index_select(0, rows_t).cpu().numpy()
    tk_all = topk.cpu().numpy()
    got = bf16_out(out)
    lg = lse.cpu().numpy()
    del scores, out, lse
    torch.cuda.empty_cache()
    # every row holds k distinct, ascending, causal-valid positions
    pos_all = mla.q_pos(0)
    assert np.all(np.diff(tk_all, axis=1) > 0) and np.all(tk_all >= 0)
    assert np.all(tk_all[:, -1] <= pos_all)
    # top-k bit-exact on the GPU's own scores for all sampled rows; scores vs the oracle
    # for 32 of them (first, last, around the middle, random)
    score_pick = np.unique(np.concatenate([[0, 1, 2047, 2048, n_q - 1], rng.choice(top_rows, 27, replace=False)]))
    sel = np.searchsorted(top_rows, score_pick)
    kc, ks = _check_scores_and_topk(mla, idx, 0, score_pick, sc[sel], tk_all[score_pick], k, "cfg5 indexer")
    for j, r in enumerate(top_rows):
        exact = oracle.topk_indices(sc[j].astype(np.float64), pos_all[r] + 1, k)
        assert np.array_equal(tk_all[r], exact), int(r)
    _log(f"top-k of {len(top_rows)} rows bit-exact on the GPU scores")
    # sparse MLA on the GPU's selections
    L = int(mla.total_len[0])
    codes = oracle.gather_paged(mla.kv_pool, mla.block_table[0], L)
    cs = oracle.gather_paged(mla.kv_scale[..., None], mla.block_table[0], L)[:, 0]
    ro, rl = oracle.sparse_mla_attention(mla.q[score_pick], codes, cs, tk_all[score_pick], mla.scale)
    assert_close(got[score_pick], ro, FP8_MAX_ABS, FP8_L1, "cfg5 sparse MLA sampled rows")
    np.testing.assert_allclose(lg[score_pick], rl, atol=LSE_ABS)
