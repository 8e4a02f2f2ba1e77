"""Pins for the oracle's MLA, indexer scores, top-k and sparse MLA (CPU only)."""
import math

import numpy as np
import pytest

import oracle
import workloads as W


def _brute_mla(qf, kf, pos, scale, dv):
    n, H, _ = qf.shape
    o = np.zeros((n, H, dv))
    for i in range(n):
        for h in range(H):
            vis = range(pos[i] + 1)
            s = [scale * math.fsum(qf[i, h] * kf[t]) for t in vis]
            m = max(s)
            ex = [math.exp(x - m) for x in s]
            z = math.fsum(ex)
            for e in range(dv):
                o[i, h, e] = math.fsum(ex[t] * kf[t, e] for t in vis) / z
    return o


def test_mla_is_mqa_over_the_dequantised_latent():
    """One latent shared by all heads: keys are all 576 dims, values the first 512."""
    mla = W.make_mla_decode(41, lengths=[9], num_q_heads=3, keep_content=True)
    codes, sc = mla.kv_contiguous(0)
    q = mla.q_rows(0)
    pos = mla.q_pos(0)
    o, _ = oracle.mla_attention(q, codes, sc, pos, mla.scale)
    kf = oracle.e4m3_decode(codes) * sc[:, None].astype(np.float64)
    ob = _brute_mla(oracle.bf16_to_f64(q), kf, pos, mla.scale, 512)
    np.testing.assert_allclose(o, ob, rtol=1e-11, atol=1e-13)


def test_mla_paged_gather_matches_contiguous():
    mla = W.make_mla_decode(42, lengths=[130, 64, 5], num_q_heads=2, keep_content=True)
    for s in range(3):
        L = int(mla.total_len[s])
        g = oracle.gather_paged(mla.kv_pool, mla.block_table[s], L)
        gs = oracle.gather_paged(mla.kv_scale[..., None],
                                 mla.block_table[s], L)[:, 0]
        c, cs = mla.kv_contiguous(s)
        assert np.array_equal(g, c) and np.array_equal(gs, cs)


def test_mla_equal_keys_give_mean_of_values():
    L = 20
    codes = np.tile(np.arange(576, dtype=np.uint8) % 0x70, (L, 1))
    codes[:, :512] = np.random.default_rng(1).integers(0, 0x70, (L, 512))
    codes[:, :] = codes[0]                           # identical keys (and so values)
    sc = np.full(L, 0.5, np.float32)
    q = W.bf16_bits(np.random.default_rng(2).standard_normal((1, 4, 576)).astype(np.float32))
    o, lse = oracle.mla_attention(q, codes, sc, np.array([L - 1]), 1 / 24)
    v0 = oracle.e4m3_decode(codes[0, :512]) * 0.5
    np.testing.assert_allclose(o[0], np.tile(v0, (4, 1)), atol=1e-12)


def _brute_indexer(q, w, k, pos):
    n, H, d = q.shape
    L = k.shape[0]
    out = np.full((n, L), -np.inf)
    for i in range(n):
        for t in range(pos[i] + 1):
            out[i, t] = math.fsum(w[i, h] * max(0.0, math.fsum(q[i, h] * k[t])) for h in range(H))
    return out


def test_indexer_brute_force():
    rng = np.random.default_rng(5)
    n, H, d, L = 4, 3, 8, 13
    q = W.bf16_bits(rng.standard_normal((n, H, d)).astype(np.float32))
    w = rng.standard_normal((n, H)).astype(np.float32)
    kc, ks = W.fp8_quantize_tokens(rng.standard_normal((L, d)).astype(np.float32))
    pos = np.array([3, 7, 11, 12])
    got = oracle.indexer_scores(q, w, kc, ks, pos)
    kf = oracle.e4m3_decode(kc) * ks[:, None].astype(np.float64)
    ref = _brute_indexer(oracle.bf16_to_f64(q), w.astype(np.float64), kf, pos)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got))
    np.testing.assert_allclose(got[fin], ref[fin], rtol=1e-12, atol=1e-12)


def test_indexer_single_head_positive_is_dot_product():
    rng = np.random.default_rng(6)
    d, L = 16, 9
    q = W.bf16_bits(np.abs(rng.standard_normal((2, 1, d))).astype(np.float32))
    kc, ks = W.fp8_quantize_tokens(np.abs(rng.standard_normal((L, d))).astype(np.float32) + 0.1)
    got = oracle.indexer_scores(q, np.ones((2, 1), np.float32), kc, ks, np.array([L - 1, L - 1]))
    kf = oracle.e4m3_decode(kc) * ks[:, None].astype(np.float64)
    np.testing.assert_allclose(got, oracle.bf16_to_f64(q)[:, 0] @ kf.T, rtol=1e-13)


def test_indexer_scale_commutes_with_relu():
    """ReLU(s x) = s ReLU(x) for s > 0: the per-token key scale can be applied after the
    weighted head sum."""
    rng = np.random.default_rng(7)
    n, H, d, L = 3, 8, 32, 40
    q = W.bf16_bits(rng.standard_normal((n, H, d)).astype(np.float32))
    w = rng.standard_normal((n, H)).astype(np.float32)
    kc, ks = W.fp8_quantize_tokens(rng.standard_normal((L, d)).astype(np.float32))
    pos = np.full(n, L - 1)
    a = oracle.indexer_scores(q, w, kc, ks, pos)
    b = oracle.indexer_scores(q, w, kc, np.ones(L, np.float32), pos) * ks[None, :].astype(np.float64)
    np.testing.assert_allclose(a, b, rtol=1e-14, atol=1e-15)


def _brute_topk(row, valid, k):
    items = sorted(range(valid), key=lambda t: (-row[t], t))[:k]
    out = sorted(items) + [-1] * (k - min(k, valid))
    return np.array(out, np.int32)


@pytest.mark.parametrize("k", [1, 3, 50, 55])
def test_topk_brute_force(k):
    rng = np.random.default_rng(8)
    L = 50
    for trial in range(20):
        row = rng.standard_normal(L + 7)
        valid = int(rng.integers(1, L + 1))
        assert np.array_equal(oracle.topk_indices(row, valid, k), _brute_topk(row, valid, k))


def test_topk_ties_go_to_lower_index():
    s = W.tie_scores(1, 10, 300)
    for r in range(10):
        row = s[r]
        for k in (1, 17, 100, 299):
            got = oracle.topk_indices(row, 300, k)
            assert np.all(np.diff(got) > 0)
            thr = np.sort(row)[::-1][k - 1]
            assert np.all(row[got] >= thr)
            above = np.flatnonzero(row > thr)
            assert set(above) <= set(got)
            eq_taken = [t for t in got if row[t] == thr]
            eq_all = np.flatnonzero(row == thr)
            assert eq_taken == list(eq_all[:len(eq_taken)])


def test_topk_k_at_least_valid_returns_all_valid_ascending():
    row = np.random.default_rng(9).standard_normal(30)
    got = oracle.topk_indices(row, 12, 20)
    assert np.array_equal(got[:12], np.arange(12)) and np.all(got[12:] == -1)


def test_topk_negative_zero_ties_positive_zero():
    row = np.array([0.0, -0.0, 0.0, -1.0, -0.0])
    assert np.array_equal(oracle.topk_indices(row, 5, 2), [0, 1])


def test_sparse_with_k_at_least_context_equals_dense():
    """GLM-5.3 report, 'How to try': prompts that fit inside the top-k still run the
    sparse kernel; so with k >= context sparse MLA must equal dense MLA."""
    mla = W.make_mla_decode(43, lengths=[70], num_q_heads=4, q_per_seq=5, keep_content=True)
    codes, sc = mla.kv_contiguous(0)
    q = mla.q_rows(0)
    pos = mla.q_pos(0)
    dense, dl = oracle.mla_attention(q, codes, sc, pos, mla.scale)
    dummy = np.random.default_rng(3).standard_normal((5, 70))
    topk = np.stack([oracle.topk_indices(dummy[i], pos[i] + 1, 128) for i in range(5)])
    sp, sl = oracle.sparse_mla_attention(q, codes, sc, topk, mla.scale)
    np.testing.assert_allclose(sp, dense, atol=1e-13)
    np.testing.assert_allclose(sl, dl, atol=1e-13)


def test_sparse_subset_equals_masked_dense():
    """Selecting a subset equals dense attention with the other keys masked out."""
    mla = W.make_mla_decode(44, lengths=[40], num_q_heads=2, q_per_seq=1, keep_content=True)
    codes, sc = mla.kv_contiguous(0)
    q = mla.q_rows(0)
    sel = np.array([[1, 5, 6, 20, 39, -1, -1]], np.int32)
    sp, _ = oracle.sparse_mla_attention(q, codes, sc, sel, mla.scale)
    keep = sel[0][sel[0] >= 0]
    dense, _ = oracle.mla_attention(q, codes[keep], sc[keep], np.array([len(keep) - 1]), mla.scale)
    np.testing.assert_allclose(sp, dense, atol=1e-14)
