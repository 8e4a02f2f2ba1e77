"""Pins for the oracle's attention (CPU only).

Each test ties the oracle to something other than itself: a hand-derived example, a
brute-force loop written independently with math.fsum, closed forms, invariants, the
GQA == repeated-KV MHA special case, block-table permutations, and the LSE merge
identity of partial results.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute(q, k, v, q_pos, scale):
    """Independent triple loop with exact summation (math.fsum)."""
    n, Hq, _ = q.shape
    L, Hkv, _ = k.shape
    G = Hq // Hkv
    o = np.zeros((n, Hq, v.shape[2]))
    lse = np.zeros((n, Hq))
    for i in range(n):
        for h in range(Hq):
            g = h // G
            vis = [t for t in range(L) if t <= q_pos[i]]
            s = [scale * math.fsum(q[i, h, e] * k[t, g, e] for e in range(q.shape[2])) for t in vis]
            m = max(s)
            ex = [math.exp(x - m) for x in s]
            z = math.fsum(ex)
            for e in range(v.shape[2]):
                o[i, h, e] = math.fsum(ex[j] * v[t, g, e] for j, t in enumerate(vis)) / z
            lse[i, h] = m + math.log(z)
    return o, lse


def test_golden_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "softmax_hand_example.json")))
    q = np.array(g["q"])[:, None, :]
    k = np.array(g["k"])[:, None, :]
    v = np.array(g["v"])[:, None, :]
    o, lse = oracle.attention(q, k, v, np.array(g["q_pos"]), 1.0)
    np.testing.assert_allclose(o[:, 0, :], np.array(g["o"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[:, 0], np.array(g["lse"]), rtol=0, atol=1e-14)
    p = oracle.attention_probs(q, k, np.array(g["q_pos"]), 1.0)
    np.testing.assert_allclose(p[0, 0], g["p_row0"], atol=1e-15)
    # split of the keys into {0} and {1, 2}, merged by log-sum-exp
    qa = q[:1]
    oa, la = oracle.attention(qa, k[:1], v[:1], np.array([2]), 1.0)
    ob, lb = oracle.attention(qa, k[1:], v[1:], np.array([1]), 1.0)
    np.testing.assert_allclose(lb[0, 0], g["split_B_lse"], atol=1e-14)
    om, lm = oracle.lse_merge([(oa, la), (ob, lb)])
    np.testing.assert_allclose(om[0, 0], g["o"][0], atol=1e-13)
    np.testing.assert_allclose(lm[0, 0], g["lse"][0], atol=1e-14)


@pytest.mark.parametrize("Hq,Hkv,L,n,d", [(2, 2, 7, 3, 4), (4, 2, 23, 5, 8), (4, 1, 40, 4, 3)])
def test_brute_force_tiny(Hq, Hkv, L, n, d):
    rng = np.random.default_rng(100 + L)
    q = rng.standard_normal((n, Hq, d))
    k = rng.standard_normal((L, Hkv, d))
    v = rng.standard_normal((L, Hkv, d + 1))
    q_pos = np.sort(rng.integers(0, L, n))
    scale = 1 / math.sqrt(d)
    o, lse = oracle.attention(q, k, v, q_pos, scale)
    ob, lb = _brute(q, k, v, q_pos, scale)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=1e-12, atol=1e-13)


def test_probability_rows_sum_to_one_and_mask_exact():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((6, 4, 16)) * 3
    k = rng.standard_normal((50, 2, 16))
    q_pos = np.array([0, 3, 17, 30, 48, 49])
    p = oracle.attention_probs(q, k, q_pos, 0.25)
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-12)
    for i, pos in enumerate(q_pos):
        assert np.all(p[i, :, pos + 1:] == 0.0)
        assert np.all(p[i, :, :pos + 1] > 0.0)


def test_closed_forms():
    rng = np.random.default_rng(8)
    L, d = 33, 8
    k = rng.standard_normal((L, 1, d))
    v = rng.standard_normal((L, 1, d))
    # q = 0: uniform weights -> mean of the visible V
    pos = np.array([0, 9, 32])
    o, lse = oracle.attention(np.zeros((3, 1, d)), k, v, pos, 1.0)
    for i, p in enumerate(pos):
        np.testing.assert_allclose(o[i, 0], v[:p + 1, 0].mean(0), atol=1e-14)
        np.testing.assert_allclose(lse[i, 0], math.log(p + 1), atol=1e-14)
    # context of one key: o = V_0 exactly
    o, _ = oracle.attention(rng.standard_normal((1, 1, d)), k[:1], v[:1], np.array([0]), 1.0)
    assert np.array_equal(o[0, 0], v[0, 0])
    # one key 50 above all others: o = that V to 1e-12
    kk = np.zeros((L, 1, d))
    kk[11, 0, 0] = 50.0
    qq = np.zeros((1, 1, d))
    qq[0, 0, 0] = 1.0
    o, _ = oracle.attention(qq, kk, v, np.array([L - 1]), 1.0)
    np.testing.assert_allclose(o[0, 0], v[11, 0], atol=1e-12 * (1 + np.abs(v).max()) * L)


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(9)
    Hq, Hkv, L, n, d = 8, 2, 45, 5, 16
    q = rng.standard_normal((n, Hq, d))
    k = rng.standard_normal((L, Hkv, d))
    v = rng.standard_normal((L, Hkv, d))
    pos = np.array([10, 20, 30, 40, 44])
    o1, l1 = oracle.attention(q, k, v, pos, 0.3)
    o2, l2 = oracle.attention(q, np.repeat(k, Hq // Hkv, 1), np.repeat(v, Hq // Hkv, 1), pos, 0.3)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)
    # and a query head really reads KV head h // G: changing KV head 1 leaves heads 0..3 fixed
    k2 = k.copy()
    k2[:, 1] += rng.standard_normal((L, d))
    o3, _ = oracle.attention(q, k2, v, pos, 0.3)
    assert np.array_equal(o3[:, :4], o1[:, :4])
    assert not np.allclose(o3[:, 4:], o1[:, 4:])


def test_paging_permutation_is_bit_identical():
    """The block pool is an indirection only: any placement gives identical results."""
    lengths = [37, 100, 16]
    kw = dict(lengths=lengths, n_new=[5, 1, 16], num_q_heads=4, num_kv_heads=2, head_dim=8)
    a = W.make_gqa(11, place_seed=101, **kw)
    b = W.make_gqa(11, place_seed=202, **kw)
    assert not np.array_equal(a.block_table, b.block_table)
    for s in range(3):
        oa, la = oracle.paged_gqa_attention(a, s)
        ob, lb = oracle.paged_gqa_attention(b, s)
        assert np.array_equal(oa, ob) and np.array_equal(la, lb)
        k, v = a.kv_contiguous(s)
        oc, lc = oracle.attention(oracle.bf16_to_f64(a.q_rows(s)), oracle.bf16_to_f64(k),
                                  oracle.bf16_to_f64(v), a.q_pos(s), a.scale)
        assert np.array_equal(oa, oc) and np.array_equal(la, lc)


def test_gather_reads_only_referenced_blocks():
    """Unreferenced pool blocks are NaN; the oracle's gather never touches them."""
    wl = W.make_prefill_tiny()
    o, lse = oracle.paged_gqa_attention(wl, 0)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    assert np.isnan(oracle.bf16_to_f64(wl.k_pool)).sum() == 48 * 8 * 16 * 64


@pytest.mark.parametrize("cuts", [[5], [1, 2, 40], [16, 32, 48], [63]])
def test_lse_merge_identity(cuts):
    rng = np.random.default_rng(10)
    L, d = 64, 8
    q = rng.standard_normal((3, 2, d))
    k = rng.standard_normal((L, 1, d))
    v = rng.standard_normal((L, 1, d))
    pos = np.array([L - 1, L - 1, L - 1])
    full = oracle.attention(q, k, v, pos, 0.5)
    edges = [0] + cuts + [L]
    parts = [oracle.attention(q, k[a:b], v[a:b], pos - a, 0.5) for a, b in zip(edges, edges[1:])]
    om, lm = oracle.lse_merge(parts)
    np.testing.assert_allclose(om, full[0], atol=1e-13)
    np.testing.assert_allclose(lm, full[1], atol=1e-13)


def test_lse_merge_with_empty_part():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((2, 1, 4))
    k = rng.standard_normal((10, 1, 4))
    v = rng.standard_normal((10, 1, 4))
    pos = np.array([3, 9])
    full = oracle.attention(q, k, v, pos, 1.0)
    # second part covers keys 5..9: empty for the query at position 3
    parts = [oracle.attention(q, k[:5], v[:5], pos, 1.0), oracle.attention(q, k[5:], v[5:], pos - 5, 1.0)]
    assert parts[1][1][0, 0] == -np.inf
    om, lm = oracle.lse_merge(parts)
    np.testing.assert_allclose(om, full[0], atol=1e-13)
    np.testing.assert_allclose(lm, full[1], atol=1e-13)
