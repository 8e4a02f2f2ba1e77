"""GPU parity: FP8-latent MLA decode (MTP), indexer scores + top-k, sparse MLA.

The oracle dequantises the same FP8 bytes the kernels read.  Top-k index sets are
compared bit-exactly against the oracle's top-k run on the GPU's own scores (identical
scores); against the oracle's fp64 scores only near-ties at the k-th score may differ.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from workloads.device import MlaOnDevice
from gpu_util import FP8_L1, FP8_MAX_ABS, LSE_ABS, assert_close, assert_close_stress, bf16_out

pytestmark = pytest.mark.gpu


def _mla_decode(pa, dev, T):
    import torch
    mla = dev.mla
    S = mla.num_seqs
    q = dev.q.view(S, T, mla.num_q_heads, 576)
    lse = torch.empty((S, T, mla.num_q_heads), dtype=torch.float32, device="cuda")
    out = pa.paged_attn_decode(q, dev.pool, dev.bt, dev.total_len, q_per_seq=T, num_q_heads=mla.num_q_heads,
                               max_context_len=dev.max_total, scale=mla.scale, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def _mla_ref(mla, s):
    L = int(mla.total_len[s])
    codes = oracle.gather_paged(mla.kv_pool, mla.block_table[s], L)
    sc = oracle.gather_paged(mla.kv_scale[..., None], mla.block_table[s], L)[:, 0]
    return oracle.mla_attention(mla.q_rows(s), codes, sc, mla.q_pos(s), mla.scale), codes, sc


def test_gather_fp8_bit_exact(pa_lib):
    import torch
    mla = W.make_mla_decode(71, lengths=[130, 64, 5], num_q_heads=16, keep_content=True)
    dev = MlaOnDevice(mla)
    for s in range(3):
        L = int(mla.total_len[s])
        k = torch.empty((L, 576), dtype=torch.uint8, device="cuda")
        sc = torch.empty((L,), dtype=torch.float32, device="cuda")
        pa_lib.pa_test_gather_kv(dev.pool, dev.bt, s, L, k, None, sc)
        torch.cuda.synchronize()
        c, cs = mla.kv_contiguous(s)
        assert np.array_equal(k.cpu().numpy(), c) and np.array_equal(sc.cpu().numpy(), cs)


@pytest.mark.parametrize("T,Hq", [(4, 64), (1, 64), (4, 16), (2, 32), (3, 128), (1, 16)])
def test_mla_decode(pa_lib, T, Hq):
    lengths = [T, 63, 64, 65, 3000, 8192 + 100, 17000]
    mla = W.make_mla_decode(72 + T, lengths=lengths, q_per_seq=T, num_q_heads=Hq)
    dev = MlaOnDevice(mla)
    out, lse = _mla_decode(pa_lib, dev, T)
    got = bf16_out(out).reshape(len(lengths) * T, Hq, 512)
    lg = lse.cpu().numpy().reshape(len(lengths) * T, Hq)
    for s in range(len(lengths)):
        (ro, rl), _, _ = _mla_ref(mla, s)
        assert_close(got[s * T:(s + 1) * T], ro, FP8_MAX_ABS, FP8_L1, f"mla T={T} Hq={Hq} L={lengths[s]}")
        np.testing.assert_allclose(lg[s * T:(s + 1) * T], rl, atol=LSE_ABS)
    # splits merged in a fixed order: a rerun is bit-identical
    out2, lse2 = _mla_decode(pa_lib, dev, T)
    assert bf16_out(out2).tobytes() == bf16_out(out).tobytes() and np.array_equal(lse2.cpu().numpy(), lse.cpu().numpy())


def test_mla_decode_peaked(pa_lib):
    mla = W.make_mla_decode(79, lengths=[5000, 20000], q_per_seq=4, num_q_heads=64, q_mult=8.0)
    dev = MlaOnDevice(mla)
    out, _ = _mla_decode(pa_lib, dev, 4)
    got = bf16_out(out).reshape(8, 64, 512)
    for s in range(2):
        (ro, _), _, _ = _mla_ref(mla, s)
        assert_close_stress(got[s * 4:(s + 1) * 4], ro, FP8_MAX_ABS, FP8_L1, f"mla peaked s={s}")


def test_topk_hook_ties_and_short_rows(pa_lib):
    import torch
    scores = W.tie_scores(3, 12, 5000)
    valid = np.array([5000, 4999, 2048, 2047, 100, 1, 4096, 3000, 2049, 5000, 777, 4500], np.int32)
    scores[1, 7] = -0.0
    scores[1, 9] = 0.0
    st = torch.from_numpy(scores).cuda()
    vt = torch.from_numpy(valid).cuda()
    for k in (2048, 1, 100):
        got = pa_lib.pa_test_topk_from_scores(st, vt, k).cpu().numpy()
        for r in range(12):
            ref = oracle.topk_indices(scores[r].astype(np.float64), valid[r], k)
            assert np.array_equal(got[r], ref), (k, r)


def test_topk_hook_random_scores(pa_lib):
    import torch
    rng = np.random.default_rng(5)
    scores = rng.standard_normal((16, 20000)).astype(np.float32)
    scores[3, :5000] = scores[3, 0]          # a long run of equal values
    valid = rng.integers(1, 20001, 16).astype(np.int32)
    valid[:4] = 20000
    got = pa_lib.pa_test_topk_from_scores(torch.from_numpy(scores).cuda(), torch.from_numpy(valid).cuda(),
                                          2048).cpu().numpy()
    for r in range(16):
        assert np.array_equal(got[r], oracle.topk_indices(scores[r].astype(np.float64), valid[r], 2048)), r


def test_topk_hook_long_and_clustered_rows(pa_lib):
    """Rows beyond the LDS bitmap (300,000 tokens) and rows whose scores crowd one
    histogram bin (all within a factor 1.001) take the multi-pass path; both must match."""
    import torch
    rng = np.random.default_rng(6)
    n = 300_000
    scores = np.empty((3, n), np.float32)
    scores[0] = rng.standard_normal(n)
    scores[1] = 1.0 + 1e-3 * rng.random(n)               # one 12-bit key bin holds everything
    scores[2] = rng.standard_normal(n)
    valid = np.array([n, 200_000, 150_000], np.int32)
    got = pa_lib.pa_test_topk_from_scores(torch.from_numpy(scores).cuda(), torch.from_numpy(valid).cuda(),
                                          2048).cpu().numpy()
    for r in range(3):
        assert np.array_equal(got[r], oracle.topk_indices(scores[r].astype(np.float64), valid[r], 2048)), r


def _sample_runs(valid):
    """Where the top-k kernel samples a row for its threshold: 8 runs of 512 scores, run w
    starting at w * (valid - 512) // 7 rounded down to a multiple of 4."""
    return [((w * (valid - 512)) // 7) & ~3 for w in range(8)]


def test_topk_hook_one_read_and_its_fallbacks(pa_lib):
    """Rows long enough for the one-read path: plain rows, rows whose sampled runs mislead
    the threshold both ways (too few keys reach it, too many), ties at the k-th key with
    more copies than are taken (also +0.0 against -0.0), rows at the length limit of the
    path and beside it, k above the path's limit, and rows that are not 16-byte aligned."""
    import torch
    rng = np.random.default_rng(7)
    n = 150_000
    rows = []
    rows.append(rng.standard_normal(n))                                   # plain
    r = rng.standard_normal(n)                                            # runs high: too few
    for a in _sample_runs(n):
        r[a:a + 512] = 10.0 + rng.standard_normal(512)
    rows.append(r)
    r = 10.0 + rng.standard_normal(n)                                     # runs low: too many
    for a in _sample_runs(n):
        r[a:a + 512] = rng.standard_normal(512)
    rows.append(r)
    r = rng.standard_normal(n)                                            # 2,000 ties, 1,548 taken
    pos = rng.permutation(n)
    r[pos[:500]] = 100.0 + np.arange(500)
    r[pos[500:2500]] = 50.0
    rows.append(r)
    r = rng.standard_normal(n) - 5.0                                      # +-0 ties
    z = rng.permutation(40_000)[:3000]
    r[z] = np.where(rng.random(3000) < 0.5, -0.0, 0.0)
    rows.append(r)
    rows.append(np.round(rng.standard_normal(n) * 4) / 4)                 # few levels: bins crowd
    scores = np.stack(rows).astype(np.float32)
    valid = np.array([n, n, n, n, 40_000, n], np.int32)
    for k in (2048, 1, 100, 2049):
        got = pa_lib.pa_test_topk_from_scores(torch.from_numpy(scores).cuda(), torch.from_numpy(valid).cuda(),
                                              k).cpu().numpy()
        for i in range(len(rows)):
            assert np.array_equal(got[i], oracle.topk_indices(scores[i].astype(np.float64), valid[i], k)), (k, i)
    # lengths at the path's limit (32,768) and one below it; an odd row stride leaves rows
    # unaligned, so the loads are scalar
    sc = rng.standard_normal((4, 40_001)).astype(np.float32)
    vl = np.array([32_768, 32_767, 40_001, 32_769], np.int32)
    got = pa_lib.pa_test_topk_from_scores(torch.from_numpy(sc).cuda(), torch.from_numpy(vl).cuda(), 2048).cpu().numpy()
    for i in range(4):
        assert np.array_equal(got[i], oracle.topk_indices(sc[i].astype(np.float64), vl[i], 2048)), ("odd", i)


def _indexer(pa, dev, k):
    import torch
    n_q = dev.q_idx.shape[0]
    scores = torch.empty((n_q, dev.max_total), dtype=torch.float32, device="cuda")
    topk = pa.mla_indexer_topk(dev.q_idx, dev.w, dev.idx_pool, dev.bt, dev.cached, dev.n_new, dev.q_start,
                               max_new_len=dev.max_new, max_total_len=dev.max_total, k=k, scores_out=scores)
    torch.cuda.synchronize()
    return topk, scores


def _idx_keys(mla, idx, s):
    L = int(mla.total_len[s])
    kc = oracle.gather_paged(idx.idx_pool, mla.block_table[s], L)
    ks = oracle.gather_paged(idx.idx_scale[..., None], mla.block_table[s], L)[:, 0]
    return kc, ks


@pytest.mark.parametrize("H", [64, 32])
def test_indexer_topk(pa_lib, H):
    lengths, n_new = [300 + 37, 5000 + 100, 70], [37, 100, 70]
    mla, idx = W.make_sparse_mla(81, lengths=lengths, n_new=n_new, num_q_heads=64, idx_heads=H)
    dev = MlaOnDevice(mla, idx)
    k = 256
    topk, scores = _indexer(pa_lib, dev, k)
    topk = topk.cpu().numpy()
    sc = scores.cpu().numpy().astype(np.float64)
    for s in range(3):
        kc, ks = _idx_keys(mla, idx, s)
        a, b = mla.q_start[s], mla.q_start[s + 1]
        pos = mla.q_pos(s)
        ref = oracle.indexer_scores(idx.q_idx[a:b], idx.w[a:b], kc, ks, pos)
        L = int(mla.total_len[s])
        got = sc[a:b, :L]
        fin = np.isfinite(ref)
        assert np.array_equal(fin, np.isfinite(got))
        assert np.all(sc[a:b, L:] == -np.inf)
        err = np.abs(got[fin] - ref[fin])
        scale_ref = np.abs(ref[fin]).max()
        print(f"indexer H={H} seq={s}: max_abs={err.max():.3e} (ref max {scale_ref:.2f})")
        assert err.max() <= 2e-3 * scale_ref
        for r in range(b - a):
            exact = oracle.topk_indices(got[r], pos[r] + 1, k)
            assert np.array_equal(topk[a + r], exact), (s, r)
            # against the oracle's own scores: any difference is a near-tie at the k-th score
            oref = oracle.topk_indices(ref[r], pos[r] + 1, k)
            diff = np.setxor1d(oref[oref >= 0], topk[a + r][topk[a + r] >= 0])
            if diff.size:
                kth = np.sort(ref[r][:pos[r] + 1])[::-1][min(k, pos[r] + 1) - 1]
                assert np.all(np.abs(ref[r][diff] - kth) <= 2 * err.max() + 1e-12)


def test_sparse_mla(pa_lib):
    import torch
    lengths, n_new = [3000 + 50, 700 + 20], [50, 20]
    mla, idx = W.make_sparse_mla(91, lengths=lengths, n_new=n_new, num_q_heads=64)
    dev = MlaOnDevice(mla, idx)
    k = 512
    topk, _ = _indexer(pa_lib, dev, k)
    out = pa_lib.sparse_mla_attn(dev.q, dev.pool, dev.bt, dev.q_seq, topk, scale=mla.scale)
    torch.cuda.synchronize()
    got = bf16_out(out)
    tk = topk.cpu().numpy()
    for s in range(2):
        L = int(mla.total_len[s])
        codes = oracle.gather_paged(mla.kv_pool, mla.block_table[s], L)
        sc = oracle.gather_paged(mla.kv_scale[..., None], mla.block_table[s], L)[:, 0]
        a, b = mla.q_start[s], mla.q_start[s + 1]
        ro, _ = oracle.sparse_mla_attention(mla.q[a:b], codes, sc, tk[a:b], mla.scale)
        assert_close(got[a:b], ro, FP8_MAX_ABS, FP8_L1, f"sparse seq={s}")


def test_sparse_mla_k_covers_context_equals_dense(pa_lib):
    """k >= context: the sparse path must reproduce dense MLA (GLM-5.3 report, 'How to try')."""
    import torch
    mla, idx = W.make_sparse_mla(92, lengths=[300], n_new=[40], num_q_heads=64)
    dev = MlaOnDevice(mla, idx)
    topk, _ = _indexer(pa_lib, dev, 512)
    tk = topk.cpu().numpy()
    pos = mla.q_pos(0)
    for r in range(40):
        assert np.array_equal(tk[r][:pos[r] + 1], np.arange(pos[r] + 1)) and np.all(tk[r][pos[r] + 1:] == -1)
    out = pa_lib.sparse_mla_attn(dev.q, dev.pool, dev.bt, dev.q_seq, topk, scale=mla.scale)
    torch.cuda.synchronize()
    (ro, _), _, _ = _mla_ref(mla, 0)
    assert_close(bf16_out(out), ro, FP8_MAX_ABS, FP8_L1, "sparse == dense")


@pytest.mark.parametrize("k,Hq", [(100, 64), (2500, 64), (300, 16), (300, 128)])
def test_sparse_mla_given_selection(pa_lib, k, Hq):
    """Selections handed in directly, in random order with -1 holes: k <= 2,048 takes the
    path with the selections' rows staged in LDS, k > 2,048 the one that resolves each
    tile's rows from global memory; 16 heads leave half of each wave's rows empty, 128
    heads take two workgroups per query.  A row with no selection at all gives zeros."""
    import torch
    n = 24
    mla, idx = W.make_sparse_mla(93, lengths=[3000 + n], n_new=[n], num_q_heads=Hq)
    dev = MlaOnDevice(mla, idx)
    rng = np.random.default_rng(1000 + k)
    pos = mla.q_pos(0)
    tk = np.full((n, k), -1, np.int32)
    for r in range(n - 1):                      # the last row keeps no selection
        m = min(k, int(pos[r]) + 1) - int(rng.integers(0, 7))
        tk[r, :m] = rng.choice(int(pos[r]) + 1, size=m, replace=False)
        tk[r] = rng.permutation(tk[r])          # holes anywhere
    topk = torch.from_numpy(tk).cuda()
    out = pa_lib.sparse_mla_attn(dev.q, dev.pool, dev.bt, dev.q_seq, topk, scale=mla.scale)
    torch.cuda.synchronize()
    got = bf16_out(out)
    L = int(mla.total_len[0])
    codes = oracle.gather_paged(mla.kv_pool, mla.block_table[0], L)
    sc = oracle.gather_paged(mla.kv_scale[..., None], mla.block_table[0], L)[:, 0]
    ro, _ = oracle.sparse_mla_attention(mla.q[0:n], codes, sc, tk, mla.scale)
    assert_close(got, ro, FP8_MAX_ABS, FP8_L1, f"sparse given selection k={k} Hq={Hq}")
    assert np.all(got[n - 1] == 0)


@pytest.mark.parametrize("num_blocks", [262143, 262144])
def test_sparse_mla_rows_near_2_24(pa_lib, num_blocks):
    """The staged path keeps each selection's physical row (block x 64 + slot) in 24 bits,
    0xffffff marking a hole: a pool of 262,143 blocks has rows up to 0xffffbf and is staged;
    one more block (rows up to 0xffffff) makes the call resolve the rows per tile from global
    memory instead.  The workload's blocks sit at the highest block ids of such a pool (every
    other id from the top; the rest of the pool is never read) and every row must match the
    oracle on the original layout."""
    import torch
    import paged_prefix_cached_amd as pa
    n, k, Hq = 8, 300, 64
    mla, idx = W.make_sparse_mla(95, lengths=[900 + n], n_new=[n], num_q_heads=Hq)
    dev = MlaOnDevice(mla, idx)
    L = int(mla.total_len[0])
    nlb = -(-L // 64)
    old_ids = mla.block_table[0, :nlb].astype(np.int64)
    new_ids = num_blocks - 1 - 2 * np.arange(nlb)
    kv = torch.empty((num_blocks, 64, 576), dtype=torch.uint8, device="cuda")
    ks = torch.empty((num_blocks, 64), dtype=torch.float32, device="cuda")
    dst = torch.from_numpy(new_ids).cuda()
    kv[dst] = torch.from_numpy(mla.kv_pool[old_ids]).cuda()
    ks[dst] = torch.from_numpy(mla.kv_scale[old_ids]).cuda()
    pool = pa.mla_pool(kv, ks)
    bt = mla.block_table.copy()
    bt[0, :nlb] = new_ids
    rng = np.random.default_rng(95)
    pos = mla.q_pos(0)
    tk = np.full((n, k), -1, np.int32)
    for r in range(n):
        m = min(k, int(pos[r]) + 1) - int(rng.integers(0, 7))
        tk[r, :m] = rng.choice(int(pos[r]) + 1, size=m, replace=False)
        tk[r] = rng.permutation(tk[r])
    out = pa_lib.sparse_mla_attn(dev.q, pool, torch.from_numpy(bt).cuda(), dev.q_seq, torch.from_numpy(tk).cuda(),
                                 scale=mla.scale)
    torch.cuda.synchronize()
    got = bf16_out(out)
    del kv, ks, pool
    torch.cuda.empty_cache()
    codes = oracle.gather_paged(mla.kv_pool, mla.block_table[0], L)
    sc = oracle.gather_paged(mla.kv_scale[..., None], mla.block_table[0], L)[:, 0]
    ro, _ = oracle.sparse_mla_attention(mla.q[0:n], codes, sc, tk, mla.scale)
    assert_close(got, ro, FP8_MAX_ABS, FP8_L1, f"sparse rows near 2^24, {num_blocks} blocks")


def _tile_overflow(scores_log2: np.ndarray, tile: int = 32, slack: float = 8.0) -> np.ndarray:
    """Per row of scores (log2 units, -inf = masked, in the kernel's key order): whether the
    MLA kernel's fixed reference (the row maximum of the first tile holding a visible key)
    is passed by more than `slack` by a later tile's maximum -- the case the kernel hands to
    its exact fallback."""
    n, L = scores_log2.shape
    pad = (-L) % tile
    s = np.concatenate([scores_log2, np.full((n, pad), -np.inf)], axis=1).reshape(n, -1, tile).max(axis=2)
    out = np.zeros(n, dtype=bool)
    for r in range(n):
        fin = np.flatnonzero(np.isfinite(s[r]))
        if fin.size:
            out[r] = bool(np.max(s[r][fin[0]:]) > s[r][fin[0]] + slack)
    return out


def test_mla_decode_fixed_reference_fallback(pa_lib):
    """Moderately peaked queries: in some work units (6,144 keys x 128 query rows) a row's
    maximum climbs far above its first tile's, so the fixed-reference kernel marks the unit
    and the exact kernel recomputes it; the other units stay on the fast path.  Both kinds
    are in this call and every row matches the oracle."""
    T, Hq = 4, 64
    lengths = [5000, 20000]
    mla = W.make_mla_decode(79, lengths=lengths, q_per_seq=T, num_q_heads=Hq, q_mult=1.8)
    n_over = n_units = 0
    for s in range(len(lengths)):
        L = lengths[s]
        codes = oracle.gather_paged(mla.kv_pool, mla.block_table[s], L)
        sc = oracle.gather_paged(mla.kv_scale[..., None], mla.block_table[s], L)[:, 0]
        k = oracle.mla_dequant(codes, sc)
        q = oracle.bf16_to_f64(mla.q_rows(s)).reshape(T * Hq, 576)
        pos = np.repeat(mla.q_pos(s), Hq)
        sl = (q @ k.T) * (mla.scale / np.log(2.0))
        sl[np.arange(L)[None, :] > pos[:, None]] = -np.inf
        for k0 in range(0, L, 6144):
            ov = _tile_overflow(sl[:, k0:k0 + 6144]).reshape(2, 128)    # two 128-row units
            n_units += 2
            n_over += int(ov.any(axis=1).sum())
    assert 0 < n_over < n_units, (n_over, n_units)
    dev = MlaOnDevice(mla)
    out, lse = _mla_decode(pa_lib, dev, T)
    got = bf16_out(out).reshape(len(lengths) * T, Hq, 512)
    lg = lse.cpu().numpy().reshape(len(lengths) * T, Hq)
    for s in range(len(lengths)):
        (ro, rl), _, _ = _mla_ref(mla, s)
        assert_close_stress(got[s * T:(s + 1) * T], ro, FP8_MAX_ABS, FP8_L1, f"mla fallback s={s}")
        np.testing.assert_allclose(lg[s * T:(s + 1) * T], rl, atol=LSE_ABS)


@pytest.mark.parametrize("Hq", [64, 32, 128])
def test_sparse_mla_fixed_reference_fallback(pa_lib, Hq):
    """Sparse MLA with peaked queries: even query rows list their selections by ascending
    score (later tiles' maxima can pass the first tile's by more than 2^8: the exact
    fallback recomputes those workgroups), odd rows in random order.  The result does not depend on
    the order; every row matches the oracle, for 32, 64 and 128 heads."""
    import torch
    n, k = 16, 300
    qm = 2.4 if Hq == 32 else 2.0          # fewer heads per row: a larger spread to overflow
    mla, idx = W.make_sparse_mla(94, lengths=[2000 + n], n_new=[n], num_q_heads=Hq, q_mult=qm)
    L = int(mla.total_len[0])
    codes = oracle.gather_paged(mla.kv_pool, mla.block_table[0], L)
    sc = oracle.gather_paged(mla.kv_scale[..., None], mla.block_table[0], L)[:, 0]
    kk = oracle.mla_dequant(codes, sc)
    rng = np.random.default_rng(94)
    pos = mla.q_pos(0)
    tk = np.full((n, k), -1, np.int32)
    over = []
    for r in range(n):
        sel = rng.choice(int(pos[r]) + 1, size=k, replace=False)
        s_row = (oracle.bf16_to_f64(mla.q[r]) @ kk[sel].T) * (mla.scale / np.log(2.0))     # [Hq][k]
        if r % 2 == 0:
            sel = sel[np.argsort(s_row.max(axis=0), kind="stable")]
            s_row = (oracle.bf16_to_f64(mla.q[r]) @ kk[sel].T) * (mla.scale / np.log(2.0))
        tk[r] = sel
        over.append(bool(_tile_overflow(s_row).any()))
    assert any(over) and not all(over), over        # both paths in one call
    dev = MlaOnDevice(mla, idx)
    out = pa_lib.sparse_mla_attn(dev.q, dev.pool, dev.bt, dev.q_seq, torch.from_numpy(tk).cuda(), scale=mla.scale)
    torch.cuda.synchronize()
    ro, _ = oracle.sparse_mla_attention(mla.q[0:n], codes, sc, tk, mla.scale)
    assert_close_stress(bf16_out(out), ro, FP8_MAX_ABS, FP8_L1, f"sparse fallback Hq={Hq}")
