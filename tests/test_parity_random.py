"""GPU parity over randomly drawn shapes (seeded): batch sizes, query tokens per sequence,
head counts, head dims, context lengths from 1 token up, sharing patterns and selection
sizes, each case checked row by row against the fp64 oracle.  The fixed-shape tests cover
the workloads' own shapes and named edge cases; these cover the combinations between them.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from workloads.device import GqaOnDevice, MlaOnDevice
from gpu_util import BF16_L1, BF16_MAX_ABS, FP8_L1, FP8_MAX_ABS, LSE_ABS, assert_close, bf16_out

pytestmark = pytest.mark.gpu


def _lengths(rng, n, lo, hi):
    """n lengths, log-uniform in [lo, hi], with the smallest allowed one mixed in."""
    L = np.floor(np.exp(rng.uniform(np.log(lo), np.log(hi + 1), n))).astype(np.int64)
    L[rng.random(n) < 0.15] = lo
    return np.clip(L, lo, hi)


@pytest.mark.parametrize("seed", range(30))
def test_random_gqa_decode(pa_lib, seed):
    import torch
    rng = np.random.default_rng(500 + seed)
    T = int(rng.integers(1, 5))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([g for g in (1, 2, 4, 8) if T * g <= 16]))
    D = int(rng.choice([64, 128]))
    n_groups = int(rng.integers(1, 8))
    # sharing groups of random sizes; members of a group share a length and a prefix
    sizes = rng.integers(1, 6, n_groups)
    glen = _lengths(rng, n_groups, T, 3000)
    lengths, groups, s = [], [], 0
    for sz, L in zip(sizes, glen):
        groups.append(list(range(s, s + int(sz))))
        lengths += [int(L)] * int(sz)
        s += int(sz)
    S = len(lengths)
    perm = rng.permutation(S)                       # members need not be adjacent in the batch
    inv = np.argsort(perm)
    lengths = [lengths[perm[i]] for i in range(S)]
    groups = [[int(inv[m]) for m in g] for g in groups]
    frac = float(rng.choice([0.0, 0.5, 0.9]))
    wl = W.make_gqa(600 + seed, lengths=lengths, n_new=[T] * S, num_q_heads=Hkv * G, num_kv_heads=Hkv,
                    head_dim=D, shared_groups=groups, shared_frac=frac)
    dev = GqaOnDevice(wl)
    H = wl.num_q_heads
    lse = torch.empty((S, T, H), dtype=torch.float32, device="cuda")
    out = pa_lib.paged_attn_decode(dev.q.view(S, T, H, D), dev.pool, dev.bt, dev.total_len, q_per_seq=T,
                                   num_q_heads=H, max_context_len=dev.max_total, scale=wl.scale, lse=lse)
    torch.cuda.synchronize()
    got = bf16_out(out).reshape(S * T, H, D)
    lg = lse.cpu().numpy().reshape(S * T, H)
    what = f"seed={seed} S={S} T={T} Hkv={Hkv} G={G} D={D} share={frac}"
    for s in range(S):
        ro, rl = oracle.paged_gqa_attention(wl, s)
        assert_close(got[s * T:(s + 1) * T], ro, BF16_MAX_ABS, BF16_L1, f"decode {what} seq={s} L={lengths[s]}")
        np.testing.assert_allclose(lg[s * T:(s + 1) * T], rl, atol=LSE_ABS)


@pytest.mark.parametrize("seed", range(20))
def test_random_gqa_prefill(pa_lib, seed):
    import torch
    rng = np.random.default_rng(700 + seed)
    S = int(rng.integers(1, 6))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    D = int(rng.choice([64, 128]))
    cached = [int(x) for x in rng.integers(0, 2500, S)]
    new = [int(x) for x in _lengths(rng, S, 1, 400)]
    lengths = [c + n for c, n in zip(cached, new)]
    wl = W.make_gqa(800 + seed, lengths=lengths, n_new=new, num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim=D)
    dev = GqaOnDevice(wl)
    H = wl.num_q_heads
    lse = torch.empty((wl.q.shape[0], H), dtype=torch.float32, device="cuda")
    out = pa_lib.paged_attn_prefill(dev.q, dev.pool, dev.bt, dev.cached, dev.n_new, dev.q_start, num_q_heads=H,
                                    max_new_len=dev.max_new, max_total_len=dev.max_total, scale=wl.scale, lse=lse)
    torch.cuda.synchronize()
    got = bf16_out(out)
    lg = lse.cpu().numpy()
    what = f"seed={seed} S={S} Hkv={Hkv} G={G} D={D}"
    for s in range(S):
        ro, rl = oracle.paged_gqa_attention(wl, s)
        a, b = wl.q_start[s], wl.q_start[s + 1]
        assert_close(got[a:b], ro, BF16_MAX_ABS, BF16_L1, f"prefill {what} seq={s} cached={cached[s]} new={new[s]}")
        np.testing.assert_allclose(lg[a:b], rl, atol=LSE_ABS)


@pytest.mark.parametrize("seed", range(12))
def test_random_mla_decode(pa_lib, seed):
    import torch
    rng = np.random.default_rng(900 + seed)
    T = int(rng.integers(1, 5))
    Hq = int(rng.choice([16, 32, 64, 128]))
    S = int(rng.integers(1, 5))
    lengths = _lengths(rng, S, T, 12000)
    mla = W.make_mla_decode(950 + seed, lengths=lengths, q_per_seq=T, num_q_heads=Hq)
    dev = MlaOnDevice(mla)
    q = dev.q.view(S, T, Hq, 576)
    lse = torch.empty((S, T, Hq), dtype=torch.float32, device="cuda")
    out = pa_lib.paged_attn_decode(q, dev.pool, dev.bt, dev.total_len, q_per_seq=T, num_q_heads=Hq,
                                   max_context_len=dev.max_total, scale=mla.scale, lse=lse)
    torch.cuda.synchronize()
    got = bf16_out(out).reshape(S * T, Hq, 512)
    lg = lse.cpu().numpy().reshape(S * T, Hq)
    for s in range(S):
        L = int(mla.total_len[s])
        codes = oracle.gather_paged(mla.kv_pool, mla.block_table[s], L)
        sc = oracle.gather_paged(mla.kv_scale[..., None], mla.block_table[s], L)[:, 0]
        ro, rl = oracle.mla_attention(mla.q_rows(s), codes, sc, mla.q_pos(s), mla.scale)
        assert_close(got[s * T:(s + 1) * T], ro, FP8_MAX_ABS, FP8_L1, f"mla seed={seed} T={T} Hq={Hq} L={L}")
        np.testing.assert_allclose(lg[s * T:(s + 1) * T], rl, atol=LSE_ABS)


@pytest.mark.parametrize("seed", range(12))
def test_random_sparse_mla(pa_lib, seed):
    import torch
    rng = np.random.default_rng(1100 + seed)
    Hq = int(rng.choice([16, 32, 64, 128]))
    n = int(rng.integers(1, 20))
    k = int(rng.choice([1, 37, 256, 2048, 2100]))
    cached = int(rng.integers(0, 4000))
    mla, idx = W.make_sparse_mla(1150 + seed, lengths=[cached + n], n_new=[n], num_q_heads=Hq)
    dev = MlaOnDevice(mla, idx)
    pos = mla.q_pos(0)
    tk = np.full((n, k), -1, np.int32)
    for r in range(n):
        m = min(k, int(pos[r]) + 1)
        m -= int(rng.integers(0, min(m, 5) + 1))     # a few holes, possibly every slot
        tk[r, :m] = rng.choice(int(pos[r]) + 1, size=m, replace=False)
        tk[r] = rng.permutation(tk[r])
    out = pa_lib.sparse_mla_attn(dev.q, dev.pool, dev.bt, dev.q_seq, torch.from_numpy(tk).cuda(), scale=mla.scale)
    torch.cuda.synchronize()
    L = int(mla.total_len[0])
    codes = oracle.gather_paged(mla.kv_pool, mla.block_table[0], L)
    sc = oracle.gather_paged(mla.kv_scale[..., None], mla.block_table[0], L)[:, 0]
    ro, _ = oracle.sparse_mla_attention(mla.q[0:n], codes, sc, tk, mla.scale)
    assert_close(bf16_out(out), ro, FP8_MAX_ABS, FP8_L1, f"sparse seed={seed} Hq={Hq} n={n} k={k} L={L}")


@pytest.mark.parametrize("seed", range(12))
def test_random_indexer_topk(pa_lib, seed):
    """Indexer scores against the oracle (relative bound as in the fixed-shape test) and the
    top-k index sets bit-exact against the oracle's top-k on the kernel's own scores, for a
    random batch of sequences, head counts and k (including k above some rows' counts)."""
    import torch
    rng = np.random.default_rng(1300 + seed)
    S = int(rng.integers(1, 4))
    H = int(rng.choice([16, 32, 48, 64]))
    k = int(rng.choice([1, 33, 256, 2048]))
    n_new = [int(x) for x in _lengths(rng, S, 1, 60)]
    cached = [int(x) for x in rng.integers(0, 9000, S)]
    lengths = [c + n for c, n in zip(cached, n_new)]
    mla, idx = W.make_sparse_mla(1350 + seed, lengths=lengths, n_new=n_new, num_q_heads=16, idx_heads=H)
    dev = MlaOnDevice(mla, idx)
    n_q = dev.q_idx.shape[0]
    scores = torch.empty((n_q, dev.max_total), dtype=torch.float32, device="cuda")
    topk = pa_lib.mla_indexer_topk(dev.q_idx, dev.w, dev.idx_pool, dev.bt, dev.cached, dev.n_new, dev.q_start,
                                   max_new_len=dev.max_new, max_total_len=dev.max_total, k=k, scores_out=scores)
    torch.cuda.synchronize()
    topk = topk.cpu().numpy()
    sc = scores.cpu().numpy().astype(np.float64)
    for s in range(S):
        L = int(mla.total_len[s])
        kc = oracle.gather_paged(idx.idx_pool, mla.block_table[s], L)
        ks = oracle.gather_paged(idx.idx_scale[..., None], mla.block_table[s], L)[:, 0]
        a, b = mla.q_start[s], mla.q_start[s + 1]
        pos = mla.q_pos(s)
        ref = oracle.indexer_scores(idx.q_idx[a:b], idx.w[a:b], kc, ks, pos)
        got = sc[a:b, :L]
        fin = np.isfinite(ref)
        assert np.array_equal(fin, np.isfinite(got)), (seed, s)
        err = np.abs(got[fin] - ref[fin])
        assert err.max() <= 2e-3 * np.abs(ref[fin]).max(), (seed, s, err.max())
        for r in range(b - a):
            assert np.array_equal(topk[a + r], oracle.topk_indices(got[r], pos[r] + 1, k)), (seed, s, r)
