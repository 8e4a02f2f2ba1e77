"""GPU parity for the packed per-block layout (one allocation per 64-token block: FP8
latent, its scales, MXFP4 index keys and their E8M0 scales): the block-table gather and
the append bit for bit against the oracle, the indexer on MXFP4 keys (scores against the
oracle, top-k bit-exact on the GPU's scores), and MLA decode / sparse MLA on the latent
view, whose outputs must equal the separate-pool layout's bit for bit (the same bytes)."""
import numpy as np
import pytest

import oracle
import workloads as W
from workloads.device import MlaOnDevice, t as to_dev
from gpu_util import FP8_L1, FP8_MAX_ABS, LSE_ABS, assert_close, bf16_out

pytestmark = pytest.mark.gpu


def _packed_dev(pa, mla, idx):
    blocks = to_dev(W.pack_mla_blocks(mla, idx), "cuda")
    lat, ix = pa.packed_mla_pools(blocks)
    return blocks, lat, ix


def test_packed_gather_bit_exact(pa_lib):
    import torch
    mla, idx = W.make_sparse_mla(111, lengths=[300, 64, 130], n_new=[3, 2, 1], num_q_heads=16, fp4_keys=True)
    dev = MlaOnDevice(mla, idx)
    blocks, lat, ix = _packed_dev(pa_lib, mla, idx)
    host = W.pack_mla_blocks(mla, idx)
    l_, ls, k_, ks = oracle.packed_fields(host)
    for s in range(3):
        L = int(mla.total_len[s])
        row = mla.block_table[s]
        k = torch.empty((L, 576), dtype=torch.uint8, device="cuda")
        sc = torch.empty((L,), dtype=torch.float32, device="cuda")
        pa_lib.pa_test_gather_kv(lat, dev.bt, s, L, k, None, sc)
        kk = torch.empty((L, 64), dtype=torch.uint8, device="cuda")
        ksc = torch.empty((L,), dtype=torch.float32, device="cuda")
        pa_lib.pa_test_gather_kv(ix, dev.bt, s, L, kk, None, ksc)
        torch.cuda.synchronize()
        assert np.array_equal(k.cpu().numpy(), oracle.gather_paged(l_, row, L))
        assert np.array_equal(sc.cpu().numpy().view(np.uint32), oracle.gather_paged(ls[..., None], row, L)[:, 0].view(np.uint32))
        assert np.array_equal(kk.cpu().numpy(), oracle.gather_paged(k_, row, L))
        assert np.array_equal(ksc.cpu().numpy().view(np.uint8).reshape(L, 4), oracle.gather_paged(ks, row, L))


def _fp4_sweep_rows(n_rows: int, seed: int):
    """Rows of 128 bf16 values with every E2M1 rounding boundary (0.25, 0.75, 1.25, 1.75,
    2.5, 3.5, 5) and its bf16 neighbours at scale 1 (each group holds 6.0), saturation
    past 6 X, tiny groups (scale clamp), all-zero groups, negative values rounding to -0."""
    rng = np.random.default_rng(seed)
    edges = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    eb = W.bf16_bits(edges).astype(np.int32)
    cand = np.concatenate([eb, eb + 1, eb - 1]).astype(np.uint16)
    vals = W.bf16_bits_to_f32(cand)
    rows = np.empty((n_rows, 128), np.float32)
    for r in range(n_rows):
        x = rng.choice(np.concatenate([vals, -vals]), 128).astype(np.float32)
        for g in range(4):
            x[32 * g + int(rng.integers(32))] = 6.0 if r % 2 == 0 else -6.0
        if r % 5 == 1:
            x[32:64] *= np.float32(1e-38)                 # a tiny group: clamped scale code
        if r % 5 == 2:
            x[64:96] = 0.0                                # an all-zero group
        if r % 5 == 3:
            x[96:128] = rng.standard_normal(32).astype(np.float32) * np.float32(7.5)   # saturation
        if r % 5 == 4:
            x[0:32] = -np.abs(rng.standard_normal(32).astype(np.float32)) * np.float32(1e-3)
            x[5] = 6.0                                    # negatives that round to -0
        rows[r] = x
    return W.bf16_bits(rows)


@pytest.mark.parametrize("part", ["latent", "keys"])
def test_packed_append_bit_exact(pa_lib, part):
    import torch
    D = 576 if part == "latent" else 128
    a = W.make_append(120 + D, cached=[0, 63, 64, 1000, 5], new=[4, 4, 130, 1, 0], block_size=64,
                      row_shape=(D,), with_v=False, row_mults=(1.0, 1e-30, 3e-3, 1e4, 0.25), zero_rows=2)
    k_new = a.k_new
    if part == "keys":                                  # the rounding sweep in the first rows
        sweep = _fp4_sweep_rows(60, 7)
        k_new = k_new.copy()
        k_new[:60] = sweep
    rng = np.random.default_rng(9)
    pool = rng.integers(0, 256, (a.num_blocks, oracle.PACKED_BLOCK_BYTES), dtype=np.uint8)
    bt = a.block_table.copy()
    bt[2, 1] = 1 << 20                                  # an out-of-range block id: not written
    blocks = to_dev(pool, "cuda")
    lat, ix = pa_lib.packed_mla_pools(blocks)
    print(f"packed append {part}: rows={k_new.shape[0]}", flush=True)
    pa_lib.paged_kv_append(lat if part == "latent" else ix, to_dev(bt, "cuda"), to_dev(a.cached_len, "cuda"),
                           to_dev(a.new_len, "cuda"), to_dev(a.q_start, "cuda"), to_dev(k_new, "cuda"),
                           max_new_len=int(a.new_len.max()))
    torch.cuda.synchronize()
    want = oracle.append_packed(pool, bt, a.cached_len, a.new_len, a.q_start, k_new, part)
    got = blocks.cpu().numpy()
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} bytes differ, first (block, byte) {bad[:4].tolist()}"
    assert not np.array_equal(got, pool)


def _indexer(pa, dev, pool, k, scores=True):
    import torch
    n_q = dev.q_idx.shape[0]
    sc = torch.empty((n_q, dev.max_total), dtype=torch.float32, device="cuda") if scores else None
    topk = pa.mla_indexer_topk(dev.q_idx, dev.w, pool, dev.bt, dev.cached, dev.n_new, dev.q_start,
                               max_new_len=dev.max_new, max_total_len=dev.max_total, k=k, scores_out=sc)
    torch.cuda.synchronize()
    return topk, sc


def _check_fp4_rows(mla, idx, s, rows, sc_rows, tk_rows, k, what):
    host = W.pack_mla_blocks(mla, idx)
    _, _, keys, kscales = oracle.packed_fields(host)
    L = int(mla.total_len[s])
    kp = oracle.gather_paged(keys, mla.block_table[s], L)
    ks = oracle.gather_paged(kscales, mla.block_table[s], L)
    pos = mla.q_pos(s)[rows - mla.q_start[s]]
    ref = oracle.indexer_scores_mxfp4(idx.q_idx[rows], idx.w[rows], kp, ks, pos)
    got = sc_rows[:, :L].astype(np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got)), what
    err = np.abs(got[fin] - ref[fin])
    scale_ref = np.abs(ref[fin]).max()
    print(f"{what}: FP4 indexer max_abs={err.max():.3e} (ref max {scale_ref:.2f})", flush=True)
    assert err.max() <= 2e-3 * scale_ref
    for r in range(len(rows)):
        assert np.array_equal(tk_rows[r], oracle.topk_indices(got[r], pos[r] + 1, k)), (what, int(rows[r]))


@pytest.mark.parametrize("H", [64, 16])
def test_packed_fp4_indexer_topk(pa_lib, H):
    lengths, n_new = [300 + 37, 9000 + 100, 70], [37, 100, 70]
    mla, idx = W.make_sparse_mla(112, lengths=lengths, n_new=n_new, num_q_heads=16, idx_heads=H, fp4_keys=True)
    dev = MlaOnDevice(mla, idx)
    blocks, lat, ix = _packed_dev(pa_lib, mla, idx)
    k = 512
    topk, sc = _indexer(pa_lib, dev, ix, k)
    tk, scn = topk.cpu().numpy(), sc.cpu().numpy()
    for s in range(3):
        rows = np.arange(mla.q_start[s], mla.q_start[s + 1])
        assert np.all(np.isneginf(scn[rows, int(mla.total_len[s]):]))
        _check_fp4_rows(mla, idx, s, rows, scn[rows], tk[rows], k, f"packed FP4 H={H} seq={s}")


def test_packed_latent_view_equals_separate_pools(pa_lib):
    """MLA MTP decode and sparse MLA read the same latent bytes through the packed view:
    the outputs and log-sum-exps equal the separate-pool layout's bit for bit, and match the
    oracle."""
    import torch
    mla, idx = W.make_sparse_mla(113, lengths=[3000 + 40, 700 + 4], n_new=[40, 4], num_q_heads=64, fp4_keys=True)
    dev = MlaOnDevice(mla, idx)
    blocks, lat, ix = _packed_dev(pa_lib, mla, idx)
    topk, _ = _indexer(pa_lib, dev, ix, 512, scores=False)
    outs = []
    for pool in (dev.pool, lat):
        lse = torch.empty((dev.q.shape[0], 64), dtype=torch.float32, device="cuda")
        o = pa_lib.sparse_mla_attn(dev.q, pool, dev.bt, dev.q_seq, topk, scale=mla.scale, lse=lse)
        torch.cuda.synchronize()
        outs.append((o.view(torch.int16).cpu().numpy(), lse.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))
    got = oracle.bf16_to_f64(outs[1][0].view(np.uint16))
    tk = topk.cpu().numpy()
    for s in range(2):
        L = int(mla.total_len[s])
        codes = oracle.gather_paged(mla.kv_pool, mla.block_table[s], L)
        cs = oracle.gather_paged(mla.kv_scale[..., None], mla.block_table[s], L)[:, 0]
        a, b = mla.q_start[s], mla.q_start[s + 1]
        ro, rl = oracle.sparse_mla_attention(mla.q[a:b], codes, cs, tk[a:b], mla.scale)
        assert_close(got[a:b], ro, FP8_MAX_ABS, FP8_L1, f"packed sparse seq={s}")
        np.testing.assert_allclose(outs[1][1][a:b], rl, atol=LSE_ABS)
    # MTP decode over the same sequences (4 query tokens each)
    mlad = W.make_mla_decode(114, lengths=[5000, 300, 4097], q_per_seq=4, num_q_heads=64)
    ddev = MlaOnDevice(mlad)
    fake_idx = W.IndexerInput(None, None, None, None,
                              fp4_pool=np.zeros(mlad.kv_pool.shape[:2] + (64,), np.uint8),
                              fp4_scale=np.full(mlad.kv_pool.shape[:2] + (4,), 127, np.uint8))
    dblocks = to_dev(W.pack_mla_blocks(mlad, fake_idx), "cuda")
    dlat, _ = pa_lib.packed_mla_pools(dblocks)
    res = []
    for pool in (ddev.pool, dlat):
        out = pa_lib.paged_attn_decode(ddev.q.view(3, 4, 64, 576), pool, ddev.bt, ddev.total_len, q_per_seq=4,
                                       num_q_heads=64, max_context_len=ddev.max_total, scale=mlad.scale)
        torch.cuda.synchronize()
        res.append(out.view(torch.int16).cpu().numpy())
    assert np.array_equal(res[0], res[1])
    got = oracle.bf16_to_f64(res[1].view(np.uint16)).reshape(12, 64, 512)
    for s in range(3):
        L = int(mlad.total_len[s])
        codes = oracle.gather_paged(mlad.kv_pool, mlad.block_table[s], L)
        cs = oracle.gather_paged(mlad.kv_scale[..., None], mlad.block_table[s], L)[:, 0]
        ro, _ = oracle.mla_attention(mlad.q_rows(s), codes, cs, mlad.q_pos(s), mlad.scale)
        assert_close(got[4 * s:4 * s + 4], ro, FP8_MAX_ABS, FP8_L1, f"packed MTP decode seq={s}")


def test_packed_sparse_chain_full_size(pa_lib):
    """131,072 cached + 4,096 new tokens on the packed layout: MXFP4 indexer (17 key
    chunks) -> top-2,048 -> sparse MLA on the latent view; sampled rows against the oracle,
    top-k bit-exact on the GPU's scores."""
    import torch
    mla, idx = W.make_sparse_mla(5, fp4_keys=True)
    dev = MlaOnDevice(mla, idx)
    blocks, lat, ix = _packed_dev(pa_lib, mla, idx)
    n_q, k = dev.q_idx.shape[0], 2048
    topk, sc = _indexer(pa_lib, dev, ix, k)
    lse = torch.empty((n_q, 64), dtype=torch.float32, device="cuda")
    out = pa_lib.sparse_mla_attn(dev.q, lat, dev.bt, dev.q_seq, topk, scale=mla.scale, lse=lse)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 777, 2048, 3000, n_q - 1])
    sc_rows = sc.index_select(0, torch.from_numpy(rows).cuda()).cpu().numpy()
    tk = topk.cpu().numpy()
    got, lg = bf16_out(out), lse.cpu().numpy()
    del sc
    torch.cuda.empty_cache()
    _check_fp4_rows(mla, idx, 0, rows, sc_rows, tk[rows], k, "packed full size")
    L = int(mla.total_len[0])
    codes = oracle.gather_paged(mla.kv_pool, mla.block_table[0], L)
    cs = oracle.gather_paged(mla.kv_scale[..., None], mla.block_table[0], L)[:, 0]
    ro, rl = oracle.sparse_mla_attention(mla.q[rows], codes, cs, tk[rows], mla.scale)
    assert_close(got[rows], ro, FP8_MAX_ABS, FP8_L1, "packed full-size sparse MLA")
    np.testing.assert_allclose(lg[rows], rl, atol=LSE_ABS)
