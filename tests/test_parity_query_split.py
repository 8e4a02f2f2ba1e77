"""GPU parity for the FP8 Q.K products whose bf16 queries are split into two E4M3 terms after
a power-of-two scale (MLA decode, sparse MLA, the indexer on FP8 and on MXFP4 keys).  The
queries are rescaled so that rows (MLA) or heads (indexer) differ in magnitude by powers of
two, and elements within a row span 2^-23 .. 1 of the row's scale: each row then takes its
own scale, and the elements below 2^-9 of the row's largest take the split's small-element
path.  Power-of-two rescaling keeps every value an exact bf16, and the oracle reads the same
bits."""
import numpy as np
import pytest

import oracle
import workloads as W
from workloads.device import MlaOnDevice, t as to_dev
from gpu_util import FP8_L1, FP8_MAX_ABS, LSE_ABS, assert_close, bf16_out
import test_parity_packed as P

pytestmark = pytest.mark.gpu


def _rescale(bits: np.ndarray, factor: np.ndarray) -> np.ndarray:
    """bits [..., d] bf16 -> bf16 of x * 2^-(j mod 24) * factor (factor over the leading axes,
    powers of two)."""
    x = W.bf16_bits_to_f32(bits).astype(np.float64)
    j = np.arange(bits.shape[-1])
    y = x * np.exp2(-(j % 24)) * factor[..., None]
    out = W.bf16_bits(y.astype(np.float32))
    assert np.array_equal(W.bf16_bits_to_f32(out).astype(np.float64), y), "rescaling must stay exact"
    return out


def _mla_rows_factor(n_rows, Hq):
    r = np.arange(n_rows)[:, None]
    h = np.arange(Hq)[None, :]
    return np.exp2(((h % 5) - 4) + (r % 3))


def test_mla_decode_query_magnitudes(pa_lib):
    import torch
    T, Hq = 4, 64
    lengths = [T, 3000, 17000]
    mla = W.make_mla_decode(201, lengths=lengths, q_per_seq=T, num_q_heads=Hq)
    mla.q = _rescale(mla.q, _mla_rows_factor(mla.q.shape[0], Hq))
    dev = MlaOnDevice(mla)
    S = mla.num_seqs
    lse = torch.empty((S, T, Hq), dtype=torch.float32, device="cuda")
    out = pa_lib.paged_attn_decode(dev.q.view(S, T, Hq, 576), dev.pool, dev.bt, dev.total_len, q_per_seq=T,
                                   num_q_heads=Hq, max_context_len=dev.max_total, scale=mla.scale, lse=lse)
    torch.cuda.synchronize()
    got = bf16_out(out).reshape(S * T, Hq, 512)
    lg = lse.cpu().numpy().reshape(S * T, Hq)
    for s in range(S):
        L = int(mla.total_len[s])
        codes = oracle.gather_paged(mla.kv_pool, mla.block_table[s], L)
        sc = oracle.gather_paged(mla.kv_scale[..., None], mla.block_table[s], L)[:, 0]
        ro, rl = oracle.mla_attention(mla.q_rows(s), codes, sc, mla.q_pos(s), mla.scale)
        assert_close(got[s * T:(s + 1) * T], ro, FP8_MAX_ABS, FP8_L1, f"mla query magnitudes L={L}")
        np.testing.assert_allclose(lg[s * T:(s + 1) * T], rl, atol=LSE_ABS)


def test_indexer_and_sparse_mla_query_magnitudes(pa_lib):
    import torch
    lengths, n_new = [3000 + 40, 9000 + 24], [40, 24]
    mla, idx = W.make_sparse_mla(202, lengths=lengths, n_new=n_new, num_q_heads=64, idx_heads=64)
    n_q, H = idx.q_idx.shape[0], idx.q_idx.shape[1]
    idx.q_idx = _rescale(idx.q_idx, np.exp2((np.arange(H) % 9) - 4)[None, :].repeat(n_q, 0))
    mla.q = _rescale(mla.q, _mla_rows_factor(mla.q.shape[0], mla.q.shape[1]))
    dev = MlaOnDevice(mla, idx)
    k = 512
    scores = torch.empty((n_q, dev.max_total), dtype=torch.float32, device="cuda")
    topk = pa_lib.mla_indexer_topk(dev.q_idx, dev.w, dev.idx_pool, dev.bt, dev.cached, dev.n_new, dev.q_start,
                                   max_new_len=dev.max_new, max_total_len=dev.max_total, k=k, scores_out=scores)
    lse = torch.empty((n_q, 64), dtype=torch.float32, device="cuda")
    out = pa_lib.sparse_mla_attn(dev.q, dev.pool, dev.bt, dev.q_seq, topk, scale=mla.scale, lse=lse)
    torch.cuda.synchronize()
    tk, sc = topk.cpu().numpy(), scores.cpu().numpy().astype(np.float64)
    got_o, got_l = bf16_out(out), lse.cpu().numpy()
    for s in range(2):
        L = int(mla.total_len[s])
        a, b = mla.q_start[s], mla.q_start[s + 1]
        pos = mla.q_pos(s)
        kc = oracle.gather_paged(idx.idx_pool, mla.block_table[s], L)
        ks = oracle.gather_paged(idx.idx_scale[..., None], mla.block_table[s], L)[:, 0]
        ref = oracle.indexer_scores(idx.q_idx[a:b], idx.w[a:b], kc, ks, pos)
        got = sc[a:b, :L]
        fin = np.isfinite(ref)
        assert np.array_equal(fin, np.isfinite(got))
        err = np.abs(got[fin] - ref[fin])
        print(f"indexer query magnitudes seq={s}: max_abs={err.max():.3e} (ref max {np.abs(ref[fin]).max():.2f})",
              flush=True)
        assert err.max() <= 2e-3 * np.abs(ref[fin]).max()
        for r in range(b - a):
            assert np.array_equal(tk[a + r], oracle.topk_indices(got[r], pos[r] + 1, k)), (s, r)
        codes = oracle.gather_paged(mla.kv_pool, mla.block_table[s], L)
        cs = oracle.gather_paged(mla.kv_scale[..., None], mla.block_table[s], L)[:, 0]
        ro, rl = oracle.sparse_mla_attention(mla.q[a:b], codes, cs, tk[a:b], mla.scale)
        assert_close(got_o[a:b], ro, FP8_MAX_ABS, FP8_L1, f"sparse mla query magnitudes seq={s}")
        np.testing.assert_allclose(got_l[a:b], rl, atol=LSE_ABS)


def test_packed_fp4_indexer_query_magnitudes(pa_lib):
    lengths, n_new = [300 + 37, 9000 + 100], [37, 100]
    mla, idx = W.make_sparse_mla(203, lengths=lengths, n_new=n_new, num_q_heads=16, idx_heads=64, fp4_keys=True)
    n_q, H = idx.q_idx.shape[0], idx.q_idx.shape[1]
    idx.q_idx = _rescale(idx.q_idx, np.exp2((np.arange(H) % 9) - 4)[None, :].repeat(n_q, 0))
    dev = MlaOnDevice(mla, idx)
    blocks, lat, ix = P._packed_dev(pa_lib, mla, idx)
    k = 512
    topk, sc = P._indexer(pa_lib, dev, ix, k)
    tk, scn = topk.cpu().numpy(), sc.cpu().numpy()
    for s in range(2):
        rows = np.arange(mla.q_start[s], mla.q_start[s + 1])
        P._check_fp4_rows(mla, idx, s, rows, scn[rows], tk[rows], k, f"packed FP4 query magnitudes seq={s}")
