"""GPU parity: paged KV append (bf16 copy and per-token FP8 quantisation) against the
oracle, bit for bit on the whole pool.  Inputs are seeded (workloads.make_append); the
pool starts as random bytes so that any stray write shows."""
import numpy as np
import pytest

import oracle
import workloads as W
from workloads.device import t as to_dev

pytestmark = pytest.mark.gpu


def _bits16(x):
    import torch
    return x.view(torch.int16).cpu().numpy().view(np.uint16)


def _run_gqa(pa, a, hkv, d, seed, poison=None):
    import torch
    rng = np.random.default_rng(seed)
    kp = rng.integers(0, 1 << 16, (a.num_blocks, hkv, 16, d), dtype=np.uint16)
    vp = rng.integers(0, 1 << 16, (a.num_blocks, hkv, 16, d), dtype=np.uint16)
    bt = a.block_table.copy()
    if poison is not None:
        bt[poison] = 1 << 20                        # out-of-range block id: not written
    kd, vd = to_dev(kp, "cuda"), to_dev(vp, "cuda")
    pool = pa.gqa_pool(kd, vd)
    print(f"append gqa: seqs={len(a.new_len)} rows={a.k_new.shape[0]} hkv={hkv} d={d}", flush=True)
    pa.paged_kv_append(pool, to_dev(bt, "cuda"), to_dev(a.cached_len, "cuda"), to_dev(a.new_len, "cuda"),
                       to_dev(a.q_start, "cuda"), to_dev(a.k_new, "cuda"), to_dev(a.v_new, "cuda"),
                       max_new_len=int(a.new_len.max()))
    torch.cuda.synchronize()
    ek, ev = oracle.append_gqa(kp, vp, bt, a.cached_len, a.new_len, a.q_start, a.k_new, a.v_new)
    assert np.array_equal(_bits16(kd), ek)
    assert np.array_equal(_bits16(vd), ev)
    return kp, ek


@pytest.mark.parametrize("hkv,d", [(8, 128), (2, 64), (1, 128)])
def test_append_gqa_ragged(pa_lib, hkv, d):
    a = W.make_append(40 + d + hkv, cached=[0, 5, 16, 31, 200, 7], new=[3, 20, 1, 0, 17, 64],
                      block_size=16, row_shape=(hkv, d), with_v=True)
    kp, ek = _run_gqa(pa_lib, a, hkv, d, 1)
    assert not np.array_equal(kp, ek)


def test_append_gqa_skips_bad_block(pa_lib):
    a = W.make_append(47, cached=[5, 0], new=[20, 40], block_size=16, row_shape=(2, 64), with_v=True)
    kp, ek = _run_gqa(pa_lib, a, 2, 64, 2, poison=(1, 1))   # seq 1, tokens 16..31
    assert np.array_equal(ek[a.block_table[1, 1]], kp[a.block_table[1, 1]])


def _run_fp8(pa, a, D, seed):
    import torch
    rng = np.random.default_rng(seed)
    pool = rng.integers(0, 256, (a.num_blocks, 64, D), dtype=np.uint8)
    sc = rng.random((a.num_blocks, 64)).astype(np.float32)
    pd, sd = to_dev(pool, "cuda"), to_dev(sc, "cuda")
    p = pa.mla_pool(pd, sd) if D == 576 else pa.indexer_pool(pd, sd)
    print(f"append fp8: seqs={len(a.new_len)} rows={a.k_new.shape[0]} D={D}", flush=True)
    pa.paged_kv_append(p, to_dev(a.block_table, "cuda"), to_dev(a.cached_len, "cuda"),
                       to_dev(a.new_len, "cuda"), to_dev(a.q_start, "cuda"), to_dev(a.k_new, "cuda"),
                       max_new_len=int(a.new_len.max()))
    torch.cuda.synchronize()
    ep, es = oracle.append_fp8(pool, sc, a.block_table, a.cached_len, a.new_len, a.q_start, a.k_new)
    got_p, got_s = pd.cpu().numpy(), sd.cpu().numpy()
    bad = np.argwhere(np.any(got_p != ep, axis=2))
    assert bad.size == 0, f"{len(bad)} rows differ, first {bad[:3].tolist()}"
    assert np.array_equal(got_s.view(np.uint32), es.view(np.uint32))


@pytest.mark.parametrize("D", [576, 128])
def test_append_fp8_ragged(pa_lib, D):
    a = W.make_append(50 + D, cached=[0, 63, 64, 1000, 5], new=[4, 4, 130, 1, 0], block_size=64,
                      row_shape=(D,), with_v=False, row_mults=(1.0, 1e-30, 3e-3, 1e4, 0.25), zero_rows=2)
    _run_fp8(pa_lib, a, D, 3)


def test_append_fp8_rounding_sweep(pa_lib):
    """Rows whose largest magnitude is exactly 448 get scale 1, so every code is the E4M3
    rounding of the exact bf16 input: every representable value, every halfway point
    between neighbours (ties to even) and the bf16 neighbours of each halfway point."""
    vals = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mid = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    mid_bits = W.bf16_bits(mid)
    assert np.array_equal(oracle.bf16_to_f64(mid_bits), mid.astype(np.float64))   # exact in bf16
    pos_bits = np.concatenate([W.bf16_bits(vals.astype(np.float32)), mid_bits,
                               mid_bits + np.uint16(1), mid_bits[1:] - np.uint16(1)])
    body = np.concatenate([pos_bits, pos_bits | np.uint16(0x8000)])
    per_row = 575
    n_rows = -(-body.size // per_row)
    flat = np.zeros(n_rows * per_row, np.uint16)
    flat[:body.size] = body
    bits = np.empty((n_rows, 576), np.uint16)
    bits[:, 0] = W.bf16_bits(np.array([448.0], np.float32))[0]
    bits[:, 1:] = flat.reshape(n_rows, per_row)
    assert np.abs(oracle.bf16_to_f64(bits)).max(axis=1).tolist() == [448.0] * n_rows
    a = W.make_append(60, cached=[3], new=[n_rows], block_size=64, row_shape=(576,), with_v=False)
    a.k_new = bits
    _run_fp8(pa_lib, a, 576, 4)


def test_append_then_decode_reads_it(pa_lib):
    """Append the last 4 tokens of every sequence into an MLA pool, then decode over it:
    the decode call sees the appended rows (compared with the oracle's attention over the
    oracle-appended pool)."""
    import torch
    from gpu_util import FP8_MAX_ABS, FP8_L1, assert_close, bf16_out
    S, T, H = 3, 4, 16
    cached = np.array([60, 200, 1])
    a = W.make_append(61, cached=cached, new=[T] * S, block_size=64, row_shape=(576,), with_v=False)
    rng = np.random.default_rng(5)
    pool = W.fp8_quantize_tokens(rng.standard_normal((a.num_blocks * 64, 576)).astype(np.float32))
    pool_b = pool[0].reshape(a.num_blocks, 64, 576)
    pool_s = pool[1].reshape(a.num_blocks, 64)
    pd, sd = to_dev(pool_b, "cuda"), to_dev(pool_s, "cuda")
    p = pa_lib.mla_pool(pd, sd)
    bt = to_dev(a.block_table, "cuda")
    pa_lib.paged_kv_append(p, bt, to_dev(a.cached_len, "cuda"), to_dev(a.new_len, "cuda"),
                           to_dev(a.q_start, "cuda"), to_dev(a.k_new, "cuda"), max_new_len=T)
    ctx = (cached + T).astype(np.int32)
    q = W.bf16_bits((rng.standard_normal((S, T, H, 576)) * 0.5).astype(np.float32))
    scale = 1.0 / np.sqrt(576)
    out = pa_lib.paged_attn_decode(to_dev(q, "cuda"), p, bt, to_dev(ctx, "cuda"), q_per_seq=T,
                                   num_q_heads=H, max_context_len=int(ctx.max()), scale=scale)
    torch.cuda.synchronize()
    ep, es = oracle.append_fp8(pool_b, pool_s, a.block_table, a.cached_len, a.new_len, a.q_start,
                               a.k_new)
    for s in range(S):
        L = int(ctx[s])
        kb = oracle.gather_paged(ep, a.block_table[s], L)
        ks = oracle.gather_paged(es, a.block_table[s], L)
        ref, _ = oracle.mla_attention(q[s], kb, ks, np.arange(L - T, L), scale)
        assert_close(bf16_out(out[s]), ref, FP8_MAX_ABS, FP8_L1, f"decode after append s={s}")


def _full_size_gqa(pa, cached, new, hkv, d, seed):
    """Append into a zeroed pool of the full workload size; every written row equals its
    input row and nothing else in the pool changes (no row of N(0,1) input is all zero)."""
    import torch
    a = W.make_append(seed, cached=cached, new=new, block_size=16, row_shape=(hkv, d), with_v=True)
    kd = torch.zeros((a.num_blocks, hkv, 16, d), dtype=torch.bfloat16, device="cuda")
    vd = torch.zeros_like(kd)
    pool = pa.gqa_pool(kd, vd)
    print(f"append gqa full size: blocks={a.num_blocks} rows={a.k_new.shape[0]}", flush=True)
    pa.paged_kv_append(pool, to_dev(a.block_table, "cuda"), to_dev(a.cached_len, "cuda"),
                       to_dev(a.new_len, "cuda"), to_dev(a.q_start, "cuda"), to_dev(a.k_new, "cuda"),
                       to_dev(a.v_new, "cuda"), max_new_len=int(a.new_len.max()))
    torch.cuda.synchronize()
    seq, pos = oracle.token_positions(a.cached_len, a.new_len, a.q_start, a.k_new.shape[0])
    blk = a.block_table[seq, pos // 16]
    for dev, src in ((kd, a.k_new), (vd, a.v_new)):
        rows = dev[torch.from_numpy(blk).cuda(), :, torch.from_numpy(pos % 16).cuda(), :]
        assert np.array_equal(_bits16(rows), src)
        changed = int((dev.view(torch.int16) != 0).any(dim=3).sum())
        assert changed == src.shape[0] * hkv


def test_append_gqa_prefill_suffix_full_size(pa_lib):
    """The suffix-prefill workload: 8 sequences x 2048 new tokens after 142000 cached,
    8 KV heads x 128."""
    _full_size_gqa(pa_lib, [142000] * 8, [2048] * 8, 8, 128, 70)


def _full_size_fp8(pa, cached, new, D, seed):
    import torch
    a = W.make_append(seed, cached=cached, new=new, block_size=64, row_shape=(D,), with_v=False)
    pd = torch.zeros((a.num_blocks, 64, D), dtype=torch.uint8, device="cuda")
    sd = torch.zeros((a.num_blocks, 64), dtype=torch.float32, device="cuda")
    p = pa.mla_pool(pd, sd) if D == 576 else pa.indexer_pool(pd, sd)
    print(f"append fp8 full size: D={D} blocks={a.num_blocks} rows={a.k_new.shape[0]}", flush=True)
    pa.paged_kv_append(p, to_dev(a.block_table, "cuda"), to_dev(a.cached_len, "cuda"),
                       to_dev(a.new_len, "cuda"), to_dev(a.q_start, "cuda"), to_dev(a.k_new, "cuda"),
                       max_new_len=int(a.new_len.max()))
    torch.cuda.synchronize()
    seq, pos = oracle.token_positions(a.cached_len, a.new_len, a.q_start, a.k_new.shape[0])
    blk = torch.from_numpy(a.block_table[seq, pos // 64]).cuda()
    r = torch.from_numpy(pos % 64).cuda()
    got_codes, got_scale = pd[blk, r].cpu().numpy(), sd[blk, r].cpu().numpy()
    for i in range(a.k_new.shape[0]):
        codes, sc = oracle.quantize_token_fp8(a.k_new[i])
        assert np.array_equal(got_codes[i], codes) and got_scale[i] == sc, f"row {i}"
    assert int((sd != 0).sum()) == a.k_new.shape[0]


def test_append_fp8_mla_decode_full_size(pa_lib):
    """The MLA MTP3 decode workload: 64 sequences x 4 new latent rows, contexts in
    [32768, 262144]."""
    ctx = np.random.default_rng(71).integers(32768, 262145, 64)
    _full_size_fp8(pa_lib, ctx - 4, [4] * 64, 576, 71)


@pytest.mark.parametrize("D", [576, 128])
def test_append_fp8_sparse_prefill_full_size(pa_lib, D):
    """The sparse-MLA workload's new tokens: 4096 rows after 131072 cached (latent and
    indexer keys)."""
    _full_size_fp8(pa_lib, [131072], [4096], D, 72 + D)


@pytest.mark.parametrize("seed", range(8))
def test_append_random_shapes(pa_lib, seed):
    """Random batches of (cached, new) pairs, bf16 rows of random head counts and dims and
    FP8 rows of both widths; the whole pool is compared bit for bit each time."""
    rng = np.random.default_rng(1500 + seed)
    S = int(rng.integers(1, 9))
    cached = [int(x) for x in rng.integers(0, 700, S)]
    new = [int(x) for x in rng.integers(0, 90, S)]
    hkv, d = int(rng.choice([1, 2, 4, 8])), int(rng.choice([64, 128]))
    a = W.make_append(1550 + seed, cached=cached, new=new, block_size=16, row_shape=(hkv, d), with_v=True)
    if a.k_new.shape[0] > 0:
        _run_gqa(pa_lib, a, hkv, d, 1600 + seed)
    D = int(rng.choice([576, 128]))
    f = W.make_append(1650 + seed, cached=cached, new=new, block_size=64, row_shape=(D,), with_v=False)
    if f.k_new.shape[0] > 0:
        _run_fp8(pa_lib, f, D, 1700 + seed)
