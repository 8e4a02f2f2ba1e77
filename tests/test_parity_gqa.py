"""GPU parity: paged GQA/MHA prefill and decode against the fp64 oracle.

Inputs are seeded synthetic workloads (workloads.gen); every expected value is computed
by oracle/ on the CPU from the same bytes.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from workloads.device import GqaOnDevice
from gpu_util import BF16_L1, BF16_MAX_ABS, LSE_ABS, assert_close, assert_close_stress, bf16_out

pytestmark = pytest.mark.gpu


def _prefill(pa, dev, lse=True):
    import torch
    wl = dev.wl
    lse_t = torch.empty((wl.q.shape[0], wl.num_q_heads), dtype=torch.float32, device="cuda") if lse else None
    out = pa.paged_attn_prefill(dev.q, dev.pool, dev.bt, dev.cached, dev.n_new, dev.q_start,
                                num_q_heads=wl.num_q_heads, max_new_len=dev.max_new,
                                max_total_len=dev.max_total, scale=wl.scale, lse=lse_t)
    torch.cuda.synchronize()
    return out, lse_t


def test_gather_bit_exact(pa_lib):
    import torch
    wl = W.make_gqa(21, lengths=[256, 37, 1], n_new=[16, 5, 1], num_q_heads=8, num_kv_heads=8, head_dim=64)
    dev = GqaOnDevice(wl)
    for s in range(wl.num_seqs):
        L = int(wl.total_len[s])
        k = torch.empty((L, 8, 64), dtype=torch.bfloat16, device="cuda")
        v = torch.empty_like(k)
        pa_lib.pa_test_gather_kv(dev.pool, dev.bt, s, L, k, v)
        torch.cuda.synchronize()
        kc, vc = wl.kv_contiguous(s)
        assert np.array_equal(k.view(torch.int16).cpu().numpy().view(np.uint16), kc)
        assert np.array_equal(v.view(torch.int16).cpu().numpy().view(np.uint16), vc)


def test_prefill_tiny_config(pa_lib):
    """1 sequence, MHA 8 x 64, 240 cached tokens in 15 shuffled blocks + 16 new tokens."""
    wl = W.make_prefill_tiny(1)
    dev = GqaOnDevice(wl)
    out, lse = _prefill(pa_lib, dev)
    ref_o, ref_l = oracle.paged_gqa_attention(wl, 0)
    assert_close(bf16_out(out), ref_o, BF16_MAX_ABS, BF16_L1, "prefill tiny")
    np.testing.assert_allclose(lse.cpu().numpy(), ref_l, atol=LSE_ABS)


@pytest.mark.parametrize("G,D,Hkv", [(1, 64, 2), (2, 128, 2), (4, 128, 2), (8, 64, 2), (4, 64, 2),
                                     (8, 128, 1), (2, 128, 16), (4, 64, 3)])
def test_prefill_ragged(pa_lib, G, D, Hkv):
    cached = [0, 5, 1000, 33, 300]
    new = [1, 17, 130, 300, 64]
    lengths = [c + n for c, n in zip(cached, new)]
    wl = W.make_gqa(30 + G + D + Hkv, lengths=lengths, n_new=new, num_q_heads=Hkv * G, num_kv_heads=Hkv,
                    head_dim=D)
    dev = GqaOnDevice(wl)
    out, lse = _prefill(pa_lib, dev)
    got = bf16_out(out)
    lg = lse.cpu().numpy()
    for s in range(wl.num_seqs):
        ro, rl = oracle.paged_gqa_attention(wl, s)
        a, b = wl.q_start[s], wl.q_start[s + 1]
        assert_close(got[a:b], ro, BF16_MAX_ABS, BF16_L1, f"prefill G={G} D={D} Hkv={Hkv} seq={s}")
        np.testing.assert_allclose(lg[a:b], rl, atol=LSE_ABS)


def test_prefill_peaked_softmax(pa_lib):
    """Stress: queries x8 make the softmax peaked (tolerances bind harder)."""
    wl = W.make_gqa(41, lengths=[700, 129], n_new=[200, 129], num_q_heads=8, num_kv_heads=2, head_dim=128,
                    q_mult=8.0)
    dev = GqaOnDevice(wl)
    out, _ = _prefill(pa_lib, dev, lse=False)
    got = bf16_out(out)
    for s in range(2):
        ro, _ = oracle.paged_gqa_attention(wl, s)
        assert_close_stress(got[wl.q_start[s]:wl.q_start[s + 1]], ro, BF16_MAX_ABS, BF16_L1, f"peaked seq={s}")


def _decode(pa, dev, T, lse=True):
    import torch
    wl = dev.wl
    S = wl.num_seqs
    q = dev.q.view(S, T, wl.num_q_heads, wl.head_dim)
    lse_t = torch.empty((S, T, wl.num_q_heads), dtype=torch.float32, device="cuda") if lse else None
    out = pa.paged_attn_decode(q, dev.pool, dev.bt, dev.total_len, q_per_seq=T, num_q_heads=wl.num_q_heads,
                               max_context_len=dev.max_total, scale=wl.scale, lse=lse_t)
    torch.cuda.synchronize()
    return out, lse_t


@pytest.mark.parametrize("T,G,D,shuffle", [(1, 4, 128, False), (1, 4, 128, True), (4, 4, 128, False),
                                            (2, 8, 64, False), (1, 1, 64, False), (3, 2, 128, True)])
def test_decode_sessions(pa_lib, T, G, D, shuffle):
    """Decode with sessions sharing 90% of their blocks; lengths span 1..several splits."""
    wl = W.make_gqa_decode(50 + T * 10 + G, n_sessions=3, members=3, lo=20, hi=5000, q_per_seq=T,
                           num_q_heads=2 * G, num_kv_heads=2, head_dim=D, shuffle_batch=shuffle,
                           keep_content=True)
    dev = GqaOnDevice(wl)
    out, lse = _decode(pa_lib, dev, T)
    got = bf16_out(out).reshape(wl.num_seqs * T, wl.num_q_heads, D)
    lg = lse.cpu().numpy().reshape(wl.num_seqs * T, wl.num_q_heads)
    for s in range(wl.num_seqs):
        ro, rl = oracle.paged_gqa_attention(wl, s)
        assert_close(got[s * T:(s + 1) * T], ro, BF16_MAX_ABS, BF16_L1, f"decode T={T} G={G} seq={s}")
        np.testing.assert_allclose(lg[s * T:(s + 1) * T], rl, atol=LSE_ABS)


@pytest.mark.parametrize("Hkv,G,T", [(1, 8, 1), (4, 4, 2), (16, 2, 1), (3, 4, 1)])
def test_decode_kv_head_counts(pa_lib, Hkv, G, T):
    """KV head counts other than 2 and 8: one head split over all 8 waves (8 sub-ranges of
    each piece), 4 heads x 2 sub-ranges, 16 heads (two per wave) and 3 heads (8 does not
    divide: one sub-range, waves 3-7 idle); sessions share 90 % of their blocks."""
    wl = W.make_gqa_decode(80 + Hkv, n_sessions=3, members=4, lo=30, hi=4000, q_per_seq=T,
                           num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim=128, keep_content=True)
    dev = GqaOnDevice(wl)
    out, lse = _decode(pa_lib, dev, T)
    got = bf16_out(out).reshape(wl.num_seqs * T, wl.num_q_heads, 128)
    lg = lse.cpu().numpy().reshape(wl.num_seqs * T, wl.num_q_heads)
    for s in range(wl.num_seqs):
        ro, rl = oracle.paged_gqa_attention(wl, s)
        assert_close(got[s * T:(s + 1) * T], ro, BF16_MAX_ABS, BF16_L1, f"decode Hkv={Hkv} G={G} T={T} seq={s}")
        np.testing.assert_allclose(lg[s * T:(s + 1) * T], rl, atol=LSE_ABS)


def test_decode_edge_lengths_and_determinism(pa_lib):
    """Contexts of 1, 16, 17, 1023, 1024, 1025 and 4097 tokens; two runs bit-identical."""
    import torch
    lengths = [1, 16, 17, 1023, 1024, 1025, 4097]
    wl = W.make_gqa(61, lengths=lengths, n_new=[1] * 7, num_q_heads=32, num_kv_heads=8, head_dim=128)
    dev = GqaOnDevice(wl)
    out1, _ = _decode(pa_lib, dev, 1)
    out2, _ = _decode(pa_lib, dev, 1)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    got = bf16_out(out1).reshape(7, 32, 128)
    for s in range(7):
        ro, _ = oracle.paged_gqa_attention(wl, s)
        assert_close(got[s:s + 1], ro, BF16_MAX_ABS, BF16_L1, f"decode L={lengths[s]}")


def test_decode_plan_beyond_the_lds_index(pa_lib):
    """A context bound of 1,000,000 tokens over 34 groups of 2 sequences (2 query tokens x 8
    heads per KV head: 16 rows each) makes 34 x 123 plan regions: more region and piece
    starts than the attention kernel's 4,096-int LDS index holds, so the separate
    scan kernel numbers them in the workspace.  The actual contexts are short, so the
    regions past them are empty: the partition, and hence the output, is bit-identical to
    the same call under the tight bound (numbered in LDS), and both match the oracle."""
    import torch
    T, Hq, Hkv, S = 2, 16, 2, 68
    lengths = [int(x) for x in np.random.default_rng(71).integers(40, 3000, S)]
    wl = W.make_gqa(71, lengths=lengths, n_new=[T] * S, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=128)
    dev = GqaOnDevice(wl)
    big = 1_000_000
    groups = S // 2
    assert groups * -(-big // 8192) + groups + 2 > 4096 and groups * -(-dev.max_total // 8192) + groups + 2 <= 4096
    bt_wide = torch.full((S, big // 16), -1, dtype=torch.int32, device="cuda")
    bt_wide[:, :dev.bt.shape[1]] = dev.bt
    q = dev.q.view(S, T, Hq, 128)
    outs = []
    for bt, bound in ((dev.bt, dev.max_total), (bt_wide, big)):
        outs.append(pa_lib.paged_attn_decode(q, dev.pool, bt, dev.total_len, q_per_seq=T, num_q_heads=Hq,
                                             max_context_len=bound, scale=wl.scale))
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    got = bf16_out(outs[1]).reshape(S * T, Hq, 128)
    for s in range(S):
        ro, _ = oracle.paged_gqa_attention(wl, s)
        assert_close(got[s * T:(s + 1) * T], ro, BF16_MAX_ABS, BF16_L1, f"decode wide plan seq={s}")


def test_decode_many_groups_in_lds_numbering(pa_lib):
    """1,100 sequences in 550 groups of two (2 query tokens x 8 heads per KV head: 16 rows
    each): the attention workgroups' in-LDS numbering runs its region scan and its group
    scan over more than one 512-thread round each.  Every sequence matches the oracle."""
    T, Hq, Hkv, S = 2, 16, 2, 1100
    lengths = [int(x) for x in np.random.default_rng(72).integers(20, 300, S)]
    wl = W.make_gqa(72, lengths=lengths, n_new=[T] * S, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=64)
    dev = GqaOnDevice(wl)
    out, lse = _decode(pa_lib, dev, T)
    got = bf16_out(out).reshape(S * T, Hq, 64)
    lg = lse.cpu().numpy().reshape(S * T, Hq)
    for s in range(S):
        ro, rl = oracle.paged_gqa_attention(wl, s)
        assert_close(got[s * T:(s + 1) * T], ro, BF16_MAX_ABS, BF16_L1, f"decode many groups seq={s}")
        np.testing.assert_allclose(lg[s * T:(s + 1) * T], rl, atol=LSE_ABS)


def test_decode_full_size_sampled(pa_lib):
    """The benchmarked decode workload at full size (64 sequences, 8 sessions, contexts
    4K-142K); a sample of sequences is checked against the oracle."""
    wl = W.make_gqa_decode(2)
    dev = GqaOnDevice(wl)
    out, lse = _decode(pa_lib, dev, 1)
    got = bf16_out(out).reshape(64, 32, 128)
    lg = lse.cpu().numpy().reshape(64, 32)
    order = np.argsort(wl.total_len)
    for s in [int(order[0]), int(order[31]), int(order[-1]), 9]:
        ro, rl = oracle.paged_gqa_attention(wl, s)
        assert_close(got[s:s + 1], ro, BF16_MAX_ABS, BF16_L1, f"decode full seq={s} L={wl.total_len[s]}")
        np.testing.assert_allclose(lg[s:s + 1], rl, atol=LSE_ABS)


# --------------------------------------------------------------------------- cold prompts and
# chunked-prefill steps (a workgroup takes a tile and its mirror in the sequence)
@pytest.mark.parametrize("G,D,new", [(4, 128, 1000), (8, 64, 1000), (1, 128, 300), (2, 64, 129)])
def test_prefill_cold_prompt(pa_lib, G, D, new):
    """Nothing cached: causal over the prompt itself.  Tile counts even and odd (a middle
    tile without a mirror), and a last partial tile."""
    wl = W.make_cold_prefill(60 + G, num_seqs=2, new=new, num_q_heads=2 * G, num_kv_heads=2,
                             head_dim=D, keep_content=True)
    dev = GqaOnDevice(wl)
    out, lse = _prefill(pa_lib, dev)
    got, lg = bf16_out(out), lse.cpu().numpy()
    for s in range(wl.num_seqs):
        ro, rl = oracle.paged_gqa_attention(wl, s)
        a, b = wl.q_start[s], wl.q_start[s + 1]
        assert_close(got[a:b], ro, BF16_MAX_ABS, BF16_L1, f"cold prompt G={G} D={D} seq={s}")
        np.testing.assert_allclose(lg[a:b], rl, atol=LSE_ABS)


def test_prefill_chunked_step(pa_lib):
    """A chunked-prefill step: two requests advance by a prefill chunk on top of their
    context, five add one decode token, in one call."""
    wl = W.make_chunked_mixed(8, n_chunked=2, chunk=130, n_decode=5, lo=200, hi=2000,
                              num_q_heads=8, num_kv_heads=2, head_dim=128, keep_content=True)
    dev = GqaOnDevice(wl)
    out, lse = _prefill(pa_lib, dev)
    got, lg = bf16_out(out), lse.cpu().numpy()
    for s in range(wl.num_seqs):
        ro, rl = oracle.paged_gqa_attention(wl, s)
        a, b = wl.q_start[s], wl.q_start[s + 1]
        assert_close(got[a:b], ro, BF16_MAX_ABS, BF16_L1, f"chunked step seq={s}")
        np.testing.assert_allclose(lg[a:b], rl, atol=LSE_ABS)


def test_prefill_cold_prompt_full_size_sampled(pa_lib):
    """The benchmarked cold-prompt shape (32,768 new tokens, 32q/8kv, d128; one sequence
    of the batch), checked on sampled query rows with the oracle's attention over the
    rows' visible keys."""
    wl = W.make_cold_prefill(7, num_seqs=1, new=32768, keep_content=False)
    dev = GqaOnDevice(wl)
    out, lse = _prefill(pa_lib, dev)
    got, lg = bf16_out(out), lse.cpu().numpy()
    L = int(wl.total_len[0])
    kp = np.swapaxes(wl.k_pool, 1, 2)
    vp = np.swapaxes(wl.v_pool, 1, 2)
    k = oracle.bf16_to_f64(oracle.gather_paged(kp, wl.block_table[0], L))
    v = oracle.bf16_to_f64(oracle.gather_paged(vp, wl.block_table[0], L))
    rows = np.array([0, 1, 31, 32, 4095, 16383, 16384, 32736, 32767])
    q = oracle.bf16_to_f64(wl.q[rows])
    ro, rl = oracle.attention(q, k, v, rows, wl.scale)
    assert_close(got[rows], ro, BF16_MAX_ABS, BF16_L1, "cold prompt 32768 sampled rows")
    np.testing.assert_allclose(lg[rows], rl, atol=LSE_ABS)


def test_prefill_split_k_long_contexts(pa_lib):
    """Few, short new-token tiles over long contexts: the prefill splits each tile's keys
    into 8,192-key ranges and merges the partials in a fixed order (decode tokens and
    prefill chunks in one call)."""
    wl = W.make_chunked_mixed(9, n_chunked=2, chunk=100, n_decode=3, lo=40000, hi=70000,
                              num_q_heads=8, num_kv_heads=2, head_dim=128, keep_content=True)
    dev = GqaOnDevice(wl)
    assert pa_lib.load().paged_attn_prefill_workspace_size(
        wl.num_seqs, 8, dev.max_new, dev.max_total, pa_lib.ctypes.byref(dev.pool)) > 0   # split-K taken
    out, lse = _prefill(pa_lib, dev)
    got, lg = bf16_out(out), lse.cpu().numpy()
    for s in range(wl.num_seqs):
        ro, rl = oracle.paged_gqa_attention(wl, s)
        a, b = wl.q_start[s], wl.q_start[s + 1]
        assert_close(got[a:b], ro, BF16_MAX_ABS, BF16_L1, f"split-K prefill seq={s}")
        np.testing.assert_allclose(lg[a:b], rl, atol=LSE_ABS)
    # fixed-order merge: bit-identical on a rerun
    out2, lse2 = _prefill(pa_lib, dev)
    assert bf16_out(out2).tobytes() == got.tobytes() and np.array_equal(lse2.cpu().numpy(), lg)


def test_prefill_split_k_clamped_lengths_and_gapped_rows(pa_lib):
    """Split-K with a new_len above the host maximum and gaps between the sequences' query
    rows: only the first max_new_len new tokens of a sequence are computed, rows outside
    the sequences and past the clamp are never written, and nothing past the caller's
    workspace of paged_attn_prefill_workspace_size bytes changes."""
    import torch
    from workloads.device import t as to_dev
    wl = W.make_chunked_mixed(10, n_chunked=2, chunk=100, n_decode=3, lo=40000, hi=70000,
                              num_q_heads=8, num_kv_heads=2, head_dim=128, keep_content=True)
    dev = GqaOnDevice(wl)
    S, H, D, max_new = wl.num_seqs, 8, 128, 60
    gap = 7
    q_start2 = (wl.q_start + gap * np.arange(S + 1)).astype(np.int32)
    n_rows = int(q_start2[-1])
    q2 = np.zeros((n_rows, H, D), np.uint16)
    for s in range(S):
        q2[q_start2[s]:q_start2[s] + wl.n_new[s]] = wl.q_rows(s)
    q2_d, qs2_d = to_dev(q2, "cuda"), to_dev(q_start2, "cuda")
    nws = pa_lib.load().paged_attn_prefill_workspace_size(S, H, max_new, dev.max_total, pa_lib.ctypes.byref(dev.pool))
    assert nws > 0                                         # split-K taken
    guard = 1 << 20
    ws = torch.full((nws + guard,), 0xA5, dtype=torch.uint8, device="cuda")
    sentinel = torch.tensor(0x7F80, dtype=torch.int16)     # bf16 +inf bit pattern
    out = torch.full((n_rows, H, D), 0x7F80, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    pa_lib.paged_attn_prefill(q2_d, dev.pool, dev.bt, dev.cached, dev.n_new, qs2_d, num_q_heads=H,
                              max_new_len=max_new, max_total_len=dev.max_total, scale=wl.scale, out=out,
                              workspace=ws[:nws])
    torch.cuda.synchronize()
    assert torch.all(ws[nws:] == 0xA5), "a write landed past the workspace"
    raw = out.view(torch.int16).cpu()
    got = bf16_out(out)
    written = np.zeros(n_rows, bool)
    for s in range(S):
        n = min(int(wl.n_new[s]), max_new)
        a = int(q_start2[s])
        written[a:a + n] = True
        ro, _ = oracle.paged_gqa_attention(wl, s)
        assert_close(got[a:a + n], ro[:n], BF16_MAX_ABS, BF16_L1, f"clamped split-K seq={s}")
    assert torch.all(raw[torch.from_numpy(~written)] == sentinel), "rows outside the computed tokens changed"
