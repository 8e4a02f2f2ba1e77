"""GPU: the allocation-free decode entry point (paged_attn_decode_noalloc) against the
workspace entry point (paged_attn_decode).  Both run the same kernels with the same fixed
partition, so their outputs and log-sum-exps must agree bit for bit.  Two calls in a row,
the second smaller, so the second runs on scratch that still holds the first call's
contents; for the GQA pool and for the FP8 MLA latent pool."""
import numpy as np
import pytest

import workloads as W
from workloads.device import GqaOnDevice, MlaOnDevice

pytestmark = pytest.mark.gpu


def _both(pa, q, pool, bt, ctx, T, H, max_ctx, scale, d_v):
    import torch
    S = bt.shape[0]
    lse_w = torch.empty((S, T, H), dtype=torch.float32, device="cuda")
    lse_n = torch.empty_like(lse_w)
    nws = pa.load().paged_attn_decode_workspace_size(S, T, H, max_ctx, pa.ctypes.byref(pool))
    assert 0 < nws <= pa.load().paged_attn_decode_noalloc_max_bytes()
    out_w = pa.paged_attn_decode(q, pool, bt, ctx, q_per_seq=T, num_q_heads=H, max_context_len=max_ctx,
                                 scale=scale, lse=lse_w)
    out_n = torch.full((S, T, H, d_v), 7.0, dtype=torch.bfloat16, device="cuda")
    pa.paged_attn_decode_noalloc(q, pool, bt, ctx, q_per_seq=T, num_q_heads=H, max_context_len=max_ctx,
                                 scale=scale, out=out_n, lse=lse_n)
    torch.cuda.synchronize()
    assert torch.equal(out_w.view(torch.int16), out_n.view(torch.int16))
    assert torch.equal(lse_w.view(torch.int32), lse_n.view(torch.int32))
    return nws


def test_noalloc_gqa_decode_matches_workspace_call(pa_lib):
    big = W.make_gqa_decode(201, n_sessions=2, members=4, lo=3000, hi=9000)
    small = W.make_gqa_decode(202, n_sessions=1, members=3, lo=100, hi=700, q_per_seq=2)
    sizes = []
    for wl, T in ((big, 1), (small, 2)):
        dev = GqaOnDevice(wl)
        S = wl.num_seqs
        q = dev.q.view(S, T, wl.num_q_heads, wl.head_dim)
        sizes.append(_both(pa_lib, q, dev.pool, dev.bt, dev.total_len, T, wl.num_q_heads, dev.max_total,
                           wl.scale, wl.head_dim))
    assert sizes[1] < sizes[0]


def test_noalloc_mla_decode_matches_workspace_call(pa_lib):
    big = W.make_mla_decode(203, lengths=[9000, 5000, 4097, 300], q_per_seq=4, num_q_heads=64)
    small = W.make_mla_decode(204, lengths=[700, 65], q_per_seq=1, num_q_heads=64)
    sizes = []
    for mla, T in ((big, 4), (small, 1)):
        dev = MlaOnDevice(mla)
        S = mla.num_seqs
        q = dev.q.view(S, T, mla.num_q_heads, 576)
        sizes.append(_both(pa_lib, q, dev.pool, dev.bt, dev.total_len, T, mla.num_q_heads, dev.max_total,
                           mla.scale, 512))
    assert sizes[1] < sizes[0]


def test_noalloc_rejects_sizes_beyond_its_scratch(pa_lib):
    import torch
    wl = W.make_gqa_decode(205, n_sessions=1, members=2, lo=100, hi=200)
    dev = GqaOnDevice(wl)
    S = wl.num_seqs
    big_ctx = 16_000_000                     # a bound whose workspace (pass lists) exceeds the scratch
    bt = torch.full((S, big_ctx // 16), -1, dtype=torch.int32, device="cuda")
    need = pa_lib.load().paged_attn_decode_workspace_size(S, 1, 32, big_ctx, pa_lib.ctypes.byref(dev.pool))
    assert need > pa_lib.load().paged_attn_decode_noalloc_max_bytes()
    with pytest.raises(pa_lib.PAError, match="PA_ERR_WORKSPACE"):
        pa_lib.paged_attn_decode_noalloc(dev.q.view(S, 1, 32, 128), dev.pool, bt, dev.total_len, q_per_seq=1,
                                         num_q_heads=32, max_context_len=big_ctx, scale=wl.scale)
