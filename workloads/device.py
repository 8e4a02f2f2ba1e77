"""Copy generated workloads into device memory (torch tensors on one GPU).

Plumbing only: the arrays are moved as-is (bf16 bit patterns as torch.bfloat16 views,
FP8 bytes as uint8, indices as int32).  Nothing here computes.
"""
from __future__ import annotations

import numpy as np


def t(x: np.ndarray, device):
    import torch
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(x).to(device)


def bf16_to_np(x) -> np.ndarray:
    """bf16 torch tensor -> uint16 bit patterns (host)."""
    import torch
    return x.detach().view(torch.int16).cpu().numpy().view(np.uint16)


class GqaOnDevice:
    """Device copies of a workloads.PagedGQA."""

    def __init__(self, wl, device="cuda"):
        import paged_prefix_cached_amd as pa
        self.wl = wl
        self.k_pool = t(wl.k_pool, device)
        self.v_pool = t(wl.v_pool, device)
        self.pool = pa.gqa_pool(self.k_pool, self.v_pool)
        self.bt = t(wl.block_table, device)
        self.total_len = t(wl.total_len.astype(np.int32), device)
        self.n_new = t(wl.n_new.astype(np.int32), device)
        self.cached = t((wl.total_len - wl.n_new).astype(np.int32), device)
        self.q_start = t(wl.q_start.astype(np.int32), device)
        self.q = t(wl.q, device)
        self.max_new = int(wl.n_new.max())
        self.max_total = int(wl.total_len.max())


class MlaOnDevice:
    """Device copies of a workloads.PagedMLA (and optionally its IndexerInput)."""

    def __init__(self, mla, idx=None, device="cuda"):
        import paged_prefix_cached_amd as pa
        self.mla = mla
        self.kv = t(mla.kv_pool, device)
        self.kv_scale = t(mla.kv_scale, device)
        self.pool = pa.mla_pool(self.kv, self.kv_scale)
        self.bt = t(mla.block_table, device)
        self.total_len = t(mla.total_len.astype(np.int32), device)
        self.n_new = t(mla.n_new.astype(np.int32), device)
        self.cached = t((mla.total_len - mla.n_new).astype(np.int32), device)
        self.q_start = t(mla.q_start.astype(np.int32), device)
        self.q = t(mla.q, device)
        self.max_new = int(mla.n_new.max())
        self.max_total = int(mla.total_len.max())
        seq_of_row = np.repeat(np.arange(mla.num_seqs, dtype=np.int32), mla.n_new)
        self.q_seq = t(seq_of_row, device)
        if idx is not None:
            self.idx_keys = t(idx.idx_pool, device)
            self.idx_scale = t(idx.idx_scale, device)
            self.idx_pool = pa.indexer_pool(self.idx_keys, self.idx_scale)
            self.q_idx = t(idx.q_idx, device)
            self.w = t(idx.w, device)
