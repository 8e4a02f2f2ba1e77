#!/usr/bin/env python3
"""Benchmark of the paged, prefix-reused attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--secondary 3,4,5] [--no-cpu-baseline]

A step is one paged_attn_decode call over the decode batch: 64 sequences x 1 query
token, 32 query / 8 KV heads, head dim 128, bf16 K/V in a shuffled 16-token block pool,
contexts log-uniform in [4,000, 142,000], sequences in 8 sessions whose first 90% of
blocks are shared (same physical blocks).  Inputs are resident in HBM before timing.

Prints one JSON line.  `value` is decode KV throughput in GB/s counting each sequence's
context (logical bytes: 4,096 B per token over the 8 KV heads, K+V, bf16).  The
roofline object uses the algorithmic HBM bytes (each distinct KV block once, plus q and
out) per launch over the decode kernel's average duration, timed with HIP events on the
launch stream.  `cpu_baseline` times the CPU oracle (oracle/) on a bounded sample of the
same batch.  `secondary` holds the other workloads (suffix prefill, MLA MTP3 decode,
indexer + top-k + sparse MLA) when requested.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import resource
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged attn: decode KV GB/s, prefill TFLOP/s, tokens/s; % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA
FP8_PEAK_TFLOPS = 5000.0
DECODE_SOURCES = ["paged_prefix_cached_amd/csrc/decode_gqa.hip", "paged_prefix_cached_amd/csrc/pa_device.h",
                  "paged_prefix_cached_amd/csrc/pa_internal.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _cpu_rusage():
    r = resource.getrusage(resource.RUSAGE_SELF)
    return r.ru_utime + r.ru_stime


def timed_steps(step, steps, warmup, kernel=None):
    """Run warmup + timed steps; returns (wall ms per step, avg ms of `kernel` launches)."""
    import torch
    import paged_prefix_cached_amd as pa
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    pa.pa_profile_enable(64 * max(1, steps))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    recs = pa.pa_profile_records()
    pa.pa_profile_disable()
    per_kernel = {}
    for name, ms in recs:
        per_kernel.setdefault(name, []).append(ms)
    avg = {k: float(np.mean(v)) for k, v in per_kernel.items()}
    return (t1 - t0) * 1e3 / steps, avg


def measured_traffic(counters_file: str, sources: list[str]):
    """HBM bytes per launch from a committed rocprofv3 counter summary (FETCH_SIZE and
    WRITE_SIZE, scaled by a copy-kernel calibration), or None when the summary is absent
    or was taken on different kernel sources (sha256 over `sources`)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", counters_file)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    for src in sources:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if fields.get("source_sha256") != h.hexdigest():
        return None
    return float(fields["traffic_bytes_per_launch"])


# --------------------------------------------------------------------------- decode (headline)
def decode_bytes(wl):
    """(unique KV bytes, logical KV bytes, q+out bytes) of a paged GQA decode batch."""
    per_tok = wl.num_kv_heads * wl.head_dim * 2 * 2
    logical = int(wl.total_len.astype(np.int64).sum()) * per_tok
    # distinct (physical block, valid rows): a shared block is read once
    seen = {}
    for s in range(wl.num_seqs):
        L = int(wl.total_len[s])
        nb = -(-L // 16)
        for j in range(nb):
            b = int(wl.block_table[s, j])
            rows = min(16, L - 16 * j)
            seen[b] = max(seen.get(b, 0), rows)
    unique = sum(seen.values()) * per_tok
    qo = wl.q.size * 2 * 2
    return unique, logical, qo


def bench_decode(args, dev_name, share=True):
    import torch
    import paged_prefix_cached_amd as pa
    import workloads as W
    from workloads.device import GqaOnDevice
    t = time.time()
    wl = W.make_gqa_decode(2, share=share)
    dev = GqaOnDevice(wl)
    log(f"[bench] decode workload ready in {time.time() - t:.1f}s")
    S, H, D = wl.num_seqs, wl.num_q_heads, wl.head_dim
    q = dev.q.view(S, 1, H, D)
    out = torch.empty((S, 1, H, D), dtype=torch.bfloat16, device="cuda")
    nws = pa.load().paged_attn_decode_workspace_size(S, 1, H, dev.max_total, pa.ctypes.byref(dev.pool))
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")

    def step():
        pa.paged_attn_decode(q, dev.pool, dev.bt, dev.total_len, q_per_seq=1, num_q_heads=H,
                             max_context_len=dev.max_total, scale=wl.scale, out=out, workspace=ws)

    ms, kern = timed_steps(step, args.steps, args.warmup)
    unique, logical, qo = decode_bytes(wl)
    k_ms = kern.get("decode_gqa", float("nan"))
    algo = unique + qo
    res = {
        "ms_per_step": ms,
        "value": logical / (ms * 1e-3) / 1e9,
        "unique_kv_gbps": unique / (ms * 1e-3) / 1e9,
        "tokens_per_s": S / (ms * 1e-3),
        "kernel_ms": kern,
        "roofline": {"bound": "hbm", "achieved": algo / (k_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": algo / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "traffic": measured_traffic("gqa_decode_kernel.hbm-counters.decode-64seq.txt", DECODE_SOURCES)
                     if share else None,
                     "kernel": "gqa_decode_kernel",
                     "bytes_per_launch": algo,
                     "per_unit": "4096 B per distinct cached token (8 KV heads x 128 x K,V x bf16) + q,out"},
        "config": {"workload": "paged GQA decode: 64 seqs x 1 query token, 32q/8kv heads, d128, bf16, "
                               "block 16, contexts log-uniform 4K-142K, 8 sessions sharing 90% of blocks",
                   "num_seqs": S, "q_heads": H, "kv_heads": wl.num_kv_heads, "head_dim": D, "block_size": 16,
                   "context_mean": float(wl.total_len.mean()), "context_median": float(np.median(wl.total_len)),
                   "unique_kv_bytes": unique, "logical_kv_bytes": logical, "device": dev_name},
    }
    return res, wl


def cpu_baseline(wl, budget_s: float):
    """Time the CPU oracle on the first sequences of the decode batch (bounded)."""
    import oracle
    per_tok = wl.num_kv_heads * wl.head_dim * 2 * 2
    done_bytes, n = 0, 0
    c0, t0 = _cpu_rusage(), time.perf_counter()
    order = list(range(wl.num_seqs))
    for s in order:
        oracle.paged_gqa_attention(wl, s)
        done_bytes += int(wl.total_len[s]) * per_tok
        n += 1
        if time.perf_counter() - t0 > budget_s:
            break
    wall = time.perf_counter() - t0
    cpu = _cpu_rusage() - c0
    return {"value": done_bytes / wall / 1e9, "unit": "GB/s", "cores": max(1, int(round(cpu / wall))),
            "kind": "oracle",
            "sample": f"first {n} of {wl.num_seqs} decode sequences ({done_bytes / 4096:.0f} context tokens), "
                      f"{wall:.1f} s wall, {cpu:.1f} s CPU",
            "host_threads_available": len(os.sched_getaffinity(0))}


# --------------------------------------------------------------------------- secondary workloads
def bench_prefill(steps, warmup):
    import torch
    import paged_prefix_cached_amd as pa
    import workloads as W
    from workloads.device import GqaOnDevice
    t = time.time()
    wl = W.make_prefix_prefill(3)
    dev = GqaOnDevice(wl)
    del wl.k_pool, wl.v_pool
    log(f"[bench] prefill workload ready in {time.time() - t:.1f}s")
    out = torch.empty((wl.q.shape[0], wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")

    def step():
        pa.paged_attn_prefill(dev.q, dev.pool, dev.bt, dev.cached, dev.n_new, dev.q_start,
                              num_q_heads=wl.num_q_heads, max_new_len=dev.max_new,
                              max_total_len=dev.max_total, scale=wl.scale, out=out)

    ms, kern = timed_steps(step, steps, warmup)
    pairs = sum(int(c) * int(n) + int(n) * (int(n) + 1) // 2
                for c, n in zip(wl.total_len - wl.n_new, wl.n_new))
    flops = pairs * wl.num_q_heads * 4 * wl.head_dim
    k_ms = kern.get("prefill_gqa", float("nan"))
    return {"workload": "prefix-cached suffix prefill: 8 seqs x (142000 cached + 2048 new), 32q/8kv, d128, bf16",
            "ms": ms, "tflops": flops / (ms * 1e-3) / 1e12, "tokens_per_s": wl.q.shape[0] / (ms * 1e-3),
            "kernel_ms": kern, "flop": flops,
            "roofline": {"bound": "mfma", "achieved": flops / (k_ms * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": flops / (k_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}}


def _bench_gqa_prefill_workload(wl, label, steps, warmup):
    """Time paged_attn_prefill on a generated GQA workload; MFMA roofline on the causal
    (query, visible key) pairs: 4 d FLOP each per query head."""
    import torch
    import paged_prefix_cached_amd as pa
    from workloads.device import GqaOnDevice
    dev = GqaOnDevice(wl)
    del wl.k_pool, wl.v_pool
    out = torch.empty((wl.q.shape[0], wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")

    def step():
        pa.paged_attn_prefill(dev.q, dev.pool, dev.bt, dev.cached, dev.n_new, dev.q_start,
                              num_q_heads=wl.num_q_heads, max_new_len=dev.max_new,
                              max_total_len=dev.max_total, scale=wl.scale, out=out)

    ms, kern = timed_steps(step, steps, warmup)
    pairs = sum(int(c) * int(n) + int(n) * (int(n) + 1) // 2
                for c, n in zip(wl.total_len - wl.n_new, wl.n_new))
    flops = pairs * wl.num_q_heads * 4 * wl.head_dim
    k_ms = kern.get("prefill_gqa", float("nan"))
    return {"workload": label, "ms": ms, "tflops": flops / (ms * 1e-3) / 1e12,
            "tokens_per_s": wl.q.shape[0] / (ms * 1e-3), "kernel_ms": kern, "flop": flops,
            "roofline": {"bound": "mfma", "achieved": flops / (k_ms * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": flops / (k_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}}


def bench_cold(steps, warmup):
    import workloads as W
    t = time.time()
    wl = W.make_cold_prefill(7)
    log(f"[bench] cold-prompt workload ready in {time.time() - t:.1f}s")
    return _bench_gqa_prefill_workload(
        wl, "cold-prompt prefill: 4 seqs x 32768 new tokens (nothing cached), 32q/8kv, d128, bf16", steps, warmup)


def bench_chunked(steps, warmup):
    """One step of the chunked-prefill scheduler, the way an engine issues it: one
    paged_attn_prefill call for the requests that advance by a prefill chunk and one
    paged_attn_decode call for the requests that add a single token."""
    import torch
    import paged_prefix_cached_amd as pa
    import workloads as W
    from workloads.device import t as to_dev
    t = time.time()
    wl = W.make_chunked_mixed(8)
    log(f"[bench] chunked-step workload ready in {time.time() - t:.1f}s")
    nc = int((wl.n_new > 1).sum())                       # chunked requests come first
    S = wl.num_seqs
    kd, vd = to_dev(wl.k_pool, "cuda"), to_dev(wl.v_pool, "cuda")
    del wl.k_pool, wl.v_pool
    pool = pa.gqa_pool(kd, vd)
    bt = to_dev(wl.block_table, "cuda")
    q = to_dev(wl.q, "cuda")
    cached = (wl.total_len - wl.n_new).astype(np.int32)
    p_bt, p_cached = bt[:nc], to_dev(cached[:nc], "cuda")
    p_new, p_qs = to_dev(wl.n_new[:nc].astype(np.int32), "cuda"), to_dev(wl.q_start[:nc + 1].astype(np.int32), "cuda")
    n_pq = int(wl.q_start[nc])
    d_bt, d_ctx = bt[nc:], to_dev(wl.total_len[nc:].astype(np.int32), "cuda")
    d_q = q[n_pq:].view(S - nc, 1, wl.num_q_heads, wl.head_dim)
    max_new, max_total = int(wl.n_new[:nc].max()), int(wl.total_len[:nc].max())
    max_ctx = int(wl.total_len[nc:].max())
    out_p = torch.empty((n_pq, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    out_d = torch.empty((S - nc, 1, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    nws = pa.load().paged_attn_decode_workspace_size(S - nc, 1, wl.num_q_heads, max_ctx, pa.ctypes.byref(pool))
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")

    def step():
        pa.paged_attn_prefill(q[:n_pq], pool, p_bt, p_cached, p_new, p_qs, num_q_heads=wl.num_q_heads,
                              max_new_len=max_new, max_total_len=max_total, scale=wl.scale, out=out_p)
        pa.paged_attn_decode(d_q, pool, d_bt, d_ctx, q_per_seq=1, num_q_heads=wl.num_q_heads,
                             max_context_len=max_ctx, scale=wl.scale, out=out_d, workspace=ws)

    ms, kern = timed_steps(step, steps, warmup)
    pairs = sum(int(c) * int(n) + int(n) * (int(n) + 1) // 2 for c, n in zip(cached[:nc], wl.n_new[:nc]))
    flops = pairs * wl.num_q_heads * 4 * wl.head_dim
    kv_bytes = int(wl.total_len[nc:].astype(np.int64).sum()) * wl.num_kv_heads * wl.head_dim * 4
    k_ms = kern.get("prefill_gqa", float("nan"))
    return {"workload": "chunked-prefill step: 4 x 512-token chunks (prefill call) + 60 decode tokens "
                        "(decode call), contexts log-uniform 4K-142K, 32q/8kv, d128, bf16",
            "ms": ms, "tokens_per_s": wl.q.shape[0] / (ms * 1e-3), "kernel_ms": kern, "flop": flops,
            "decode_kv_bytes": kv_bytes,
            "decode_kv_gbps": kv_bytes / (kern.get("decode_gqa", float("nan")) * 1e-3) / 1e9,
            "roofline": {"bound": "mfma", "achieved": flops / (k_ms * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": flops / (k_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                         "kernel": "gqa_prefill_kernel"}}


def bench_mla(steps, warmup):
    import torch
    import paged_prefix_cached_amd as pa
    import workloads as W
    from workloads.device import MlaOnDevice
    t = time.time()
    mla = W.make_mla_decode(4)
    dev = MlaOnDevice(mla)
    log(f"[bench] MLA workload ready in {time.time() - t:.1f}s")
    S, T, H = mla.num_seqs, 4, mla.num_q_heads
    q = dev.q.view(S, T, H, 576)
    out = torch.empty((S, T, H, 512), dtype=torch.bfloat16, device="cuda")
    nws = pa.load().paged_attn_decode_workspace_size(S, T, H, dev.max_total, pa.ctypes.byref(dev.pool))
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")

    def step():
        pa.paged_attn_decode(q, dev.pool, dev.bt, dev.total_len, q_per_seq=T, num_q_heads=H,
                             max_context_len=dev.max_total, scale=mla.scale, out=out, workspace=ws)

    ms, kern = timed_steps(step, steps, warmup)
    L = mla.total_len.astype(np.int64)
    pairs = int(sum(4 * l - 6 for l in L))            # sum_j (L - 4 + j + 1), j = 0..3
    flops = pairs * H * 2 * (576 + 512)
    kv_bytes = int(L.sum()) * 580
    k_ms = kern.get("decode_mla", float("nan"))
    return {"workload": "MLA latent decode MTP3: 64 seqs x 4 tokens, 64 heads, FP8 latent 512+64, "
                        "contexts U[32768, 262144], block 64",
            "ms": ms, "tflops": flops / (ms * 1e-3) / 1e12, "kv_gbps": kv_bytes / (ms * 1e-3) / 1e9,
            "tokens_per_s": S * T / (ms * 1e-3), "kernel_ms": kern, "flop": flops, "kv_bytes": kv_bytes,
            "roofline": {"bound": "mfma", "achieved": flops / (k_ms * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": flops / (k_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}}


def bench_sparse(steps, warmup):
    import torch
    import paged_prefix_cached_amd as pa
    import workloads as W
    from workloads.device import MlaOnDevice
    t = time.time()
    mla, idx = W.make_sparse_mla(5)
    dev = MlaOnDevice(mla, idx)
    log(f"[bench] sparse workload ready in {time.time() - t:.1f}s")
    n_q, k = dev.q_idx.shape[0], 2048
    topk = torch.empty((n_q, k), dtype=torch.int32, device="cuda")
    nws = pa.load().mla_indexer_topk_workspace_size(n_q, 64, dev.max_total, k)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    out = torch.empty((n_q, 64, 512), dtype=torch.bfloat16, device="cuda")

    def step():
        pa.mla_indexer_topk(dev.q_idx, dev.w, dev.idx_pool, dev.bt, dev.cached, dev.n_new, dev.q_start,
                            max_new_len=dev.max_new, max_total_len=dev.max_total, k=k, topk_idx=topk,
                            workspace=ws)
        pa.sparse_mla_attn(dev.q, dev.pool, dev.bt, dev.q_seq, topk, scale=mla.scale, out=out)

    ms, kern = timed_steps(step, steps, warmup)
    cached = int(mla.total_len[0] - mla.n_new[0])
    pairs = sum(cached + i + 1 for i in range(n_q))
    idx_flops = pairs * 64 * 128 * 2
    sp_flops = n_q * k * 64 * 2 * (576 + 512)
    out = {"workload": "indexer (64 heads x 128, FP8 keys) + top-2048 + sparse MLA (64 heads, FP8 latent): "
                       "1 seq, 131072 cached + 4096 new",
           "ms": ms, "tokens_per_s": n_q / (ms * 1e-3), "kernel_ms": kern,
           "indexer_tflops": idx_flops / (kern.get("indexer", float("nan")) * 1e-3) / 1e12,
           "sparse_mla_tflops": sp_flops / (kern.get("sparse_mla", float("nan")) * 1e-3) / 1e12,
           "flop": idx_flops + sp_flops}
    out["roofline"] = {"bound": "mfma", "achieved": out["indexer_tflops"], "peak": BF16_PEAK_TFLOPS,
                       "unit": "TFLOP/s", "frac": out["indexer_tflops"] / BF16_PEAK_TFLOPS,
                       "kernel": "indexer_kernel"}
    return out


def bench_append(steps, warmup):
    """paged_kv_append on the three workloads' new tokens, into pools of their full size:
    the suffix prefill (8 x 2048 rows of 8 KV heads x 128, bf16 K and V), the MLA MTP3
    decode step (64 x 4 latent rows) and the sparse-MLA prefill (4096 latent rows plus
    4096 indexer-key rows), the FP8 rows quantised per token.  Algorithmic bytes: input
    rows read once, pool rows (and scales) written once."""
    import torch
    import paged_prefix_cached_amd as pa
    import workloads as W
    from workloads.device import t as to_dev
    g = torch.Generator(device="cuda")
    g.manual_seed(80)

    def layout(seed, cached, new, bs):
        a = W.make_append(seed, cached=cached, new=new, block_size=bs, row_shape=(1,), with_v=False)
        return a, [to_dev(x, "cuda") for x in (a.block_table, a.cached_len, a.new_len, a.q_start)]

    def rows(n, *shape):
        return torch.randn((n,) + shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)

    a3, d3 = layout(81, [142000] * 8, [2048] * 8, 16)
    kp = torch.empty((a3.num_blocks, 8, 16, 128), dtype=torch.bfloat16, device="cuda")
    vp = torch.empty_like(kp)
    gqa = pa.gqa_pool(kp, vp)
    k3, v3 = rows(16384, 8, 128), rows(16384, 8, 128)
    ctx = np.random.default_rng(82).integers(32768, 262145, 64)
    a4, d4 = layout(82, ctx - 4, [4] * 64, 64)
    p4 = torch.empty((a4.num_blocks, 64, 576), dtype=torch.uint8, device="cuda")
    s4 = torch.empty((a4.num_blocks, 64), dtype=torch.float32, device="cuda")
    mla4 = pa.mla_pool(p4, s4)
    x4 = rows(256, 576)
    a5, d5 = layout(83, [131072], [4096], 64)
    p5 = torch.empty((a5.num_blocks, 64, 576), dtype=torch.uint8, device="cuda")
    s5 = torch.empty((a5.num_blocks, 64), dtype=torch.float32, device="cuda")
    i5 = torch.empty((a5.num_blocks, 64, 128), dtype=torch.uint8, device="cuda")
    is5 = torch.empty((a5.num_blocks, 64), dtype=torch.float32, device="cuda")
    mla5, idx5 = pa.mla_pool(p5, s5), pa.indexer_pool(i5, is5)
    x5, xi5 = rows(4096, 576), rows(4096, 128)
    torch.cuda.synchronize()

    def step():
        pa.paged_kv_append(gqa, *d3, k3, v3, max_new_len=2048)
        pa.paged_kv_append(mla4, *d4, x4, max_new_len=4)
        pa.paged_kv_append(mla5, *d5, x5, max_new_len=4096)
        pa.paged_kv_append(idx5, *d5, xi5, max_new_len=4096)

    ms, kern = timed_steps(step, steps, warmup)
    gqa_bytes = 2 * (16384 * 8 * 128 * 2 * 2)
    fp8_bytes = 256 * (576 * 3 + 4) + 4096 * (576 * 3 + 4) + 4096 * (128 * 3 + 4)
    k_ms = kern.get("append_gqa", float("nan"))
    ach = gqa_bytes / (k_ms * 1e-3) / 1e9
    return {"workload": "KV append: 8 x 2048 bf16 rows (8 KV heads x 128) + 64 x 4 and 4096 FP8 latent "
                        "rows (576) + 4096 FP8 indexer rows (128), per-token quantisation",
            "ms": ms, "kernel_ms": kern, "bytes": gqa_bytes + fp8_bytes,
            "gbps": (gqa_bytes + fp8_bytes) / (ms * 1e-3) / 1e9,
            "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": ach / HBM_PEAK_GBS, "kernel": "append_gqa_kernel"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--secondary", default="", help="comma list of extra workloads: 2n (decode with no "
                                                    "shared blocks), 3 (prefill), 4 (MLA MTP3 decode), "
                                                    "5 (indexer + sparse MLA), a (KV append), c (cold-prompt prefill), "
                                                    "m (chunked-prefill step)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one 1 GiB device-to-device copy (reference kernel for HBM counters)")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle time")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the paged-attention kernels "
                                   "are single-device; multi-GPU context splitting is not built"}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    import paged_prefix_cached_amd as pa
    pa.load()
    dev_name = torch.cuda.get_device_name(0)
    if args.calibrate_copy:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    res, wl = bench_decode(args, dev_name)
    line = {"metric": METRIC, "value": res["value"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": res["config"], "tokens_per_s": res["tokens_per_s"],
            "unique_kv_gbps": res["unique_kv_gbps"], "kernel_ms": res["kernel_ms"], "roofline": res["roofline"]}
    if args.secondary:
        sec = {}
        for c in [x.strip() for x in args.secondary.split(",") if x.strip()]:
            if c == "2n":   # control: the same decode batch with no shared blocks
                r, _ = bench_decode(args, dev_name, share=False)
                sec["decode_no_sharing"] = {k: r[k] for k in ("ms_per_step", "value", "unique_kv_gbps",
                                                              "tokens_per_s", "kernel_ms", "roofline")}
                continue
            f = {"3": ("prefill_suffix", bench_prefill), "4": ("mla_decode_mtp3", bench_mla),
                 "5": ("indexer_topk_sparse_mla", bench_sparse), "a": ("kv_append", bench_append),
                 "c": ("cold_prompt_prefill", bench_cold), "m": ("chunked_prefill_step", bench_chunked)}[c]
            sec[f[0]] = f[1](max(2, args.steps // 4), max(1, args.warmup // 2))
            torch.cuda.empty_cache()
        line["secondary"] = sec
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
        line["cpu_baseline"]["unit"] = "GB/s"
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
