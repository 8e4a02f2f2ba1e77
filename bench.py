#!/usr/bin/env python3
"""Benchmark of the paged, prefix-reused attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--secondary 2n,3,4,5,5p] [--no-cpu-baseline]

A step is one paged_attn_decode call over the decode batch: 64 sequences x 1 query
token, 32 query / 8 KV heads, head dim 128, bf16 K/V in a shuffled 16-token block pool,
contexts log-uniform in [4,000, 142,000], sequences in 8 sessions whose first 90% of
blocks are shared (same physical blocks).  Inputs are resident in HBM before timing.

Timing: W untimed warm-up steps, then K timed steps; before every step a 1 GiB
device-to-device copy followed by a read of another 1 GiB evicts L2 and the MALL (so reuse
within a call counts, reuse across calls does not, and no dirty flush data is written back
inside the timed step), and HIP events on the launch stream time each step alone.  ms_per_step
is the median step; the minimum and mean are reported beside it, and the library's own
events time each kernel launch.

Prints one JSON line.  `value` is the step's algorithmic HBM throughput: the bytes the
method must move (every distinct KV block once, 4,096 B per token over the 8 KV heads,
K+V, bf16, plus q and out) over the median step time.  `effective_kv_gbps` counts each
sequence's whole context instead (shared prefix blocks once per sequence).  The roofline
object uses the same algorithmic bytes over the decode kernel's average launch time.
`cpu_baseline` times the CPU oracle (oracle/) on the same batch with a process pool over
the sequences, one single-threaded process per host core.  `secondary` holds the other
workloads (by default: the same decode batch with no shared blocks as a control, suffix
prefill, MLA MTP3 decode, indexer + top-k + sparse MLA on separate pools and on the packed
per-block layout with MXFP4 index keys).
"""
from __future__ import annotations

import argparse
import json
import math
import os
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
_HDRS = ["paged_prefix_cached_amd/csrc/pa_device.h", "paged_prefix_cached_amd/csrc/pa_internal.h"]
PREFILL_SOURCES = ["paged_prefix_cached_amd/csrc/prefill_gqa.hip"] + _HDRS
MLA_SOURCES = ["paged_prefix_cached_amd/csrc/mla.hip"] + _HDRS
INDEXER_SOURCES = ["paged_prefix_cached_amd/csrc/indexer.hip"] + _HDRS
TOPK_SOURCES = ["paged_prefix_cached_amd/csrc/topk.hip"] + _HDRS
SPARSE_PROFILE = "indexer_topk_sparse_mla.131072+4096.txt"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


_FLUSH = []


def _flush():
    """Evict L2 and the MALL (256 MB) between timed steps, on the launch stream, outside the
    timed events: overwrite 1 GiB (a device copy), then read another 1 GiB, so the caches
    hold only clean lines of unrelated data and the timed kernel neither hits on its own
    previous data nor pays for writing back the flush's dirty lines."""
    import torch
    if not _FLUSH:
        _FLUSH.append(torch.ones(1 << 30, dtype=torch.uint8, device="cuda"))
        _FLUSH.append(torch.empty(1 << 30, dtype=torch.uint8, device="cuda"))
        _FLUSH.append(torch.ones(1 << 28, dtype=torch.float32, device="cuda"))
    _FLUSH[1].copy_(_FLUSH[0])
    _FLUSH[2].sum()


def _per_kernel(recs):
    per_kernel = {}
    for name, ms in recs:
        per_kernel.setdefault(name, []).append(ms)
    return {k: {"mean": float(np.mean(v)), "median": float(np.median(v)), "min": float(np.min(v)), "n": len(v)}
            for k, v in per_kernel.items()}


def timed_steps(step, steps, warmup, only=None):
    """W warm-up steps, then `steps` timed steps, each after a cache flush.  Returns a dict:
    median / min / mean ms per step (HIP events around each step on the launch stream),
    wall ms per step including the flushes, and per-kernel launch times (ms) recorded by
    the library's own events: {name: {"mean", "median", "min", "n"}}.
    With `only`, the library brackets only that kernel's launches inside the timed steps
    (each event record costs the stream a few microseconds, which would otherwise count in
    a short step's time); the other kernels' times then come from a second, separate pass
    of `steps` instrumented steps, listed under "breakdown_pass"."""
    import torch
    import paged_prefix_cached_amd as pa
    for _ in range(warmup):
        _flush()
        step()
    torch.cuda.synchronize()
    pa.pa_profile_enable(64 * max(1, steps))
    if only:
        pa.pa_profile_select(only)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        _flush()
        ev[i][0].record()
        step()
        ev[i][1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    per_step = np.array([a.elapsed_time(b) for a, b in ev])
    kern = _per_kernel(pa.pa_profile_records())
    pa.pa_profile_disable()
    breakdown = []
    if only:
        pa.pa_profile_enable(64 * max(1, steps))
        for _ in range(steps):
            _flush()
            step()
        torch.cuda.synchronize()
        rest = _per_kernel(pa.pa_profile_records())
        pa.pa_profile_disable()
        for k, v in rest.items():
            if k not in kern:
                kern[k] = v
                breakdown.append(k)
    return {"ms": float(np.median(per_step)), "ms_min": float(per_step.min()), "ms_mean": float(per_step.mean()),
            "wall_ms_incl_flush": (t1 - t0) * 1e3 / steps, "kernels": kern, "breakdown_pass": breakdown}


def _kmean(t, name):
    return t["kernels"].get(name, {}).get("mean", float("nan"))


def _kms(t):
    return {k: v["mean"] for k, v in t["kernels"].items()}


# Sustained dense-GEMM rate on this device (vendor library, random operands), measured once
# per run: under full matrix-core load with random data the engine clock drops well below
# its peak, so this -- not the published peak -- is the rate a kernel can actually reach.
GEMM_CEILING = {}


def gemm_ceiling(n=8192, reps=10):
    """TFLOP/s of torch.matmul (hipBLASLt) on random n x n fp16 and bf16 operands."""
    import torch
    out = {}
    for name, dt in (("fp16", torch.float16), ("bf16", torch.bfloat16)):
        g = torch.Generator(device="cuda").manual_seed(7)
        a = torch.randn(n, n, device="cuda", dtype=dt, generator=g)
        b = torch.randn(n, n, device="cuda", dtype=dt, generator=g)
        for _ in range(3):
            torch.matmul(a, b)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.matmul(a, b)
        e1.record()
        torch.cuda.synchronize()
        out[name] = 2.0 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12
        del a, b
    return out


# The FP8 products of the MLA and indexer kernels take each bf16 query as two E4M3 terms:
# twice the FP8 flops at twice the fp16 rate, so their useful-flop peak is the bf16/fp16 one.
SPLIT_PEAK_NOTE = ("Q.K on the FP8 MFMA with the bf16 query as two E4M3 terms (2x the FP8 flops at 2x the "
                   "bf16 rate): the useful-flop peak is the bf16/fp16 dense peak")


def _mfma_roof(flops, k_ms, kernel, per_unit, peak=None, dtype="fp16", peak_note=None):
    peak = BF16_PEAK_TFLOPS if peak is None else peak
    ach = flops / (k_ms * 1e-3) / 1e12
    r = {"bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s", "frac": ach / peak,
         "traffic": None, "kernel": kernel, "flop_per_launch": flops, "per_unit": per_unit}
    if peak_note:
        r["peak_note"] = peak_note
    if dtype in GEMM_CEILING:
        r["sustained_gemm_tflops"] = GEMM_CEILING[dtype]
        r["frac_of_sustained_gemm"] = ach / GEMM_CEILING[dtype]
    return r


def measured_traffic(counters_file: str, sources: list[str], section: str | None = None):
    """HBM bytes per launch from a committed rocprofv3 counter summary (FETCH_SIZE and
    WRITE_SIZE, scaled by a copy-kernel calibration), or None when the summary is absent
    or was taken on different kernel sources (sha256 over `sources`).  `section` selects the
    block whose "[...]" title starts with it, in summaries that cover several kernels."""
    import hashlib
    path = os.path.join(ROOT, "profiles", counters_file)
    if not os.path.exists(path):
        return None
    fields = {}
    inside = section is None
    for line in open(path):
        if line.startswith("["):
            if section is not None:
                inside = line[1:].startswith(section)
            continue
        if inside and ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip().split()[0] if v.strip() else ""
    h = hashlib.sha256()
    for src in sources:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if fields.get("source_sha256") != h.hexdigest():
        return None
    return float(fields["traffic_bytes_per_launch"]) if "traffic_bytes_per_launch" in fields else None


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


def bench_decode(args, dev_name, wl=None, share=True):
    import torch
    import paged_prefix_cached_amd as pa
    import workloads as W
    from workloads.device import GqaOnDevice
    t = time.time()
    if wl is None:
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

    tm = timed_steps(step, args.steps, args.warmup, only="decode_gqa")
    unique, logical, qo = decode_bytes(wl)
    ms = tm["ms"]
    k_ms = _kmean(tm, "decode_gqa")
    algo = unique + qo
    res = {
        "ms_per_step": ms,
        "ms_per_step_min": tm["ms_min"],
        "ms_per_step_mean": tm["ms_mean"],
        "wall_ms_per_step_incl_flush": tm["wall_ms_incl_flush"],
        "value": algo / (ms * 1e-3) / 1e9,
        "effective_kv_gbps": logical / (ms * 1e-3) / 1e9,
        "tokens_per_s": S / (ms * 1e-3),
        "kernel_ms": _kms(tm),
        "kernel_ms_median": {k: v["median"] for k, v in tm["kernels"].items()},
        "kernel_ms_from_breakdown_pass": tm["breakdown_pass"],
        "workspace_bytes": nws,
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


# ---- CPU oracle baseline: a process pool over the decode sequences (forked before the
# GPU is touched, so the workers hold no device state); each worker single-threaded.
_CPU_WL = None


def _cpu_one(s):
    import oracle
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        oracle.paged_gqa_attention(_CPU_WL, s)
    return s


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, budget_s: float):
    """Time the CPU oracle on the decode batch: one process per host core, each taking
    whole sequences as they finish, stopped once `budget_s` of wall time has passed.  The rate
    counts the sample's distinct KV bytes (shared blocks once), like the GPU's value."""
    import multiprocessing as mp
    global _CPU_WL
    _CPU_WL = wl
    ncores = len(os.sched_getaffinity(0))
    per_tok = wl.num_kv_heads * wl.head_dim * 2 * 2
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    done = []
    with ctx.Pool(ncores) as pool:
        for s in pool.imap_unordered(_cpu_one, range(wl.num_seqs)):
            done.append(s)
            if time.perf_counter() - t0 > budget_s:
                pool.terminate()
                break
    wall = time.perf_counter() - t0
    seen = {}
    for s in done:
        L = int(wl.total_len[s])
        for j in range(-(-L // 16)):
            b = int(wl.block_table[s, j])
            seen[b] = max(seen.get(b, 0), min(16, L - 16 * j))
    distinct = sum(seen.values()) * per_tok + len(done) * wl.num_q_heads * wl.head_dim * 4
    logical = int(sum(int(wl.total_len[s]) for s in done)) * per_tok
    return {"value": distinct / wall / 1e9, "unit": "GB/s", "cores": ncores, "kind": "oracle",
            "sample": f"{len(done)} of {wl.num_seqs} decode sequences ({logical // per_tok} context tokens, "
                      f"{distinct / 1e9:.2f} GB distinct), {wall:.1f} s wall on {ncores} single-threaded "
                      f"fp64 numpy processes",
            "effective_kv_gbps": logical / wall / 1e9, "cpu_model": _cpu_model()}


# --------------------------------------------------------------------------- secondary workloads
def _prefill_flops(wl):
    pairs = sum(int(c) * int(n) + int(n) * (int(n) + 1) // 2
                for c, n in zip(wl.total_len - wl.n_new, wl.n_new))
    return pairs * wl.num_q_heads * 4 * wl.head_dim


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

    tm = timed_steps(step, steps, warmup)
    flops = _prefill_flops(wl)
    ms = tm["ms"]
    return {"workload": label, "ms": ms, "ms_min": tm["ms_min"], "tflops": flops / (ms * 1e-3) / 1e12,
            "tokens_per_s": wl.q.shape[0] / (ms * 1e-3), "kernel_ms": _kms(tm), "flop": flops,
            "roofline": _mfma_roof(flops, _kmean(tm, "prefill_gqa"), "gqa_prefill_kernel",
                                   "4 x 128 FLOP per (query head, visible key)", dtype="bf16")}


def bench_prefill(steps, warmup):
    import workloads as W
    t = time.time()
    wl = W.make_prefix_prefill(3)
    log(f"[bench] prefill workload ready in {time.time() - t:.1f}s")
    r = _bench_gqa_prefill_workload(
        wl, "prefix-cached suffix prefill: 8 seqs x (142000 cached + 2048 new), 32q/8kv, d128, bf16", steps, warmup)
    r["roofline"]["traffic"] = measured_traffic("gqa_prefill_kernel.suffix-prefill-8x142000+2048.txt",
                                                PREFILL_SOURCES, section="gqa_prefill_kernel")
    return r


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

    tm = timed_steps(step, steps, warmup)
    pairs = sum(int(c) * int(n) + int(n) * (int(n) + 1) // 2 for c, n in zip(cached[:nc], wl.n_new[:nc]))
    flops = pairs * wl.num_q_heads * 4 * wl.head_dim
    kv_bytes = int(wl.total_len[nc:].astype(np.int64).sum()) * wl.num_kv_heads * wl.head_dim * 4
    ms = tm["ms"]
    return {"workload": "chunked-prefill step: 4 x 512-token chunks (prefill call) + 60 decode tokens "
                        "(decode call), contexts log-uniform 4K-142K, 32q/8kv, d128, bf16",
            "ms": ms, "ms_min": tm["ms_min"], "tokens_per_s": wl.q.shape[0] / (ms * 1e-3), "kernel_ms": _kms(tm),
            "flop": flops, "decode_kv_bytes": kv_bytes,
            "decode_kv_gbps": kv_bytes / (_kmean(tm, "decode_gqa") * 1e-3) / 1e9,
            "roofline": _mfma_roof(flops, _kmean(tm, "prefill_gqa"), "gqa_prefill_kernel",
                                   "4 x 128 FLOP per (query head, visible key)", dtype="bf16")}


def bench_mla(steps, warmup):
    import torch
    import paged_prefix_cached_amd as pa
    import workloads as W
    from workloads.device import MlaOnDevice
    t = time.time()
    mla = W.make_mla_decode(4)
    dev = MlaOnDevice(mla)
    del mla.kv_pool, mla.kv_scale
    log(f"[bench] MLA workload ready in {time.time() - t:.1f}s")
    S, T, H = mla.num_seqs, 4, mla.num_q_heads
    q = dev.q.view(S, T, H, 576)
    out = torch.empty((S, T, H, 512), dtype=torch.bfloat16, device="cuda")
    nws = pa.load().paged_attn_decode_workspace_size(S, T, H, dev.max_total, pa.ctypes.byref(dev.pool))
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")

    def step():
        pa.paged_attn_decode(q, dev.pool, dev.bt, dev.total_len, q_per_seq=T, num_q_heads=H,
                             max_context_len=dev.max_total, scale=mla.scale, out=out, workspace=ws)

    tm = timed_steps(step, steps, warmup)
    L = mla.total_len.astype(np.int64)
    pairs = int(sum(4 * l - 6 for l in L))            # sum_j (L - 4 + j + 1), j = 0..3
    flops = pairs * H * 2 * (576 + 512)
    kv_bytes = int(L.sum()) * 580
    ms = tm["ms"]
    k_ms = _kmean(tm, "decode_mla")
    roof = _mfma_roof(flops, k_ms, "mla_kernel (decode)", "2 x (576 + 512) FLOP per (query row, visible key)",
                      peak_note=SPLIT_PEAK_NOTE)
    roof["traffic"] = measured_traffic("mla_kernel.mla-mtp3-decode-64seq-ctx32k-256k.txt", MLA_SOURCES,
                                       section="mla_kernel<false")
    roof["hbm_frac"] = kv_bytes / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBS
    return {"workload": "MLA latent decode MTP3: 64 seqs x 4 tokens, 64 heads, FP8 latent 512+64, "
                        "contexts U[32768, 262144], block 64",
            "ms": ms, "ms_min": tm["ms_min"], "tflops": flops / (ms * 1e-3) / 1e12,
            "kv_gbps": kv_bytes / (ms * 1e-3) / 1e9,
            "tokens_per_s": S * T / (ms * 1e-3), "kernel_ms": _kms(tm), "flop": flops, "kv_bytes": kv_bytes,
            "roofline": roof}


def bench_sparse(steps, warmup, packed=False):
    """Indexer + top-2,048 + sparse MLA at 131,072 + 4,096 tokens.  packed: the packed
    per-block layout (one allocation per 64-token block: FP8 latent + scales + MXFP4 index
    keys + E8M0 scales), the indexer reading the MXFP4 keys and sparse MLA the latent view."""
    import torch
    import paged_prefix_cached_amd as pa
    import workloads as W
    from workloads.device import MlaOnDevice, t as to_dev
    t = time.time()
    mla, idx = W.make_sparse_mla(5, fp4_keys=packed)
    dev = MlaOnDevice(mla, idx)
    lat_pool, idx_pool = dev.pool, dev.idx_pool
    if packed:
        blocks = to_dev(W.pack_mla_blocks(mla, idx), "cuda")
        lat_pool, idx_pool = pa.packed_mla_pools(blocks)
    log(f"[bench] sparse workload ready in {time.time() - t:.1f}s")
    n_q, k = dev.q_idx.shape[0], 2048
    topk = torch.empty((n_q, k), dtype=torch.int32, device="cuda")
    nws = pa.load().mla_indexer_topk_workspace_size(n_q, 64, dev.max_total, k)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    out = torch.empty((n_q, 64, 512), dtype=torch.bfloat16, device="cuda")

    def step():
        pa.mla_indexer_topk(dev.q_idx, dev.w, idx_pool, dev.bt, dev.cached, dev.n_new, dev.q_start,
                            max_new_len=dev.max_new, max_total_len=dev.max_total, k=k, topk_idx=topk,
                            workspace=ws)
        pa.sparse_mla_attn(dev.q, lat_pool, dev.bt, dev.q_seq, topk, scale=mla.scale, out=out)

    tm = timed_steps(step, steps, warmup)
    cached = int(mla.total_len[0] - mla.n_new[0])
    pairs = sum(cached + i + 1 for i in range(n_q))
    idx_flops = pairs * 64 * 128 * 2
    sp_flops = n_q * k * 64 * 2 * (576 + 512)
    topk_bytes = pairs * 4 + n_q * k * 4              # the valid scores read once, indices written
    ms = tm["ms"]
    k_top = _kmean(tm, "topk")
    roofs = {
        "indexer": _mfma_roof(idx_flops, _kmean(tm, "indexer"), "indexer_kernel",
                              "2 x 128 FLOP per (query, indexer head, visible key)", dtype="bf16",
                              peak_note=SPLIT_PEAK_NOTE),
        "topk": {"bound": "hbm", "achieved": topk_bytes / (k_top * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                 "unit": "GB/s", "frac": topk_bytes / (k_top * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": None,
                 "kernel": "topk_kernel", "bytes_per_launch": topk_bytes,
                 "per_unit": "4 B per valid score (read once) + 4 B per selected index"},
        "sparse_mla": _mfma_roof(sp_flops, _kmean(tm, "sparse_mla"), "mla_kernel (sparse)",
                                 "2 x (576 + 512) FLOP per (query row, selected key)", peak_note=SPLIT_PEAK_NOTE),
    }
    # counter traffic from the committed summary, while the kernels' sources are unchanged
    tag = "MXFP4 keys, packed layout" if packed else "FP8 keys"
    roofs["indexer"]["traffic"] = measured_traffic(SPARSE_PROFILE, INDEXER_SOURCES, section=f"indexer_kernel<4> ({tag})")
    roofs["topk"]["traffic"] = measured_traffic(SPARSE_PROFILE, TOPK_SOURCES, section=f"topk_kernel ({tag} run)")
    roofs["sparse_mla"]["traffic"] = measured_traffic(SPARSE_PROFILE, MLA_SOURCES,
                                                      section=f"mla_kernel<true, 2, 4, true> (sparse, {tag} run)")
    L = int(mla.total_len[0])
    kv_per_token = 576 + 4 + (64 + 4 if packed else 128 + 4)
    return {"workload": ("packed per-block layout: MXFP4 indexer keys" if packed else "indexer (FP8 keys)")
                        + " (64 heads x 128) + top-2048 + sparse MLA (64 heads, FP8 latent): 1 seq, "
                        "131072 cached + 4096 new",
            "kv_bytes_per_token": kv_per_token, "kv_bytes": kv_per_token * L,
            "ms": ms, "ms_min": tm["ms_min"], "tokens_per_s": n_q / (ms * 1e-3), "kernel_ms": _kms(tm),
            "indexer_tflops": roofs["indexer"]["achieved"], "sparse_mla_tflops": roofs["sparse_mla"]["achieved"],
            "flop": idx_flops + sp_flops, "roofline": roofs["indexer"], "rooflines": roofs}


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
    # the same rows into the packed per-block layout: latent view and MXFP4 index view
    blocks5 = torch.empty((a5.num_blocks, W.PACKED_BLOCK_BYTES), dtype=torch.uint8, device="cuda")
    lat5p, idx5p = pa.packed_mla_pools(blocks5)
    torch.cuda.synchronize()

    def step():
        pa.paged_kv_append(gqa, *d3, k3, v3, max_new_len=2048)
        pa.paged_kv_append(mla4, *d4, x4, max_new_len=4)
        pa.paged_kv_append(mla5, *d5, x5, max_new_len=4096)
        pa.paged_kv_append(idx5, *d5, xi5, max_new_len=4096)
        pa.paged_kv_append(lat5p, *d5, x5, max_new_len=4096)
        pa.paged_kv_append(idx5p, *d5, xi5, max_new_len=4096)

    tm = timed_steps(step, steps, warmup)
    ms = tm["ms"]
    gqa_bytes = 2 * (16384 * 8 * 128 * 2 * 2)
    fp8_bytes = 256 * (576 * 3 + 4) + 2 * 4096 * (576 * 3 + 4) + 4096 * (128 * 3 + 4)
    fp4_bytes = 4096 * (128 * 2 + 64 + 4)        # bf16 row read, 64 code bytes + 4 E8M0 codes written
    k_ms = _kmean(tm, "append_gqa")
    ach = gqa_bytes / (k_ms * 1e-3) / 1e9
    return {"workload": "KV append: 8 x 2048 bf16 rows (8 KV heads x 128) + 64 x 4 and 4096 FP8 latent "
                        "rows (576) + 4096 FP8 indexer rows (128), per-token quantisation; the 4096 latent "
                        "and indexer rows again into the packed layout (FP8 latent, MXFP4 index keys)",
            "ms": ms, "kernel_ms": _kms(tm), "bytes": gqa_bytes + fp8_bytes + fp4_bytes,
            "gbps": (gqa_bytes + fp8_bytes + fp4_bytes) / (ms * 1e-3) / 1e9,
            "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": ach / HBM_PEAK_GBS, "kernel": "append_gqa_kernel"}}


def _clocks():
    """Current engine / memory clock levels as the driver reports them (best effort)."""
    out = {}
    for name in ("pp_dpm_sclk", "pp_dpm_mclk"):
        for card in sorted(os.listdir("/sys/class/drm")) if os.path.isdir("/sys/class/drm") else []:
            path = f"/sys/class/drm/{card}/device/{name}"
            try:
                cur = [l.strip() for l in open(path) if l.strip().endswith("*")]
            except OSError:
                continue
            if cur:
                out[name[7:]] = cur[0]
                break
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--secondary", default="2n,3,4,5,5p",
                    help="comma list of extra workloads (default 2n,3,4,5,5p; '' for none): 2n (decode with no "
                         "shared blocks), 3 (suffix prefill), 4 (MLA MTP3 decode), 5 (indexer + top-k + "
                         "sparse MLA), 5p (the same on the packed layout with MXFP4 index keys), a (KV append), "
                         "c (cold-prompt prefill), m (chunked-prefill step)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one 1 GiB device-to-device copy (reference kernel for HBM counters)")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle wall time")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the paged-attention kernels "
                                   "are single-device; multi-GPU context splitting is not built"}))
        sys.exit(2)
    import workloads as W
    t = time.time()
    wl = W.make_gqa_decode(2)
    log(f"[bench] decode batch generated in {time.time() - t:.1f}s")
    cpu = None
    if not args.no_cpu_baseline:       # before the GPU is touched: the workers are plain forks
        cpu = cpu_baseline(wl, args.cpu_budget)
        log(f"[bench] cpu baseline: {cpu['sample']}")
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
    res, wl = bench_decode(args, dev_name, wl=wl)
    log(f"[bench] decode: {res['ms_per_step']:.4f} ms/step, kernel {res['kernel_ms'].get('decode_gqa', 0):.4f} ms")
    line = {"metric": METRIC, "value": res["value"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": res["config"]}
    for k in ("ms_per_step_min", "ms_per_step_mean", "wall_ms_per_step_incl_flush", "effective_kv_gbps",
              "tokens_per_s", "kernel_ms", "kernel_ms_median", "kernel_ms_from_breakdown_pass",
              "workspace_bytes", "roofline"):
        line[k] = res[k]
    line["clocks"] = _clocks()
    if args.secondary:
        GEMM_CEILING.update(gemm_ceiling())
        line["sustained_gemm_tflops"] = dict(GEMM_CEILING)
        log(f"[bench] sustained GEMM rate: {GEMM_CEILING}")
        sec = {}
        for c in [x.strip() for x in args.secondary.split(",") if x.strip()]:
            if c == "2n":   # control: the same decode batch with no shared blocks
                r, _ = bench_decode(args, dev_name, share=False)
                sec["decode_no_sharing"] = {k: r[k] for k in ("ms_per_step", "value", "effective_kv_gbps",
                                                              "tokens_per_s", "kernel_ms", "roofline")}
                continue
            f = {"3": ("prefill_suffix", bench_prefill), "4": ("mla_decode_mtp3", bench_mla),
                 "5": ("indexer_topk_sparse_mla", bench_sparse),
                 "5p": ("packed_fp4_indexer_topk_sparse_mla", lambda st, wu: bench_sparse(st, wu, packed=True)),
                 "a": ("kv_append", bench_append),
                 "c": ("cold_prompt_prefill", bench_cold), "m": ("chunked_prefill_step", bench_chunked)}[c]
            sec[f[0]] = f[1](max(3, args.steps // 4), max(1, args.warmup // 2))
            log(f"[bench] {f[0]}: {sec[f[0]]['ms']:.3f} ms")
            torch.cuda.empty_cache()
        line["secondary"] = sec
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
