"""Python binding of libpa.so, the gfx950 paged-attention library.

Argument marshalling only: every step of the computation runs in the HIP kernels behind
the C ABI declared in include/pa.h.  torch provides device memory and the current HIP
stream.  There is no CPU or Python fallback: if the library is missing or a call fails,
an exception is raised.

Functions (same names as the C entry points):
    paged_attn_prefill, paged_attn_decode, mla_indexer_topk, sparse_mla_attn,
    paged_kv_append
Pool descriptors:
    gqa_pool(k_pool, v_pool), mla_pool(kv_pool, kv_scale), indexer_pool(keys, scale),
    packed_mla_pools(blocks) (latent and index views of the packed per-block layout)
Test hooks:
    pa_test_gather_kv, pa_test_topk_from_scores
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["load", "PAError", "KVPool", "gqa_pool", "mla_pool", "indexer_pool", "packed_mla_pools",
           "paged_attn_prefill", "paged_attn_decode", "paged_attn_decode_noalloc", "mla_indexer_topk",
           "sparse_mla_attn",
           "paged_kv_append", "pa_test_gather_kv", "pa_test_topk_from_scores", "pa_profile_enable",
           "pa_profile_select", "pa_profile_records", "pa_profile_disable", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")
PA_BF16, PA_FP8_E4M3, PA_PACKED_MLA = 1, 2, 3
_lib = None

_c_i32, _c_sz, _vp, _c_f = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float


class PAError(RuntimeError):
    pass


class KVPool(ctypes.Structure):
    _fields_ = [("num_blocks", _c_i32), ("block_size", _c_i32), ("num_kv_heads", _c_i32),
                ("head_dim_qk", _c_i32), ("head_dim_v", _c_i32), ("kv_dtype", _c_i32),
                ("k", _vp), ("v", _vp), ("scale", _vp)]


_SIGS = {
    "pa_status_string": (ctypes.c_char_p, [_c_i32]),
    "pa_last_error_detail": (ctypes.c_char_p, []),
    "pa_version": (_c_i32, []),
    "paged_attn_prefill_workspace_size": (_c_sz, [_c_i32, _c_i32, _c_i32, _c_i32, _vp]),
    "paged_attn_prefill": (_c_i32, [_vp, _vp, _vp, _c_i32, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32,
                                    _c_i32, _c_f, _vp, _vp, _vp, _c_sz, _vp]),
    "paged_attn_decode_workspace_size": (_c_sz, [_c_i32, _c_i32, _c_i32, _c_i32, _vp]),
    "paged_attn_decode": (_c_i32, [_vp, _vp, _vp, _c_i32, _vp, _c_i32, _c_i32, _c_i32, _c_i32,
                                   _c_f, _vp, _vp, _vp, _c_sz, _vp]),
    "paged_attn_decode_noalloc_max_bytes": (_c_sz, []),
    "paged_attn_decode_noalloc": (_c_i32, [_vp, _vp, _vp, _c_i32, _vp, _c_i32, _c_i32, _c_i32, _c_i32,
                                           _c_f, _vp, _vp, _vp]),
    "mla_indexer_topk_workspace_size": (_c_sz, [_c_i32, _c_i32, _c_i32, _c_i32]),
    "mla_indexer_topk": (_c_i32, [_vp, _vp, _vp, _vp, _c_i32, _vp, _vp, _vp, _c_i32, _c_i32,
                                  _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _vp, _c_sz, _vp]),
    "sparse_mla_attn_workspace_size": (_c_sz, [_c_i32, _c_i32, _c_i32]),
    "sparse_mla_attn": (_c_i32, [_vp, _vp, _vp, _c_i32, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_f,
                                 _vp, _vp, _vp, _c_sz, _vp]),
    "paged_kv_append": (_c_i32, [_vp, _vp, _c_i32, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _vp,
                                 _vp, _vp]),
    "pa_test_gather_kv": (_c_i32, [_vp, _vp, _c_i32, _c_i32, _c_i32, _vp, _vp, _vp, _vp]),
    "pa_test_topk_workspace_size": (_c_sz, [_c_i32, _c_i32]),
    "pa_test_topk_from_scores": (_c_i32, [_vp, _vp, _c_i32, _c_i32, _c_i32, _vp, _vp, _c_sz, _vp]),
    "pa_profile_enable": (_c_i32, [_c_i32]),
    "pa_profile_select": (_c_i32, [ctypes.c_char_p]),
    "pa_profile_count": (_c_i32, []),
    "pa_profile_record": (_c_i32, [_c_i32, ctypes.c_char_p, _c_i32, ctypes.POINTER(_c_f)]),
    "pa_profile_disable": (_c_i32, []),
}
EXPORTED = tuple(_SIGS)


def load(path: str | None = None):
    """Load libpa.so (built in-tree by paged_prefix_cached_amd.build).  Raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise PAError(f"{p} not found: build it with `python -m paged_prefix_cached_amd.build`")
    # torch ships its own HIP runtime; importing it first makes libpa.so bind to that one.
    # Loaded the other way round, the process would hold two HIP runtimes.
    import torch  # noqa: F401
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(st: int, what: str) -> None:
    if st != 0:
        lib = load()
        raise PAError(f"{what}: {lib.pa_status_string(st).decode()}: {lib.pa_last_error_detail().decode()}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ws(nbytes: int, like):
    import torch
    if nbytes == 0:
        return None
    return torch.empty(int(nbytes), dtype=torch.uint8, device=like.device)


def _bf16_out(shape, like):
    import torch
    return torch.empty(shape, dtype=torch.bfloat16, device=like.device)


# --------------------------------------------------------------------------- pools
def gqa_pool(k_pool, v_pool) -> KVPool:
    """bf16 pools [num_blocks][num_kv_heads][16][head_dim] (any 2-byte dtype)."""
    nb, hkv, bs, d = k_pool.shape
    assert v_pool.shape == k_pool.shape and k_pool.element_size() == 2
    pool = KVPool(nb, bs, hkv, d, d, PA_BF16, k_pool.data_ptr(), v_pool.data_ptr(), None)
    pool._keep = (k_pool, v_pool)
    return pool


def mla_pool(kv_pool, kv_scale) -> KVPool:
    """FP8 latent pool [num_blocks][64][576] (uint8) with fp32 scales [num_blocks][64]."""
    nb, bs, d = kv_pool.shape
    assert kv_pool.element_size() == 1 and tuple(kv_scale.shape) == (nb, bs)
    pool = KVPool(nb, bs, 1, d, 512, PA_FP8_E4M3, kv_pool.data_ptr(), None, kv_scale.data_ptr())
    pool._keep = (kv_pool, kv_scale)
    return pool


def indexer_pool(keys, scale) -> KVPool:
    """FP8 indexer keys [num_blocks][64][128] (uint8) with fp32 scales [num_blocks][64]."""
    nb, bs, d = keys.shape
    pool = KVPool(nb, bs, 1, d, 0, PA_FP8_E4M3, keys.data_ptr(), None, scale.data_ptr())
    pool._keep = (keys, scale)
    return pool


def packed_mla_pools(blocks):
    """The two views of a packed per-block pool [num_blocks][41472] (uint8): (latent view
    for decode / sparse MLA / latent append, index view for the indexer / key append)."""
    nb, nbytes = blocks.shape
    assert blocks.element_size() == 1 and nbytes == 41472
    lat = KVPool(nb, 64, 1, 576, 512, PA_PACKED_MLA, blocks.data_ptr(), None, None)
    idx = KVPool(nb, 64, 1, 128, 0, PA_PACKED_MLA, blocks.data_ptr(), None, None)
    lat._keep = idx._keep = (blocks,)
    return lat, idx


# --------------------------------------------------------------------------- calls
def paged_attn_prefill(q, pool: KVPool, block_table, cached_len, new_len, q_start, *,
                       num_q_heads: int, max_new_len: int, max_total_len: int, scale: float,
                       out=None, lse=None, workspace=None):
    lib = load()
    if out is None:
        out = _bf16_out((q.shape[0], num_q_heads, pool.head_dim_v), q)
    if workspace is None:
        nws = lib.paged_attn_prefill_workspace_size(block_table.shape[0], num_q_heads, max_new_len,
                                                    max_total_len, ctypes.byref(pool))
        workspace = _ws(nws, q)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.paged_attn_prefill(_p(q), ctypes.byref(pool), _p(block_table), block_table.shape[1],
                                  _p(cached_len), _p(new_len), _p(q_start), block_table.shape[0],
                                  num_q_heads, max_new_len, max_total_len, scale, _p(out), _p(lse),
                                  _p(workspace), nbytes, _stream(q)), "paged_attn_prefill")
    return out


def paged_attn_decode(q, pool: KVPool, block_table, context_len, *, q_per_seq: int,
                      num_q_heads: int, max_context_len: int, scale: float, out=None, lse=None,
                      workspace=None):
    """q [num_seqs][q_per_seq][num_q_heads][d_qk] -> out [num_seqs][q_per_seq][num_q_heads][d_v]."""
    lib = load()
    S = block_table.shape[0]
    if out is None:
        out = _bf16_out((S, q_per_seq, num_q_heads, pool.head_dim_v), q)
    nws = lib.paged_attn_decode_workspace_size(S, q_per_seq, num_q_heads, max_context_len,
                                               ctypes.byref(pool))
    if workspace is None:
        workspace = _ws(nws, q)
    _check(lib.paged_attn_decode(_p(q), ctypes.byref(pool), _p(block_table), block_table.shape[1],
                                 _p(context_len), S, q_per_seq, num_q_heads, max_context_len, scale,
                                 _p(out), _p(lse), _p(workspace),
                                 0 if workspace is None else workspace.numel() * workspace.element_size(),
                                 _stream(q)), "paged_attn_decode")
    return out


def paged_attn_decode_noalloc(q, pool: KVPool, block_table, context_len, *, q_per_seq: int,
                              num_q_heads: int, max_context_len: int, scale: float, out=None, lse=None):
    """paged_attn_decode on the library's own per-GPU scratch array (no workspace)."""
    lib = load()
    S = block_table.shape[0]
    if out is None:
        out = _bf16_out((S, q_per_seq, num_q_heads, pool.head_dim_v), q)
    _check(lib.paged_attn_decode_noalloc(_p(q), ctypes.byref(pool), _p(block_table), block_table.shape[1],
                                         _p(context_len), S, q_per_seq, num_q_heads, max_context_len, scale,
                                         _p(out), _p(lse), _stream(q)), "paged_attn_decode_noalloc")
    return out


def mla_indexer_topk(q_idx, w, idx_pool: KVPool, block_table, cached_len, new_len, q_start, *,
                     max_new_len: int, max_total_len: int, k: int, topk_idx=None,
                     scores_out=None, workspace=None):
    import torch
    lib = load()
    n_q, H, _ = q_idx.shape
    if topk_idx is None:
        topk_idx = torch.empty((n_q, k), dtype=torch.int32, device=q_idx.device)
    nws = lib.mla_indexer_topk_workspace_size(n_q, H, max_total_len, k)
    if workspace is None:
        workspace = _ws(nws, q_idx)
    _check(lib.mla_indexer_topk(_p(q_idx), _p(w), ctypes.byref(idx_pool), _p(block_table),
                                block_table.shape[1], _p(cached_len), _p(new_len), _p(q_start),
                                block_table.shape[0], n_q, H, max_new_len, max_total_len, k,
                                _p(topk_idx), _p(scores_out), _p(workspace),
                                0 if workspace is None else workspace.numel(), _stream(q_idx)),
           "mla_indexer_topk")
    return topk_idx


def sparse_mla_attn(q, pool: KVPool, block_table, q_seq, topk_idx, *, scale: float, out=None,
                    lse=None):
    lib = load()
    n_q, Hq, _ = q.shape
    k = topk_idx.shape[1]
    if out is None:
        out = _bf16_out((n_q, Hq, 512), q)
    _check(lib.sparse_mla_attn(_p(q), ctypes.byref(pool), _p(block_table), block_table.shape[1],
                               _p(q_seq), _p(topk_idx), n_q, k, Hq, scale, _p(out), _p(lse), None, 0,
                               _stream(q)), "sparse_mla_attn")
    return out


def paged_kv_append(pool: KVPool, block_table, cached_len, new_len, q_start, k_new, v_new=None,
                    *, max_new_len: int):
    """Write the new rows k_new (and v_new for a bf16 pool) into the pool in place.

    GQA: k_new, v_new [n_tokens][num_kv_heads][head_dim] bf16.  FP8 pools (MLA latent or
    indexer keys): k_new [n_tokens][head_dim_qk] bf16, quantised per token on the GPU; the
    pool's bytes and scales are updated."""
    lib = load()
    _check(lib.paged_kv_append(ctypes.byref(pool), _p(block_table), block_table.shape[1],
                               _p(cached_len), _p(new_len), _p(q_start), block_table.shape[0],
                               k_new.shape[0], max_new_len, _p(k_new), _p(v_new),
                               _stream(k_new)), "paged_kv_append")


def pa_profile_enable(max_records: int) -> None:
    _check(load().pa_profile_enable(max_records), "pa_profile_enable")


def pa_profile_select(name: str | None) -> None:
    """Record only launches of kernel `name` (None: every launch)."""
    _check(load().pa_profile_select(name.encode() if name else None), "pa_profile_select")


def pa_profile_records():
    """[(kernel name, milliseconds)] for every launch recorded since pa_profile_enable."""
    lib = load()
    out = []
    buf = ctypes.create_string_buffer(64)
    ms = _c_f()
    for i in range(lib.pa_profile_count()):
        _check(lib.pa_profile_record(i, buf, 64, ctypes.byref(ms)), "pa_profile_record")
        out.append((buf.value.decode(), float(ms.value)))
    return out


def pa_profile_disable() -> None:
    load().pa_profile_disable()


def pa_test_gather_kv(pool: KVPool, block_table, seq: int, n_tokens: int, k_out, v_out=None,
                      scale_out=None):
    lib = load()
    _check(lib.pa_test_gather_kv(ctypes.byref(pool), _p(block_table), block_table.shape[1], seq,
                                 n_tokens, _p(k_out), _p(v_out), _p(scale_out), _stream(k_out)),
           "pa_test_gather_kv")


def pa_test_topk_from_scores(scores, valid_len, k: int, out=None):
    import torch
    lib = load()
    n, stride = scores.shape
    if out is None:
        out = torch.empty((n, k), dtype=torch.int32, device=scores.device)
    _check(lib.pa_test_topk_from_scores(_p(scores), _p(valid_len), n, stride, k, _p(out), None, 0,
                                        _stream(scores)), "pa_test_topk_from_scores")
    return out
