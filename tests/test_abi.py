"""C-ABI checks that need no GPU: the library loads, exports every function that
include/pa.h declares, and rejects invalid arguments before launching anything."""
import ctypes
import os
import re

import pytest

import paged_prefix_cached_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "pa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:pa_status|size_t|const char\*|int32_t)\s+(\w+)\s*\(", src, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pa.LIB_PATH):
        from paged_prefix_cached_amd import build
        build.build()
    return pa.load()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(pa.EXPORTED)


def test_status_strings(lib):
    assert lib.pa_status_string(0) == b"PA_OK"
    assert lib.pa_status_string(3) == b"PA_ERR_WORKSPACE"
    assert lib.pa_version() >= 1


FAKE = 0x10000          # 16-byte-aligned non-null address; never dereferenced (validation fails first)


def _gqa_pool(**kw):
    d = dict(num_blocks=64, block_size=16, num_kv_heads=8, head_dim_qk=64, head_dim_v=64, kv_dtype=1,
             k=FAKE, v=FAKE, scale=None)
    d.update(kw)
    return pa.KVPool(**d)


def _prefill(lib, pool, **kw):
    a = dict(q=FAKE, bt=FAKE, stride=16, cached=FAKE, new=FAKE, qs=FAKE, S=1, Hq=8, max_new=16,
             max_total=256, scale=0.125, out=FAKE)
    a.update(kw)
    return lib.paged_attn_prefill(a["q"], ctypes.byref(pool), a["bt"], a["stride"], a["cached"], a["new"],
                                  a["qs"], a["S"], a["Hq"], a["max_new"], a["max_total"], a["scale"],
                                  a["out"], None, None, 0, None)


@pytest.mark.parametrize("kw,pool_kw,code", [
    (dict(q=None), {}, 1),
    (dict(out=None), {}, 1),
    (dict(q=FAKE + 4), {}, 1),                 # misaligned
    (dict(Hq=12), {}, 1),                      # not a multiple of num_kv_heads
    (dict(Hq=8 * 16), {}, 2),                  # group size 16 unsupported
    (dict(stride=4), {}, 1),                   # table too short for max_total_len
    (dict(scale=0.0), {}, 1),
    (dict(scale=float("nan")), {}, 1),
    ({}, dict(head_dim_qk=96, head_dim_v=96), 2),
    ({}, dict(block_size=32), 2),
    ({}, dict(k=None), 1),
    ({}, dict(kv_dtype=2), 2),
])
def test_prefill_rejects(lib, kw, pool_kw, code):
    assert _prefill(lib, _gqa_pool(**pool_kw), **kw) == code
    assert lib.pa_last_error_detail()


def test_prefill_empty_batch_is_ok(lib):
    assert _prefill(lib, _gqa_pool(), S=0) == 0


def _decode(lib, pool, ws=None, wsb=0, **kw):
    a = dict(q=FAKE, bt=FAKE, stride=9000, ctx=FAKE, S=64, T=1, Hq=32, max_ctx=142000, scale=0.088, out=FAKE)
    a.update(kw)
    return lib.paged_attn_decode(a["q"], ctypes.byref(pool), a["bt"], a["stride"], a["ctx"], a["S"], a["T"],
                                 a["Hq"], a["max_ctx"], a["scale"], a["out"], None, ws, wsb, None)


def test_decode_validation(lib):
    pool = _gqa_pool(head_dim_qk=128, head_dim_v=128)
    need = lib.paged_attn_decode_workspace_size(64, 1, 32, 142000, ctypes.byref(pool))
    # pass-balanced decode: partials for every (group, workgroup) piece -- 8 groups of 8
    # sequences, plus one per workgroup boundary (a workgroup per compute unit; 256 when no
    # device is visible) -- per KV head, 32 rows of (128 + 1) floats, plus the pass lists
    # (16 B per (member, 32-key tile) slot of each of the 8 x ceil(142000 / 8192) regions).
    regions = 8 * -(-142000 // 8192)
    partials = (8 + 256 - 1) * 8 * 32 * 129 * 4
    passes = regions * 256 * 8 * 16
    assert partials + passes <= need <= partials + passes + 64 * 1024
    assert need <= lib.paged_attn_decode_noalloc_max_bytes()        # the benchmark batch fits
    assert _decode(lib, pool) == 3                                  # no workspace
    assert _decode(lib, pool, ws=FAKE, wsb=need - 1) == 3           # too small
    assert _decode(lib, pool, T=5) == 2                             # q_per_seq > 4
    assert _decode(lib, pool, T=4, Hq=64) == 2                      # 4 x 8 rows > 16
    assert _decode(lib, pool, ctx=None) == 1
    assert _decode(lib, pool, S=0, ws=None) == 0
    mla = pa.KVPool(100, 64, 1, 576, 512, 2, FAKE, None, FAKE)
    assert _decode(lib, mla, T=4, Hq=64, stride=4096, max_ctx=262144) == 3
    assert _decode(lib, mla, T=4, Hq=40, stride=4096, max_ctx=262144) == 2
    bad = pa.KVPool(100, 64, 1, 576, 512, 2, FAKE, None, None)      # FP8 pool without scales
    assert _decode(lib, bad, T=4, Hq=64, stride=4096, max_ctx=262144) == 1


def test_indexer_and_sparse_validation(lib):
    ip = pa.KVPool(100, 64, 1, 128, 0, 2, FAKE, None, FAKE)
    args = [FAKE, FAKE, ctypes.byref(ip), FAKE, 2200, FAKE, FAKE, FAKE, 1, 4096, 64, 4096, 135168]
    assert lib.mla_indexer_topk(*args, 2048, FAKE, None, None, 0, None) == 3
    assert lib.mla_indexer_topk(*args, 0, FAKE, None, None, 0, None) == 2
    assert lib.mla_indexer_topk(*args[:10], 40, *args[11:], 2048, FAKE, None, None, 0, None) == 2
    mp = pa.KVPool(100, 64, 1, 576, 512, 2, FAKE, None, FAKE)
    assert lib.sparse_mla_attn(FAKE, ctypes.byref(mp), FAKE, 10, FAKE, FAKE, 0, 2048, 64, 0.04, FAKE, None,
                               None, 0, None) == 0            # valid, empty batch: nothing launched
    assert lib.sparse_mla_attn(FAKE, ctypes.byref(mp), FAKE, 10, FAKE, FAKE, 4, 2048, 96, 0.04, FAKE, None,
                               None, 0, None) == 2
    assert lib.sparse_mla_attn(FAKE, ctypes.byref(mp), FAKE, 10, FAKE, None, 4, 2048, 64, 0.04, FAKE, None,
                               None, 0, None) == 1


def test_fp8_pool_rows_fit_int32(lib):
    """The MLA kernels address FP8 pool rows (block * 64 + offset) in 32 bits."""
    big = pa.KVPool(2**31 // 64, 64, 1, 576, 512, 2, FAKE, None, FAKE)
    assert lib.sparse_mla_attn(FAKE, ctypes.byref(big), FAKE, 10, FAKE, FAKE, 4, 2048, 64, 0.04, FAKE, None,
                               None, 0, None) == 2
    ok = pa.KVPool(2**31 // 64 - 1, 64, 1, 576, 512, 2, FAKE, None, FAKE)
    assert lib.sparse_mla_attn(FAKE, ctypes.byref(ok), FAKE, 10, FAKE, FAKE, 0, 2048, 64, 0.04, FAKE, None,
                               None, 0, None) == 0


def test_decode_noalloc_rejects_oversized_calls_before_launch(lib):
    """The allocation-free decode checks its scratch need on the host: sizes whose
    workspace exceeds PA_NOALLOC_SCRATCH_BYTES fail with PA_ERR_WORKSPACE before any HIP
    call (fake device pointers are never touched)."""
    pool = _gqa_pool(head_dim_qk=128, head_dim_v=128)
    big = 4_000_000
    need = lib.paged_attn_decode_workspace_size(64, 1, 32, big, ctypes.byref(pool))
    assert need > lib.paged_attn_decode_noalloc_max_bytes() == 64 << 20
    st = lib.paged_attn_decode_noalloc(FAKE, ctypes.byref(pool), FAKE, big // 16, FAKE, 64, 1, 32, big, 0.088,
                                       FAKE, None, None)
    assert st == 3, lib.pa_last_error_detail()
    assert b"scratch" in lib.pa_last_error_detail()
    # invalid shapes are still reported as such, not as a scratch shortage
    assert lib.paged_attn_decode_noalloc(FAKE, ctypes.byref(pool), FAKE, 16, FAKE, 1, 5, 32, 256, 0.088, FAKE,
                                         None, None) == 2
