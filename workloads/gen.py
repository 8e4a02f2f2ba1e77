"""Seeded synthetic workloads for paged, prefix-reused attention.

Shapes follow the workloads the pages describe (vLLM AgentX article, news.ainew.jp:
"Re-evaluating agentic workloads" gives the 142K median input, >96 % prefix-cache hits
and sub-agent forks; the GLM-5.3 report, aisoku.org, "What's new" gives the 64-head
shared latent KV, the 2,048-token indexer and MTP3; its table gives FP8 KV).  The data
are N(0,1) draws, not model activations: the AgentX traces are not available and are
never reconstructed.

Everything here is storage-format plumbing: random draws, bf16 / FP8-E4M3 rounding,
block pools, block tables.  No attention, score or top-k arithmetic lives here.

Layouts (all row-major, int32 indices; the packed per-block layout is at pack_mla_blocks):
  GQA pool   k_pool, v_pool : bf16 bits  uint16 [num_blocks][Hkv][16][d]
  MLA pool   kv_pool        : e4m3 bytes uint8  [num_blocks][64][576]  (0..511 latent = V)
             kv_scale       : float32           [num_blocks][64]
  Indexer    idx_pool       : e4m3 bytes uint8  [num_blocks][64][128]
             idx_scale      : float32           [num_blocks][64]
  block_table : int32 [num_seqs][max_blocks], -1 past the end of a sequence.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "BF16_NAN", "FP8_NAN", "bf16_bits", "bf16_bits_to_f32", "e4m3_encode",
    "fp8_quantize_tokens", "normal_f32", "PagedGQA", "PagedMLA", "IndexerInput",
    "make_prefill_tiny", "make_gqa_decode", "make_prefix_prefill", "make_mla_decode",
    "make_sparse_mla", "make_gqa", "tie_scores", "CONFIG_NAMES", "AppendInput", "make_append",
    "make_cold_prefill", "make_chunked_mixed", "mxfp4_quantize_tokens", "pack_mla_blocks",
    "PACKED_BLOCK_BYTES",
]

BF16_NAN = np.uint16(0x7FC0)
FP8_NAN = np.uint8(0x7F)
_GARBAGE_BF16 = 30000.0          # large finite values in the unused tail of a partial block
_POOL_SLACK = 0.05               # unreferenced (poisoned) blocks added to every pool

CONFIG_NAMES = {
    1: "tiny prefix-cached prefill (MHA 8x64, 240 cached + 16 new)",
    2: "paged GQA decode (64 seqs, 32q/8kv heads, d128, 8 sessions sharing 90% of blocks)",
    3: "prefix-cached suffix prefill (8 seqs x (142000 cached + 2048 new), 32q/8kv, d128)",
    4: "MLA latent decode with MTP3 (64 seqs x 4 tokens, 64 heads, FP8 latent 512+64)",
    5: "sparse MLA with indexer (131072 cached + 4096 new, top-2048)",
}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# --------------------------------------------------------------------------- formats
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even.  Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """float32 -> OCP FP8 E4M3FN codes (uint8): round to nearest even, saturate at 448.

    Normal codes carry a 3-bit mantissa with exponent bias 7; |y| < 2^-6 maps onto the
    subnormal grid m * 2^-9 (m = 0..8, where m = 8 is the smallest normal, code 0x08).
    NaN is never produced; finite inputs beyond 448 saturate to 0x7E / 0xFE.
    """
    y = np.asarray(y, dtype=np.float32)
    sign = (y.view(np.uint32) >> np.uint32(24)).astype(np.uint8) & np.uint8(0x80)
    a = np.abs(y)
    # subnormal range: exact scaling by 2^9 then round-half-even
    sub = np.rint(a * np.float32(512.0)).astype(np.int32)
    # normal range: RNE of the fp32 mantissa to 3 bits
    u = a.view(np.uint32)
    u = u + np.uint32(0x7FFFF) + ((u >> np.uint32(20)) & np.uint32(1))
    e = (u >> np.uint32(23)).astype(np.int32) - 127 + 7
    m = ((u >> np.uint32(20)) & np.uint32(7)).astype(np.int32)
    norm = (e << 3) | m
    norm = np.minimum(norm, 0x7E)                    # saturate (also catches e >= 16)
    code = np.where(a < np.float32(2.0 ** -6), sub, norm).astype(np.uint8)
    return code | sign


def fp8_quantize_tokens(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-token FP8 quantisation of x[..., D]: scale = amax/448, codes = e4m3(x/scale)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    codes = e4m3_encode(x / scale[..., None])
    return codes, scale


def mxfp4_quantize_tokens(x: np.ndarray, group: int = 32) -> tuple[np.ndarray, np.ndarray]:
    """MXFP4 storage of x[..., D]: per group of 32, E8M0 code e = floor(log2 amax) - 2 + 127
    (127 for an all-zero group, kept in [2, 252]), elements E2M1 of x / 2^(e-127) rounded to
    nearest, ties to even, saturating at 6; two elements a byte, element 2j in the low
    nibble.  Returns (packed [..., D/2] uint8, scale codes [..., D/32] uint8)."""
    x = np.asarray(x, dtype=np.float32)
    lead = x.shape[:-1]
    g = x.reshape(lead + (x.shape[-1] // group, group)).astype(np.float64)
    amax = np.max(np.abs(g), axis=-1)
    _, p = np.frexp(amax)
    e = np.where(amax > 0, np.clip(p - 1 - 2 + 127, 2, 252), 127).astype(np.int64)
    y = g / np.ldexp(1.0, e - 127)[..., None]
    a = np.abs(y)
    mag = ((a > 0.25).astype(np.uint8) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5)
           + (a > 5.0)).astype(np.uint8)
    code = (mag | np.where(np.signbit(y), np.uint8(8), np.uint8(0))).reshape(x.shape)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    return packed, e.astype(np.uint8)


def normal_f32(seed: int, stream: int, n: int, *, chunk: int = 1 << 22) -> np.ndarray:
    """n N(0,1) float32 draws, deterministic in (seed, stream) whatever the thread count.

    Chunk c draws from SeedSequence(seed, spawn_key=(stream, c)), so chunks can be filled
    in parallel.
    """
    out = np.empty(n, dtype=np.float32)
    nchunks = max(1, -(-n // chunk))

    def fill(c: int) -> None:
        lo, hi = c * chunk, min(n, (c + 1) * chunk)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(stream, c))))
        out[lo:hi] = g.standard_normal(hi - lo, dtype=np.float32)

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def _bf16_normal(seed: int, stream: int, shape, mult: float = 1.0) -> np.ndarray:
    x = normal_f32(seed, stream, int(np.prod(shape)))
    if mult != 1.0:
        x *= np.float32(mult)
    return _par_map(bf16_bits, x).reshape(shape)


def _par_map(fn, x: np.ndarray, *, chunk: int = 1 << 22) -> np.ndarray:
    """Apply an elementwise fn over a flat array in parallel chunks."""
    x = x.reshape(-1)
    if x.size <= chunk:
        return fn(x)
    parts = [x[i:i + chunk] for i in range(0, x.size, chunk)]
    with ThreadPoolExecutor(_threads()) as ex:
        return np.concatenate(list(ex.map(fn, parts)))


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(1000 + stream,))))


# --------------------------------------------------------------------------- GQA / MHA
@dataclass
class PagedGQA:
    """Paged bf16 K/V (block size 16) with a packed query batch.

    Sequence s has total_len[s] tokens in the pool (cached prefix + new tokens) and
    n_new[s] query tokens at logical positions total_len[s]-n_new[s] ... total_len[s]-1.
    Queries are packed: rows q_start[s] .. q_start[s+1]-1 of q belong to sequence s.
    """
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: float
    total_len: np.ndarray          # int32 [S]
    n_new: np.ndarray              # int32 [S]
    q_start: np.ndarray            # int32 [S+1]
    block_table: np.ndarray        # int32 [S][max_blocks]
    k_pool: np.ndarray             # uint16 [NB][Hkv][bs][d]
    v_pool: np.ndarray
    q: np.ndarray                  # uint16 [n_q][Hq][d]
    logical_blocks: list = field(default_factory=list)   # per seq: indices into content
    content_k: np.ndarray | None = None                    # uint16 [n_unique][Hkv][bs][d]
    content_v: np.ndarray | None = None
    name: str = ""

    @property
    def num_seqs(self) -> int:
        return int(self.total_len.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.k_pool.shape[0])

    def q_rows(self, s: int) -> np.ndarray:
        return self.q[self.q_start[s]:self.q_start[s + 1]]

    def q_pos(self, s: int) -> np.ndarray:
        n = int(self.n_new[s])
        return np.arange(int(self.total_len[s]) - n, int(self.total_len[s]), dtype=np.int64)

    def kv_contiguous(self, s: int) -> tuple[np.ndarray, np.ndarray]:
        """Logical K/V of sequence s as [L][Hkv][d] bf16 bits, built from the per-block
        content (not from the pool), so it is independent of the physical placement."""
        assert self.content_k is not None, "content not kept for this workload"
        L = int(self.total_len[s])
        ids = self.logical_blocks[s]
        k = self.content_k[ids].transpose(0, 2, 1, 3).reshape(-1, self.num_kv_heads, self.head_dim)[:L]
        v = self.content_v[ids].transpose(0, 2, 1, 3).reshape(-1, self.num_kv_heads, self.head_dim)[:L]
        return np.ascontiguousarray(k), np.ascontiguousarray(v)


def _place_blocks(rng, n_unique: int, slack: float) -> tuple[int, np.ndarray]:
    pool = max(n_unique + 1, int(math.ceil(n_unique * (1.0 + slack))))
    perm = rng.permutation(pool).astype(np.int64)
    return pool, perm[:n_unique]


def make_gqa(seed: int, *, lengths, n_new, num_q_heads: int, num_kv_heads: int, head_dim: int,
             shared_groups=None, shared_frac: float = 0.0, q_mult: float = 1.0,
             keep_content: bool = True, block_size: int = 16, scale: float | None = None,
             garbage_tails: bool = True, name: str = "", place_seed: int | None = None) -> PagedGQA:
    """General GQA/MHA paged workload.

    lengths[s]   total tokens of sequence s (prefix + new); n_new[s] query tokens.
    shared_groups: list of lists of sequence ids whose first floor(shared_frac*nblocks)
                 blocks are the same physical blocks with the same content (prefix reuse).
                 Members of one group must have equal length.
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    n_new = np.asarray(n_new, dtype=np.int64)
    S = lengths.shape[0]
    bs = block_size
    nb = -(-lengths // bs)
    # logical block content ids per sequence
    logical: list[list[int]] = [None] * S
    n_unique = 0
    if shared_groups is None:
        shared_groups = [[s] for s in range(S)]
    for grp in shared_groups:
        L0 = lengths[grp[0]]
        assert all(lengths[g] == L0 for g in grp), "members of a sharing group need equal lengths"
        nbg = int(nb[grp[0]])
        sh = int(math.floor(shared_frac * nbg)) if len(grp) > 1 else 0
        sh = min(sh, nbg - 1) if len(grp) > 1 else 0   # the block holding the query is private
        shared_ids = list(range(n_unique, n_unique + sh))
        n_unique += sh
        for g in grp:
            priv = list(range(n_unique, n_unique + nbg - sh))
            n_unique += nbg - sh
            logical[g] = shared_ids + priv
    rng_place = _rng(seed if place_seed is None else place_seed, 1)
    NB, phys = _place_blocks(rng_place, n_unique, _POOL_SLACK)
    Hkv, d = num_kv_heads, head_dim
    shape = (n_unique, Hkv, bs, d)
    ck = _bf16_normal(seed, 2, shape)
    cv = _bf16_normal(seed, 3, shape)
    if garbage_tails:
        g = _rng(seed, 4)
        for s in range(S):
            tail = int(nb[s] * bs - lengths[s])
            if tail:
                last = logical[s][-1]
                sgn = np.where(g.random((Hkv, tail, d)) < 0.5, -1.0, 1.0).astype(np.float32)
                ck[last, :, bs - tail:, :] = bf16_bits(sgn * _GARBAGE_BF16)
                cv[last, :, bs - tail:, :] = bf16_bits(-sgn * _GARBAGE_BF16)
    k_pool = np.full((NB, Hkv, bs, d), BF16_NAN, dtype=np.uint16)
    v_pool = np.full((NB, Hkv, bs, d), BF16_NAN, dtype=np.uint16)
    k_pool[phys] = ck
    v_pool[phys] = cv
    maxb = int(nb.max())
    bt = np.full((S, maxb), -1, dtype=np.int32)
    for s in range(S):
        bt[s, :nb[s]] = phys[np.asarray(logical[s], dtype=np.int64)]
    q_start = np.zeros(S + 1, dtype=np.int32)
    q_start[1:] = np.cumsum(n_new)
    q = _bf16_normal(seed, 5, (int(q_start[-1]), num_q_heads, d), q_mult)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    w = PagedGQA(num_q_heads, num_kv_heads, d, bs, float(scale), lengths.astype(np.int32),
                 n_new.astype(np.int32), q_start, bt, k_pool, v_pool, q, logical,
                 ck if keep_content else None, cv if keep_content else None, name)
    return w


def make_prefill_tiny(seed: int = 1) -> PagedGQA:
    """1 sequence, MHA 8 heads x 64, 240 cached tokens (15 blocks) + 16 new, 64-block pool.

    The 16 blocks are the first 16 entries of a seeded permutation of the 64 pool blocks.
    """
    rng = _rng(seed, 1)
    perm = rng.permutation(64)
    Hkv, d, bs = 8, 64, 16
    ck = _bf16_normal(seed, 2, (16, Hkv, bs, d))
    cv = _bf16_normal(seed, 3, (16, Hkv, bs, d))
    k_pool = np.full((64, Hkv, bs, d), BF16_NAN, dtype=np.uint16)
    v_pool = np.full((64, Hkv, bs, d), BF16_NAN, dtype=np.uint16)
    k_pool[perm[:16]] = ck
    v_pool[perm[:16]] = cv
    bt = perm[:16].astype(np.int32)[None, :]
    q = _bf16_normal(seed, 5, (16, 8, d))
    return PagedGQA(8, 8, d, bs, 1.0 / 8.0, np.array([256], np.int32), np.array([16], np.int32),
                    np.array([0, 16], np.int32), bt, k_pool, v_pool, q, [list(range(16))], ck, cv,
                    CONFIG_NAMES[1])


def session_lengths(seed: int, n_sessions: int, lo: float, hi: float) -> np.ndarray:
    rng = _rng(seed, 0)
    return np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), n_sessions))).astype(np.int64)


def make_gqa_decode(seed: int = 2, *, n_sessions: int = 8, members: int = 8, lo: float = 4000,
                    hi: float = 142000, shared_frac: float = 0.9, q_per_seq: int = 1,
                    num_q_heads: int = 32, num_kv_heads: int = 8, head_dim: int = 128,
                    share: bool = True, shuffle_batch: bool = False, q_mult: float = 1.0,
                    keep_content: bool = False) -> PagedGQA:
    """Decode batch of n_sessions*members sequences; members of a session share the
    first floor(shared_frac * nblocks) blocks (same physical ids and content).  Sequence i
    is in session i // members unless shuffle_batch permutes the batch order.
    context length includes the q_per_seq query tokens."""
    Ls = session_lengths(seed, n_sessions, lo, hi)
    S = n_sessions * members
    order = np.arange(S)
    if shuffle_batch:
        order = _rng(seed, 6).permutation(S)
    lengths = np.empty(S, dtype=np.int64)
    groups = []
    for sidx in range(n_sessions):
        members_ids = [int(order[sidx * members + m]) for m in range(members)]
        for g in members_ids:
            lengths[g] = Ls[sidx]
        if share:
            groups.append(members_ids)
        else:
            groups.extend([[g] for g in members_ids])
    return make_gqa(seed, lengths=lengths, n_new=np.full(S, q_per_seq), num_q_heads=num_q_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim, shared_groups=groups,
                    shared_frac=shared_frac, q_mult=q_mult, keep_content=keep_content,
                    name=CONFIG_NAMES[2])


def make_prefix_prefill(seed: int = 3, *, num_seqs: int = 8, cached: int = 142000, new: int = 2048,
                        num_q_heads: int = 32, num_kv_heads: int = 8, head_dim: int = 128,
                        q_mult: float = 1.0, keep_content: bool = False) -> PagedGQA:
    lengths = np.full(num_seqs, cached + new)
    return make_gqa(seed, lengths=lengths, n_new=np.full(num_seqs, new), num_q_heads=num_q_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim, q_mult=q_mult,
                    keep_content=keep_content, name=CONFIG_NAMES[3])


def make_cold_prefill(seed: int = 7, *, num_seqs: int = 4, new: int = 32768, num_q_heads: int = 32,
                      num_kv_heads: int = 8, head_dim: int = 128, keep_content: bool = False) -> PagedGQA:
    """Cold prompts: nothing cached, the whole prompt is new and causal over itself.  The
    vLLM AgentX article (news.ainew.jp), "Two-level scheduling", names the rare long fresh
    prefills that fill the prefix cache; the GLM-5.3 report (aisoku.org), "What's new",
    measures PCP on 32K prompts."""
    lengths = np.full(num_seqs, new)
    return make_gqa(seed, lengths=lengths, n_new=lengths, num_q_heads=num_q_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim, keep_content=keep_content,
                    name=f"cold prompt prefill ({num_seqs} x {new} new, no cached prefix)")


def make_chunked_mixed(seed: int = 8, *, n_chunked: int = 4, chunk: int = 512, n_decode: int = 60,
                       lo: float = 4000, hi: float = 142000, num_q_heads: int = 32,
                       num_kv_heads: int = 8, head_dim: int = 128,
                       keep_content: bool = False) -> PagedGQA:
    """One step of the chunked-prefill scheduler: the vLLM AgentX article, "Two-level
    scheduling" (resolving head-of-line blocking), caps one request's tokens per step at 512
    so that short turns share the step.  n_chunked requests advance by a chunk-token prefill
    chunk on top of what they hold; n_decode requests add one token.  Contexts are
    log-uniform in [lo, hi]."""
    rng = _rng(seed, 30)
    ctx = np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), n_chunked + n_decode))).astype(np.int64)
    lengths = np.concatenate([ctx[:n_chunked] + chunk, ctx[n_chunked:]])
    n_new = np.concatenate([np.full(n_chunked, chunk), np.ones(n_decode, np.int64)])
    return make_gqa(seed, lengths=lengths, n_new=n_new, num_q_heads=num_q_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim, keep_content=keep_content,
                    name=f"chunked-prefill step ({n_chunked} x {chunk}-token chunks + {n_decode} decode tokens)")


# --------------------------------------------------------------------------- MLA (FP8 latent)
MLA_D_QK = 576
MLA_D_V = 512
MLA_BLOCK = 64


@dataclass
class PagedMLA:
    """FP8 latent cache (one 576-wide latent per token shared by all query heads)."""
    num_q_heads: int
    block_size: int
    scale: float
    total_len: np.ndarray          # int32 [S]
    n_new: np.ndarray              # int32 [S] query tokens per sequence
    q_start: np.ndarray            # int32 [S+1]
    block_table: np.ndarray        # int32 [S][max_blocks]
    kv_pool: np.ndarray            # uint8 [NB][bs][576]
    kv_scale: np.ndarray           # float32 [NB][bs]
    q: np.ndarray                  # uint16 [n_q][Hq][576]
    logical_blocks: list = field(default_factory=list)
    content_kv: np.ndarray | None = None     # uint8 [n_unique][bs][576]
    content_scale: np.ndarray | None = None  # float32 [n_unique][bs]
    name: str = ""

    @property
    def num_seqs(self) -> int:
        return int(self.total_len.shape[0])

    def q_rows(self, s: int) -> np.ndarray:
        return self.q[self.q_start[s]:self.q_start[s + 1]]

    def q_pos(self, s: int) -> np.ndarray:
        n = int(self.n_new[s])
        return np.arange(int(self.total_len[s]) - n, int(self.total_len[s]), dtype=np.int64)

    def kv_contiguous(self, s: int) -> tuple[np.ndarray, np.ndarray]:
        assert self.content_kv is not None, "content not kept for this workload"
        L = int(self.total_len[s])
        ids = self.logical_blocks[s]
        return (np.ascontiguousarray(self.content_kv[ids].reshape(-1, MLA_D_QK)[:L]),
                np.ascontiguousarray(self.content_scale[ids].reshape(-1)[:L]))


def _fp8_tokens(seed: int, stream: int, n_tokens: int, dim: int, *, chunk_tokens: int = 1 << 15):
    """n_tokens N(0,1) vectors of width dim, FP8-quantised per token (threaded, chunked)."""
    codes = np.empty((n_tokens, dim), dtype=np.uint8)
    scales = np.empty(n_tokens, dtype=np.float32)
    nchunks = max(1, -(-n_tokens // chunk_tokens))

    def fill(c: int) -> None:
        lo, hi = c * chunk_tokens, min(n_tokens, (c + 1) * chunk_tokens)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(stream, c))))
        x = g.standard_normal((hi - lo, dim), dtype=np.float32)
        codes[lo:hi], scales[lo:hi] = fp8_quantize_tokens(x)

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return codes, scales


def _mxfp4_tokens(seed: int, stream: int, n_tokens: int, dim: int, *, chunk_tokens: int = 1 << 15):
    """n_tokens N(0,1) vectors of width dim (the same draws as _fp8_tokens for the same
    seed and stream), stored as MXFP4."""
    packed = np.empty((n_tokens, dim // 2), dtype=np.uint8)
    scales = np.empty((n_tokens, dim // 32), dtype=np.uint8)
    nchunks = max(1, -(-n_tokens // chunk_tokens))

    def fill(c: int) -> None:
        lo, hi = c * chunk_tokens, min(n_tokens, (c + 1) * chunk_tokens)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(stream, c))))
        x = g.standard_normal((hi - lo, dim), dtype=np.float32)
        packed[lo:hi], scales[lo:hi] = mxfp4_quantize_tokens(x)

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return packed, scales


def _paged_fp8(seed: int, stream: int, lengths, dim: int, bs: int, perm_stream: int,
               keep_content: bool):
    """Private (unshared) FP8 token pool for the given sequence lengths."""
    lengths = np.asarray(lengths, dtype=np.int64)
    S = lengths.shape[0]
    nb = -(-lengths // bs)
    n_unique = int(nb.sum())
    NB, phys = _place_blocks(_rng(seed, perm_stream), n_unique, _POOL_SLACK)
    codes, scales = _fp8_tokens(seed, stream, n_unique * bs, dim)
    codes = codes.reshape(n_unique, bs, dim)
    scales = scales.reshape(n_unique, bs)
    logical, off = [], 0
    for s in range(S):
        logical.append(list(range(off, off + int(nb[s]))))
        off += int(nb[s])
        tail = int(nb[s] * bs - lengths[s])
        if tail:  # finite garbage in the unused tail of the last block
            codes[logical[s][-1], bs - tail:, :] = np.uint8(0x7E)
            scales[logical[s][-1], bs - tail:] = np.float32(100.0)
    pool = np.full((NB, bs, dim), FP8_NAN, dtype=np.uint8)
    pscale = np.full((NB, bs), np.nan, dtype=np.float32)
    pool[phys] = codes
    pscale[phys] = scales
    maxb = int(nb.max())
    bt = np.full((S, maxb), -1, dtype=np.int32)
    for s in range(S):
        bt[s, :nb[s]] = phys[np.asarray(logical[s], dtype=np.int64)]
    if not keep_content:
        codes = scales = None
    return pool, pscale, bt, logical, codes, scales


def make_mla_decode(seed: int = 4, *, num_seqs: int = 64, q_per_seq: int = 4, lo: int = 32768,
                    hi: int = 262144, num_q_heads: int = 64, q_mult: float = 1.0,
                    keep_content: bool = False, lengths=None) -> PagedMLA:
    """MLA MTP3 decode: L ~ U{lo..hi} including the q_per_seq query tokens."""
    if lengths is None:
        lengths = _rng(seed, 0).integers(lo, hi + 1, num_seqs)
    lengths = np.asarray(lengths, dtype=np.int64)
    S = lengths.shape[0]
    pool, pscale, bt, logical, ck, cs = _paged_fp8(seed, 2, lengths, MLA_D_QK, MLA_BLOCK, 1,
                                                   keep_content)
    q_start = np.arange(S + 1, dtype=np.int32) * q_per_seq
    q = _bf16_normal(seed, 5, (S * q_per_seq, num_q_heads, MLA_D_QK), q_mult)
    return PagedMLA(num_q_heads, MLA_BLOCK, 1.0 / math.sqrt(MLA_D_QK), lengths.astype(np.int32),
                    np.full(S, q_per_seq, np.int32), q_start, bt, pool, pscale, q, logical, ck, cs,
                    CONFIG_NAMES[4])


@dataclass
class IndexerInput:
    """Indexer keys (FP8, one 128-wide key per token shared by all indexer heads),
    indexer queries and per-(token, head) weights, for the query tokens of `mla`."""
    idx_pool: np.ndarray           # uint8 [NB][bs][128]
    idx_scale: np.ndarray          # float32 [NB][bs]
    q_idx: np.ndarray              # uint16 [n_q][H_idx][128]
    w: np.ndarray                  # float32 [n_q][H_idx]
    content_k: np.ndarray | None = None     # uint8 [n_unique][bs][128]
    content_scale: np.ndarray | None = None
    # MXFP4 keys of the packed layout (make_sparse_mla(..., fp4_keys=True)): the same draws
    fp4_pool: np.ndarray | None = None       # uint8 [NB][bs][64]  (two E2M1 a byte)
    fp4_scale: np.ndarray | None = None      # uint8 [NB][bs][4]   (E8M0 per 32 elements)

    def k_contiguous(self, mla: PagedMLA, s: int) -> tuple[np.ndarray, np.ndarray]:
        assert self.content_k is not None
        L = int(mla.total_len[s])
        ids = mla.logical_blocks[s]
        return (np.ascontiguousarray(self.content_k[ids].reshape(-1, self.q_idx.shape[2])[:L]),
                np.ascontiguousarray(self.content_scale[ids].reshape(-1)[:L]))


def make_sparse_mla(seed: int = 5, *, cached: int = 131072, new: int = 4096, num_q_heads: int = 64,
                    idx_heads: int = 64, idx_dim: int = 128, q_mult: float = 1.0,
                    keep_content: bool = False, lengths=None, n_new=None, fp4_keys: bool = False):
    """One (or more) sequences with `cached` prefix tokens and `new` query tokens.
    Returns (PagedMLA for the latent cache and MLA queries, IndexerInput).  With fp4_keys
    the indexer keys are also stored as MXFP4 (fp4_pool / fp4_scale, same draws, same
    block table) for the packed per-block layout."""
    if lengths is None:
        lengths = np.array([cached + new], dtype=np.int64)
        n_new = np.array([new], dtype=np.int64)
    lengths = np.asarray(lengths, dtype=np.int64)
    n_new = np.asarray(n_new, dtype=np.int64)
    S = lengths.shape[0]
    pool, pscale, bt, logical, ck, cs = _paged_fp8(seed, 2, lengths, MLA_D_QK, MLA_BLOCK, 1,
                                                   keep_content)
    # indexer keys share the block table: same physical block ids, their own pool
    nb = -(-lengths // MLA_BLOCK)
    n_unique = int(nb.sum())
    kc, ks = _fp8_tokens(seed, 7, n_unique * MLA_BLOCK, idx_dim)
    kc = kc.reshape(n_unique, MLA_BLOCK, idx_dim)
    ks = ks.reshape(n_unique, MLA_BLOCK)
    NB = pool.shape[0]
    ipool = np.full((NB, MLA_BLOCK, idx_dim), FP8_NAN, dtype=np.uint8)
    iscale = np.full((NB, MLA_BLOCK), np.nan, dtype=np.float32)
    for s in range(S):
        tail = int(nb[s] * MLA_BLOCK - lengths[s])
        if tail:
            kc[logical[s][-1], MLA_BLOCK - tail:, :] = np.uint8(0x7E)
            ks[logical[s][-1], MLA_BLOCK - tail:] = np.float32(100.0)
        phys = bt[s, :nb[s]].astype(np.int64)
        ipool[phys] = kc[logical[s]]
        iscale[phys] = ks[logical[s]]
    fpool = fscale = None
    if fp4_keys:
        fk, fs = _mxfp4_tokens(seed, 7, n_unique * MLA_BLOCK, idx_dim)
        fk = fk.reshape(n_unique, MLA_BLOCK, idx_dim // 2)
        fs = fs.reshape(n_unique, MLA_BLOCK, idx_dim // 32)
        fpool = np.full((NB, MLA_BLOCK, idx_dim // 2), 0x77, dtype=np.uint8)     # poison: NaN scales
        fscale = np.full((NB, MLA_BLOCK, idx_dim // 32), 0xFF, dtype=np.uint8)
        for s in range(S):
            tail = int(nb[s] * MLA_BLOCK - lengths[s])
            if tail:     # large finite garbage in the unused tail: 6 * 2^73
                fk[logical[s][-1], MLA_BLOCK - tail:, :] = np.uint8(0x77)
                fs[logical[s][-1], MLA_BLOCK - tail:, :] = np.uint8(200)
            phys = bt[s, :nb[s]].astype(np.int64)
            fpool[phys] = fk[logical[s]]
            fscale[phys] = fs[logical[s]]
    q_start = np.zeros(S + 1, dtype=np.int32)
    q_start[1:] = np.cumsum(n_new)
    nq = int(q_start[-1])
    q = _bf16_normal(seed, 5, (nq, num_q_heads, MLA_D_QK), q_mult)
    q_idx = _bf16_normal(seed, 8, (nq, idx_heads, idx_dim))
    w = (normal_f32(seed, 9, nq * idx_heads) / np.float32(8.0)).reshape(nq, idx_heads)
    mla = PagedMLA(num_q_heads, MLA_BLOCK, 1.0 / math.sqrt(MLA_D_QK), lengths.astype(np.int32),
                   n_new.astype(np.int32), q_start, bt, pool, pscale, q, logical, ck, cs,
                   CONFIG_NAMES[5])
    idx = IndexerInput(ipool, iscale, q_idx, w, kc if keep_content else None,
                       ks if keep_content else None, fpool, fscale)
    return mla, idx


# --------------------------------------------------------------------------- packed blocks
# One allocation per 64-token block for every cache group of the MLA layer: bytes
# [0, 36864) FP8 latent [64][576]; [36864, 37120) fp32 latent scales [64]; [37120, 41216)
# MXFP4 index keys [64][64]; [41216, 41472) E8M0 key scales [64][4].
PACKED_BLOCK_BYTES = 41472


def pack_mla_blocks(mla: PagedMLA, idx: IndexerInput) -> np.ndarray:
    """The packed pool [NB][41472] bytes of a latent pool plus its MXFP4 index keys (same
    block ids).  Byte copies only."""
    nb = mla.kv_pool.shape[0]
    out = np.empty((nb, PACKED_BLOCK_BYTES), dtype=np.uint8)
    out[:, :36864] = mla.kv_pool.reshape(nb, -1)
    out[:, 36864:37120] = np.ascontiguousarray(mla.kv_scale, dtype=np.float32).view(np.uint8).reshape(nb, -1)
    out[:, 37120:41216] = idx.fp4_pool.reshape(nb, -1)
    out[:, 41216:] = idx.fp4_scale.reshape(nb, -1)
    return out


# --------------------------------------------------------------------------- top-k fixtures
def tie_scores(seed: int, n_rows: int, n_cols: int, levels: int = 3) -> np.ndarray:
    """Scores drawn from {0, 1, ..., levels-1}: heavy ties for the lower-index rule."""
    return _rng(seed, 11).integers(0, levels, (n_rows, n_cols)).astype(np.float32)


# --------------------------------------------------------------------------- KV append
@dataclass
class AppendInput:
    """New KV rows of one step and where they go: sequence s appends new_len[s] rows (input
    rows q_start[s] ...) after its cached_len[s] tokens.  Every sequence owns distinct
    blocks (a shuffled pool), so no two rows share a destination."""
    block_size: int
    num_blocks: int
    block_table: np.ndarray        # int32 [S][width], -1 past a sequence's last block
    cached_len: np.ndarray         # int32 [S]
    new_len: np.ndarray            # int32 [S]
    q_start: np.ndarray            # int32 [S]
    k_new: np.ndarray              # uint16 bf16 bits [n][*row_shape]
    v_new: np.ndarray | None       # same shape or None (FP8 pools)


def make_append(seed: int, *, cached, new, block_size: int, row_shape, with_v: bool,
                row_mults=(1.0,), zero_rows: int = 0, slack: int = 3) -> AppendInput:
    """Append layout plus N(0,1) rows; row i is scaled by row_mults[i % len(row_mults)] and
    the first zero_rows rows are all zero (the degenerate amax = 0 case)."""
    rng = _rng(seed, 20)
    cached = np.asarray(cached, np.int64)
    new = np.asarray(new, np.int64)
    need = -(-(cached + new) // block_size)
    width = int(max(1, need.max()))
    nb = int(need.sum()) + slack
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((len(cached), width), -1, np.int32)
    k = 0
    for s, m in enumerate(need):
        bt[s, :m] = perm[k:k + m]
        k += int(m)
    q_start = np.concatenate([[0], np.cumsum(new)[:-1]]).astype(np.int32)
    n = int(new.sum())
    shape = (n,) + tuple(row_shape)
    mult = np.asarray(row_mults, np.float32)[np.arange(n) % len(row_mults)]
    mult = mult.reshape((n,) + (1,) * len(row_shape))

    def rows(stream):
        x = normal_f32(seed, stream, int(np.prod(shape))).reshape(shape) * mult
        x[:zero_rows] = 0
        return _par_map(bf16_bits, x).reshape(shape)

    return AppendInput(block_size, nb, bt, cached.astype(np.int32), new.astype(np.int32), q_start,
                       rows(21), rows(22) if with_v else None)
