"""CPU oracle for paged, prefix-reused attention.  TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this
package.  The product path (the HIP library and its Python binding) never imports,
calls or links it, and it shares no code with that path.

Everything is plain numpy in float64 over contiguous (un-paged) K/V.  Inputs are
converted exactly from their storage formats (bf16 bits, OCP FP8 E4M3 bytes times an
fp32 per-token scale).  Each function states the passage of the pages it follows; the
pages name the operations (paged KV over one shared block pool, a latent KV shared by 64
heads, FP8 KV, an indexer choosing 2,048 tokens, sparse MLA over the chosen tokens, an
LSE merge of partial outputs) but print no formulas, so every definition here is the
textbook reading of the named operation.

Pins (tests/test_oracle_*.py) tie each function to something other than itself:
brute-force loops with math.fsum, closed forms, invariants, permuted block tables,
special cases (k >= context => dense; GQA == MHA with repeated KV), the OCP E4M3 table.
The KV append (append.py) quantises each new token to FP8 by a nearest-value search over
the E4M3 table; that encoder is pinned to the format's halfway points and saturation, to
the round trip of every code and to PyTorch's own float8_e4m3fn conversion.  The MXFP4
indexer keys of the packed per-block layout (E2M1 elements, E8M0 group scales) are decoded
by table and quantised by a nearest-value search; both are pinned to the OCP MX format's
values, halfway points, saturation and shared-exponent rule.
No function here is "parity unpinned".
"""
from .formats import bf16_to_f64, e4m3_decode, e2m1_decode, e8m0_decode, mxfp4_decode  # noqa: F401
from .attention import (  # noqa: F401
    gather_paged, attention, attention_probs, lse_merge, paged_gqa_attention,
    mla_dequant, mla_attention, indexer_scores, indexer_scores_mxfp4, indexer_scores_from_keys,
    topk_indices, sparse_mla_attention,
)
from .append import (  # noqa: F401
    e4m3_nearest, quantize_token_fp8, token_positions, append_gqa, append_fp8,
    e2m1_nearest, mx_shared_exponent, quantize_token_mxfp4, packed_fields, append_packed,
    PACKED_BLOCK_BYTES, PACKED_LATENT, PACKED_LATENT_SCALE, PACKED_KEYS, PACKED_KEY_SCALES,
)
