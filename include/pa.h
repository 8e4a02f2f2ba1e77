/*
 * pa.h -- paged, prefix-reused attention for AMD MI355X (gfx950).  C ABI.
 *
 * Five calls make up the hot path of agentic serving as the pages describe it: new
 * query tokens attend to a paged KV cache whose long prefix is reused across turns.
 *
 *   paged_attn_prefill   suffix prefill on top of a cached prefix (GQA / MHA, bf16)
 *   paged_attn_decode    decode with 1..4 query tokens per sequence (GQA bf16, or the
 *                        FP8 MLA latent cache shared by all query heads)
 *   mla_indexer_topk     indexer scores plus per-query top-k (k = 2048 in the pages)
 *   sparse_mla_attn      MLA attention restricted to the selected tokens
 *   paged_kv_append      writes the new tokens' K/V into the pool (FP8 pools quantised
 *                        per token)
 *
 * Sources (page title, section):
 *   [AgentX] vLLM AgentX article (news.ainew.jp):
 *            "Hybrid KV cache management" -- one shared block pool, the page (block) is
 *                                            the single allocation unit (Figure 4);
 *            "Re-evaluating agentic workloads" -- long inputs, >96 % prefix reuse, short
 *                                            new prefill per turn;
 *            "Kimi K3" -- MLA keeps one latent head; partial outputs and their
 *                         log-sum-exp are merged with online softmax (Figure 7);
 *            "DeepSeek V4" -- 64-head indexer, one global top-k per token; sparse MLA
 *                             gathers the top-k entries, then attends.
 *   [GLM]    GLM-5.3 on 16xH200 report (aisoku.org):
 *            "What's new" -- latent KV shared by 64 heads; the indexer picks 2,048
 *                            tokens; MTP3 speculative decoding (the table);
 *            "Configuration and numbers" table -- FP8 KV;
 *            "How to try" -- prompts inside the top-k still use the sparse MLA kernel.
 *
 * Conventions shared by every call
 *   - All pointers are caller-owned and borrowed.  Pointers marked "dev" are device
 *     memory and must stay valid until the work enqueued on `stream` has finished.
 *     Pool descriptors (pa_kv_pool) are host structs read during the call only.
 *   - All integer arrays are int32, row-major, contiguous.  bf16 tensors are passed as
 *     raw 16-bit patterns; FP8 is OCP E4M3FN (bias 7, max 448, no infinities).
 *   - Logical token t of sequence s lives in physical block block_table[s*bt_stride +
 *     t/block_size], row t%block_size.  Entries past a sequence's last block are never
 *     read (callers put -1 there).  A kernel that meets an out-of-range block id within
 *     a sequence treats that block as all-zero keys and values instead of reading it.
 *   - Causality: the query at logical position p sees keys t <= p.
 *   - Every call validates its arguments BEFORE enqueueing anything; on error nothing is
 *     launched, outputs are untouched and the return value says why
 *     (pa_last_error_detail() has a thread-local message).  Values that live only in
 *     device memory (lengths, block ids) cannot be checked on the host; kernels clamp
 *     lengths to the host-given maxima and skip out-of-range block ids.
 *   - Calls are asynchronous on `stream`; there is no host synchronisation inside.
 *     The library never allocates or frees memory: scratch space is a caller-provided
 *     workspace of at least *_workspace_size(...) bytes (16-byte aligned).
 *   - No C++ exception crosses this interface.  Thread-safe across streams.
 *   - lse outputs (nullable) are natural-log log-sum-exp of the scaled logits, fp32.
 *   - Value domains.  Inputs must be finite.  Some operands are converted once from bf16
 *     to fp16 inside the kernels (round toward zero): the prefill's V values, and the MLA
 *     / sparse-MLA queries in the exact recomputation kernel (units whose scores outgrow
 *     the fixed softmax reference).  The conversion is exact for magnitudes in
 *     [2^-14, 65504]; smaller ones become fp16 subnormals (absolute error < 2^-25) and
 *     larger ones saturate to +-65504, so those operands must stay within +-65504.  In the
 *     main MLA kernel each query row is scaled by a power of two (largest magnitude into
 *     [128, 256)) and split into two E4M3 terms for the FP8 Q.K product: exact for
 *     elements at least 2^-9 of the row's largest, absolute error <= 2^-10 in the scaled
 *     units below that.  Softmax probabilities are fed to P.V as fp16 (prefill, MLA) or
 *     as a bf16 hi + lo pair (GQA decode); FP8 values convert to fp16 / bf16 exactly.
 *   - Library state.  Besides the thread-local error text, the library keeps (a) the
 *     compute-unit count of each device it has run on (read once per device and process,
 *     used to size grids and the prefill split), and (b) the optional profiling tables of
 *     pa_profile_*, which exist only between pa_profile_enable and pa_profile_disable and
 *     are guarded by a mutex.  Neither holds caller pointers; no call's result depends on
 *     them except through the device's compute-unit count.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int pa_status;
#define PA_OK 0
#define PA_ERR_INVALID_ARG 1   /* null pointer, bad shape, misalignment             */
#define PA_ERR_UNSUPPORTED 2   /* valid but not implemented (head dim, block size)  */
#define PA_ERR_WORKSPACE 3     /* workspace smaller than *_workspace_size(...)      */
#define PA_ERR_HIP 4           /* a launch failed (hipGetLastError after enqueue)   */

#define PA_BF16 1
#define PA_FP8_E4M3 2
#define PA_PACKED_MLA 3

/* One shared block pool ([AgentX] "Hybrid KV cache management").
 *   GQA / MHA (kv_dtype PA_BF16, block_size 16, head_dim_qk == head_dim_v in {64, 128}):
 *     k, v : dev bf16 [num_blocks][num_kv_heads][block_size][head_dim]   scale: NULL
 *   MLA latent (kv_dtype PA_FP8_E4M3, block_size 64, num_kv_heads 1,
 *               head_dim_qk 576, head_dim_v 512):
 *     k    : dev e4m3 [num_blocks][block_size][576]; bytes 0..511 are the latent, which
 *            is also V ([AgentX] "Kimi K3"; [GLM] "What's new"), bytes 512..575 rope.
 *     v    : NULL
 *     scale: dev fp32 [num_blocks][block_size], dequantised K_t = scale_t * e4m3(k_t).
 *   Indexer keys (kv_dtype PA_FP8_E4M3, block_size 64, num_kv_heads 1,
 *                 head_dim_qk 128, head_dim_v 0): k e4m3 [num_blocks][64][128] plus
 *     scale as above; they share the MLA block table.
 *   Packed per-block layout (kv_dtype PA_PACKED_MLA; [AgentX] "Hybrid KV cache
 *     management", Figure 5: every cache group of a block in one allocation; with the FP4
 *     indexer it saves about 10 % of KV memory).  k points to [num_blocks][41472] bytes, v
 *     and scale are unused (NULL).  A 64-token block holds, at byte offsets:
 *         0      FP8 E4M3 latent   [64][576]   (as the MLA pool above)
 *         36864  fp32 latent scale [64]
 *         37120  MXFP4 index keys  [64][64]    128 FP4 E2M1 elements a token, element 2j
 *                                              in the low nibble of byte j
 *         41216  E8M0 key scales   [64][4]     one per 32 elements: 2^(code - 127)
 *     648 B per token against 712 B for the FP8 latent and FP8 index-key pools.  The MX
 *     format (OCP Microscaling MXFP4) is the reading of the page's "FP4 indexer"; key
 *     scale codes must lie in [2, 252] (paged_kv_append only writes such codes); the
 *     indexer applies them inside its FP8 x FP4 MFMA, so each 32-element partial dot
 *     product times 2^(code - 127) must stay within the float range.  The same k pointer serves two views:
 *       latent view   (block_size 64, num_kv_heads 1, head_dim_qk 576, head_dim_v 512)
 *                     for paged_attn_decode, sparse_mla_attn and the latent append;
 *       index view    (block_size 64, num_kv_heads 1, head_dim_qk 128, head_dim_v 0)
 *                     for mla_indexer_topk and the key append (MXFP4 quantisation).
 *   FP8 and packed pools: num_blocks * 64 must fit in int32 (PA_ERR_UNSUPPORTED
 *   otherwise). */
typedef struct {
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim_qk;
  int32_t head_dim_v;
  int32_t kv_dtype;
  const void* k;
  const void* v;
  const float* scale;
} pa_kv_pool;

const char* pa_status_string(pa_status s);
const char* pa_last_error_detail(void);
int32_t pa_version(void);

/* ---------------------------------------------------------------------------------
 * 1. Prefix-cached suffix prefill ([AgentX] "Re-evaluating agentic workloads": each turn
 *    re-sends the whole history, most of it an already-cached prefix, and the new
 *    prefill is short; [AgentX] "Two-level scheduling": chunked prefill).
 *
 * For sequence s, new_len[s] query tokens at logical positions cached_len[s] ...
 * cached_len[s]+new_len[s]-1 attend causally to the new tokens and fully to the cached
 * prefix.  The pool must already hold the KV of all cached_len[s]+new_len[s] tokens.
 *   q         dev bf16 [total_q][num_q_heads][head_dim]; rows q_start[s] ...
 *             q_start[s]+new_len[s]-1 belong to sequence s (packed batch).
 *   pool      GQA/MHA bf16 pool; num_q_heads % num_kv_heads == 0; query head h reads
 *             KV head h / (num_q_heads/num_kv_heads).
 *   block_table dev int32 [num_seqs][bt_stride].
 *   cached_len, new_len  dev int32 [num_seqs];  q_start dev int32 [num_seqs+1].  The
 *             rows q_start[s] .. q_start[s]+min(new_len[s], max_new_len)-1 must lie inside
 *             q and out; gaps between the sequences' rows are allowed and never touched.
 *   max_new_len    host upper bound of new_len[s] (grid sizing).  A sequence with more
 *                  new tokens has only its first max_new_len computed (at positions
 *                  cached_len[s] + j); the output rows of the rest are not written.
 *   max_total_len  host upper bound of cached_len[s]+new_len[s].
 *   scale     softmax scale (1/sqrt(head_dim) for the pages' workloads).
 *   out       dev bf16 [total_q][num_q_heads][head_dim].
 *   lse       dev fp32 [total_q][num_q_heads] or NULL.
 * Supported: PA_BF16, block_size 16, head_dim 64 or 128, num_q_heads/num_kv_heads in
 * {1, 2, 4, 8}.
 * Workspace: when the new-token tiles are too few to fill the GPU and the contexts are
 * long (a chunked-prefill step: [AgentX] "Two-level scheduling", 512-token chunks), the
 * keys of each tile are split into ranges whose partial (output, log-sum-exp) pairs are
 * merged in a fixed order; paged_attn_prefill_workspace_size() then returns the bytes of
 * those partials (0 when the call runs unsplit).  The choice depends only on the sizes
 * and the device, so the size query and the call agree; results are deterministic.  The
 * partials of new token j of sequence s live in token slot s * max_new_len + j, so the
 * call never writes past the workspace size returned for the same num_seqs and maxima.
 * ------------------------------------------------------------------------------- */
size_t paged_attn_prefill_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                         int32_t max_new_len, int32_t max_total_len,
                                         const pa_kv_pool* pool);
pa_status paged_attn_prefill(const void* q, const pa_kv_pool* pool,
                             const int32_t* block_table, int32_t bt_stride,
                             const int32_t* cached_len, const int32_t* new_len,
                             const int32_t* q_start, int32_t num_seqs, int32_t num_q_heads,
                             int32_t max_new_len, int32_t max_total_len, float scale,
                             void* out, float* lse, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * 2. Paged decode with q_per_seq query tokens per sequence (1 for plain decode, 4 for
 *    MTP3 verification: [GLM] table, three draft tokens).
 *
 * context_len[s] counts every token in the pool for sequence s, including its
 * q_per_seq query tokens, which sit at positions context_len[s]-q_per_seq+j and are
 * causal among themselves.  Long contexts are split into key ranges whose partial
 * (output, log-sum-exp) pairs are merged in a fixed order ([AgentX] "Kimi K3"), so the
 * result is deterministic run to run.
 *   q     dev bf16 [num_seqs][q_per_seq][num_q_heads][head_dim_qk]
 *   out   dev bf16 [num_seqs][q_per_seq][num_q_heads][head_dim_v]
 *   lse   dev fp32 [num_seqs][q_per_seq][num_q_heads] or NULL
 *   max_context_len  host upper bound of context_len[s].
 * Supported: the GQA bf16 pool (head_dim 64/128, block 16, group size 1..8) and the MLA
 * FP8 latent pool (576/512, block 64, num_q_heads 64... any multiple of 16 up to 128);
 * 1 <= q_per_seq <= 4.
 * ------------------------------------------------------------------------------- */
size_t paged_attn_decode_workspace_size(int32_t num_seqs, int32_t q_per_seq,
                                        int32_t num_q_heads, int32_t max_context_len,
                                        const pa_kv_pool* pool);
pa_status paged_attn_decode(const void* q, const pa_kv_pool* pool,
                            const int32_t* block_table, int32_t bt_stride,
                            const int32_t* context_len, int32_t num_seqs, int32_t q_per_seq,
                            int32_t num_q_heads, int32_t max_context_len, float scale,
                            void* out, float* lse, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * 2b. Decode without a workspace argument, for callers that cannot allocate device
 *     memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 *     hipMalloc.  Same arguments, kernels and results as paged_attn_decode (bit for bit),
 *     minus the workspace: the call runs on a scratch array of PA_NOALLOC_SCRATCH_BYTES
 *     that the library keeps in device memory, one per GPU, held until the process ends.
 *     It allocates nothing and calls no allocating routine.
 *   Limit: sizes whose paged_attn_decode_workspace_size(...) exceeds
 *     PA_NOALLOC_SCRATCH_BYTES are rejected with PA_ERR_WORKSPACE before anything is
 *     launched (use paged_attn_decode with a workspace for those).
 *   Concurrency: every call on one GPU uses that GPU's one scratch array.  Calls that
 *     overlap on one GPU (different streams, or different host threads without ordering)
 *     race on it and give undefined results; calls in one stream are ordered and safe.
 *     The array keeps the last call's contents; each call writes every part it later
 *     reads, so nothing needs clearing between calls.
 * ------------------------------------------------------------------------------- */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
size_t paged_attn_decode_noalloc_max_bytes(void);
pa_status paged_attn_decode_noalloc(const void* q, const pa_kv_pool* pool,
                                    const int32_t* block_table, int32_t bt_stride,
                                    const int32_t* context_len, int32_t num_seqs,
                                    int32_t q_per_seq, int32_t num_q_heads,
                                    int32_t max_context_len, float scale, void* out, float* lse,
                                    hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * 3. Indexer scores and top-k ([AgentX] "DeepSeek V4": 64 indexer heads, one global
 *    top-k per token; [GLM] "What's new": 2,048 tokens selected per query token).
 *
 * For query row i of sequence s (rows q_start[s] ... q_start[s]+new_len[s]-1, at logical
 * positions cached_len[s] + (i - q_start[s])):
 *   I[i,t] = sum_h w[i,h] * max(0, <q_idx[i,h,:], k_t>)   for t <= pos(i)
 * with k_t = scale_t * e4m3(key bytes of token t) from idx_pool (one 128-wide key per
 * token shared by all indexer heads).  topk_idx[i] receives the k largest I[i,t], ties
 * broken toward the lower t, in ascending t, padded with -1 when pos(i)+1 < k.
 *   q_idx     dev bf16 [n_q][num_idx_heads][128]
 *   w         dev fp32 [n_q][num_idx_heads]
 *   idx_pool  FP8 indexer-key pool, or the index view of a packed pool (MXFP4 keys:
 *             k_t is then the decoded MXFP4 vector, no per-token scale)
 *   topk_idx  dev int32 [n_q][k]
 *   scores_out dev fp32 [n_q][max_total_len] or NULL: row i gets I[i,0..pos(i)] and -inf
 *              after it (-0.0 is written as +0.0).  The top-k is exactly the selection
 *              made from these values.
 * Supported: num_idx_heads a multiple of 16 (<= 64), head dim 128, block 64,
 * 1 <= k <= 4096.
 * ------------------------------------------------------------------------------- */
size_t mla_indexer_topk_workspace_size(int32_t n_q, int32_t num_idx_heads,
                                       int32_t max_total_len, int32_t k);
pa_status mla_indexer_topk(const void* q_idx, const float* w, const pa_kv_pool* idx_pool,
                           const int32_t* block_table, int32_t bt_stride,
                           const int32_t* cached_len, const int32_t* new_len,
                           const int32_t* q_start, int32_t num_seqs, int32_t n_q,
                           int32_t num_idx_heads, int32_t max_new_len, int32_t max_total_len,
                           int32_t k, int32_t* topk_idx, float* scores_out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * 4. Sparse MLA ([AgentX] "DeepSeek V4": gather the top-k latent entries, then attend;
 *    [GLM] "How to try": the same kernel serves prompts shorter than k).
 *
 * Query row i (sequence q_seq[i]) attends, with all num_q_heads heads sharing the one
 * latent, only to the logical positions topk_idx[i][0..k-1] (entries < 0 are skipped;
 * duplicates count twice).  A row with no selected token gets out = 0, lse = -inf.
 *   q         dev bf16 [n_q][num_q_heads][576]
 *   pool      MLA FP8 latent pool
 *   q_seq     dev int32 [n_q]
 *   topk_idx  dev int32 [n_q][k]
 *   out       dev bf16 [n_q][num_q_heads][512];  lse dev fp32 [n_q][num_q_heads] or NULL
 * Supported: num_q_heads a multiple of 16 up to 128; 1 <= k <= 8192.
 * ------------------------------------------------------------------------------- */
size_t sparse_mla_attn_workspace_size(int32_t n_q, int32_t k, int32_t num_q_heads);
pa_status sparse_mla_attn(const void* q, const pa_kv_pool* pool, const int32_t* block_table,
                          int32_t bt_stride, const int32_t* q_seq, const int32_t* topk_idx,
                          int32_t n_q, int32_t k, int32_t num_q_heads, float scale, void* out,
                          float* lse, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * 5. Paged KV append with per-token FP8 quantisation ([AgentX] "Hybrid KV cache
 *    management": the new tokens' KV goes into blocks of the one shared pool through the
 *    block table; [GLM] "Configuration and numbers" table: FP8 KV; "What's new": one
 *    latent row per token, shared by the query heads).
 *
 * New token j < new_len[s] of sequence s is input row q_start[s] + j and is written to
 * logical position cached_len[s] + j, i.e. row (cached_len[s]+j) % block_size of block
 * block_table[s*bt_stride + (cached_len[s]+j)/block_size].  Nothing else in the pool
 * changes.  This is the call that fills the pool before prefill (cached_len = prefix
 * length) or decode (cached_len = context_len - q_per_seq).
 *   pool    GQA bf16 pool: k_new, v_new dev bf16 [n_tokens][num_kv_heads][head_dim] are
 *           copied bit for bit.
 *           FP8 pools (MLA latent 576 or indexer keys 128): k_new dev bf16
 *           [n_tokens][head_dim_qk], v_new ignored.  Each row x is quantised on its
 *           own: scale = amax/448 with amax = max|x| (scale = 1 for an all-zero row),
 *           code[e] = OCP E4M3 round-to-nearest-even of x[e]/scale, both divisions IEEE
 *           float32, magnitudes past 448 clamped to 448; pool->scale gets the scale.
 *           The pages print no quantiser: this per-token amax scaling is the plain one.
 *           Packed pools: the latent view takes [n_tokens][576] rows as above (codes and
 *           scale into the block's latent fields); the index view takes [n_tokens][128]
 *           rows quantised to MXFP4 per group of 32 (OCP MX conversion): scale code
 *           e = floor(log2 amax) - 2 + 127 kept in [2, 252] (127 for an all-zero group),
 *           element code = E2M1 round-to-nearest-even of x / 2^(e-127), saturating at 6,
 *           the sign kept (-0 for a negative value that rounds to zero).
 *           pool->k, pool->v and pool->scale must point to writable device memory.
 *   block_table dev int32 [num_seqs][bt_stride]; cached_len, new_len, q_start dev int32
 *           [num_seqs].
 *   n_tokens     number of input rows; rows outside [0, n_tokens) are never read.
 *   max_new_len  host upper bound of new_len[s] (grid sizing; larger values are clamped).
 * Tokens whose position falls outside the block table's bt_stride entries, or whose
 * block id is out of range, are not written.  The destination rows of different
 * sequences must be distinct (prefix-shared blocks are full and never appended to); if
 * two tokens map to one row, which one lands is unspecified.  Inputs must be finite.
 * Supported: the GQA pool of call 1 and the FP8 MLA / indexer pools; num_seqs <= 65535.
 * No workspace.
 * ------------------------------------------------------------------------------- */
pa_status paged_kv_append(const pa_kv_pool* pool, const int32_t* block_table, int32_t bt_stride,
                          const int32_t* cached_len, const int32_t* new_len,
                          const int32_t* q_start, int32_t num_seqs, int32_t n_tokens,
                          int32_t max_new_len, const void* k_new, const void* v_new,
                          hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * Test hooks (not part of the serving API).
 *
 * pa_test_gather_kv: copies the first n_tokens logical tokens of sequence `seq` out of
 *   the pool into contiguous buffers with the same block-table walk the attention
 *   kernels use.  GQA: k_out, v_out dev bf16 [n_tokens][num_kv_heads][head_dim].  FP8
 *   pools: k_out dev bytes [n_tokens][head_dim_qk], scale_out dev fp32 [n_tokens],
 *   v_out unused.  The index view of a packed pool: k_out [n_tokens][64] (FP4 codes),
 *   scale_out receives each token's 4 E8M0 codes as one 32-bit word.  Bit-exact copy.
 * pa_test_topk_from_scores: the top-k selection stage alone, on caller-given fp32
 *   scores [n_rows][row_stride] with valid_len dev int32 [n_rows]; same ordering and
 *   tie rules as mla_indexer_topk.  Workspace: pa_test_topk_workspace_size.
 * ------------------------------------------------------------------------------- */
pa_status pa_test_gather_kv(const pa_kv_pool* pool, const int32_t* block_table,
                            int32_t bt_stride, int32_t seq, int32_t n_tokens, void* k_out,
                            void* v_out, float* scale_out, hipStream_t stream);
size_t pa_test_topk_workspace_size(int32_t n_rows, int32_t k);
pa_status pa_test_topk_from_scores(const float* scores, const int32_t* valid_len,
                                   int32_t n_rows, int32_t row_stride, int32_t k,
                                   int32_t* out_idx, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * Profiling hooks (not part of the serving path).
 *
 * pa_profile_enable(max_records): from now on, every kernel the library launches (up to
 *   max_records launches) is bracketed by two hipEvents recorded on the call's stream.
 *   Creates 2*max_records events (no device memory is allocated); resets the records.
 *   The events are timing-only (created with hipEventDisableSystemFence): a record
 *   writes back and invalidates no cache, yet each still costs the stream a few
 *   microseconds, so a step that must be timed as a whole brackets only the launch it
 *   reports.
 * pa_profile_select(name): records only launches of that kernel name (see below); NULL
 *   or "" records every launch again.  PA_ERR_INVALID_ARG for a name of 64 characters or
 *   more.  pa_profile_disable clears the selection.
 * pa_profile_count(): number of launches recorded so far.
 * pa_profile_record(i, name, cap, ms): waits for record i and returns its kernel name
 *   ("prefill_gqa", "decode_gqa", "decode_mla", "combine", "indexer", "topk",
 *   "sparse_mla", "append_gqa", "append_fp8") and its duration in milliseconds.
 * pa_profile_disable(): stops recording and destroys the events.
 * ------------------------------------------------------------------------------- */
pa_status pa_profile_enable(int32_t max_records);
pa_status pa_profile_select(const char* name);
int32_t pa_profile_count(void);
pa_status pa_profile_record(int32_t i, char* name_out, int32_t name_cap, float* ms_out);
pa_status pa_profile_disable(void);

#ifdef __cplusplus
}
#endif
#endif /* PA_H_ */
