// Host-side launch interfaces between the C ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// MLA decode: keys per split of the key range.  Each split yields a partial (o, lse) pair
// that the combine kernel merges in split order.
#ifndef PA_DECODE_SPLIT_MLA
#define PA_DECODE_SPLIT_MLA 6144
#endif
constexpr int kDecodeSplitMla = PA_DECODE_SPLIT_MLA;

// GQA decode: the plan covers kPlanTiles 32-key tiles of a group per workgroup (a region).
constexpr int kPlanTiles = 256;
// Ints of LDS the GQA decode kernel sets aside for region and piece starts.
constexpr int kDecodeIdxLds = 4096;

// Compute units of the current device (read once per device): the GQA decode grid and the
// prefill split decision depend on it, so workspace queries and calls agree.
int device_cus();

// Host-side sizes of the GQA decode workspace (shared by the C ABI and the launcher).
struct GqaDecodeDims {
  int32_t members;      // sequences per group: 32 / (q_per_seq * group size), >= 1
  int32_t n_groups;     // ceil(num_seqs / members)
  int32_t n_chunks;     // plan regions per group: ceil(ceil(max_context_len / 32) / kPlanTiles)
  int32_t region_cap;   // pass capacity of one (group, chunk) region: kPlanTiles * members
  int32_t grid;         // attention workgroups: one per compute unit
  int32_t subs;         // sub-ranges per (piece, KV head): 8 / Hkv when Hkv divides 8, else 1
  int32_t pieces_cap;   // upper bound of pieces: groups + grid - 1
  int32_t scan_in_kernel;  // 1: every attention workgroup numbers the passes and pieces
                           //   itself, in LDS (regions + groups + 2 <= kDecodeIdxLds);
                           //   0: decode_scan_kernel numbers them in the workspace
};
GqaDecodeDims gqa_decode_dims(int num_seqs, int q_per_seq, int num_q_heads, int num_kv_heads,
                              int max_context_len);

struct GqaPrefillArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* bt;
  const int32_t* cached_len;
  const int32_t* new_len;
  const int32_t* q_start;
  uint16_t* out;
  float* lse;
  int32_t bt_stride, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks;
  int32_t max_new_len, max_total_len;
  float scale_log2;  // softmax scale * log2(e)
  // Split-K (split_len > 0): the keys of a tile are cut into ranges of split_len; each
  // workgroup writes the partial (o, log2-sum-exp) of one range for its rows at
  // [seq * max_new_len + token][split][num_q_heads] of part_o / part_lse, and the combine
  // kernel merges them.
  float* part_o;
  float* part_lse;
  int32_t split_len, max_splits;
};
// Key-range length for split-K prefill, or 0 when the prefill runs unsplit.  Depends only
// on the sizes (and the device's compute-unit count), so that the workspace query and the
// call agree.
int prefill_split_len(int num_seqs, int num_q_heads, int num_kv_heads, int max_new_len, int max_total_len);

struct GqaDecodeArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* bt;
  const int32_t* context_len;
  float* part_o;        // [pieces_cap * subs * Hkv * 32][D]: piece p, sub-range b, KV head h,
                        //   tile row r at ((p * subs + b) * Hkv + h) * 32 + r
  float* part_lse;      // [pieces_cap * subs * Hkv * 32], log2 units
  uint32_t* passes;     // [n_groups * n_chunks][region_cap][4]: {key base | (valid keys - 1),
                        //   block A, block B, member mask}
  int32_t* n_passes;    // [n_groups * n_chunks]
  int32_t* region_start;  // [n_groups * n_chunks + 1]: compact index of each region's first
                          //   pass; the total last
  int32_t* piece_start;   // [n_groups + 1]: first piece of each group; total last
  int32_t bt_stride, num_seqs, q_per_seq, num_q_heads, num_kv_heads, head_dim, num_blocks;
  int32_t max_context_len;
  GqaDecodeDims dims;
  float scale_log2;
};

struct CombineArgs {
  const float* part_o;
  const float* part_lse;
  const int32_t* context_len;   // [S]
  uint16_t* out;                // [S][rows][D]
  float* lse;                   // [S][rows] or null
  int32_t num_seqs, rows, head_dim, max_splits, split, max_context_len;
  // GQA decode partials (piece_start != null): row (t, hq) of sequence s reads the pieces
  // of its group (subs partials each); otherwise partials are [S][max_splits][rows] with
  // split `split`.
  const int32_t* piece_start;
  int32_t members, num_kv_heads, q_per_seq, subs;
  // Split-K prefill partials (pf_q_start != null): workgroup (s, j, head) merges the
  // partials of new token j of sequence s, written at [s * pf_max_new + j][split][rows]
  // (rows = heads), and writes output row q_start[s] + j.
  const int32_t* pf_q_start;
  const int32_t* pf_cached;
  const int32_t* pf_new_len;
  int32_t pf_max_new, pf_max_total;
};

// FP8 latent rows of a paged pool: row r of block b at kv + b * blk_bytes + r * 576, its
// fp32 scale at kv_sbase + b * sblk_bytes + 4 r.  Separate pools: blk_bytes 36,864,
// sblk_bytes 256; the packed per-block layout: both 41,472 (scales at byte 36,864 of a
// block).
struct MlaDecodeArgs {
  const uint16_t* q;            // [S][T][Hq][576]
  const uint8_t* kv;            // latent rows (see above)
  const uint8_t* kv_sbase;      // latent scales
  int64_t blk_bytes, sblk_bytes;
  const int32_t* bt;
  const int32_t* context_len;
  float* part_o;                // [S][max_splits][T*Hq][512]
  float* part_lse;
  int32_t bt_stride, num_seqs, q_per_seq, num_q_heads, num_blocks, max_context_len, max_splits;
  float scale_log2;
};

struct SparseMlaArgs {
  const uint16_t* q;            // [n_q][Hq][576]
  const uint8_t* kv;            // as MlaDecodeArgs
  const uint8_t* kv_sbase;
  int64_t blk_bytes, sblk_bytes;
  const int32_t* bt;
  const int32_t* q_seq;
  const int32_t* topk;          // [n_q][k]
  uint16_t* out;                // [n_q][Hq][512]
  float* lse;
  int32_t bt_stride, n_q, k, num_q_heads, num_blocks;
  float scale_log2;
};

struct IndexerArgs {
  const uint16_t* q_idx;        // [n_q][H][128]
  const float* w;               // [n_q][H]
  // Key row r of block b at keys + b * blk_bytes + r * row_bytes, its scale at
  // key_sbase + b * sblk_bytes + 4 r.  FP8 keys (fp4 = 0): 128-byte rows, one fp32 scale
  // per key.  MXFP4 keys of the packed layout (fp4 = 1): 64-byte rows (element 2j in the
  // low nibble of byte j), four E8M0 codes per key (one per 32 elements).
  const uint8_t* keys;
  const uint8_t* key_sbase;
  int64_t blk_bytes, sblk_bytes;
  int32_t fp4;
  const int32_t* bt;
  const int32_t* cached_len;
  const int32_t* new_len;
  const int32_t* q_start;
  float* scores;                // [n_q][score_stride]
  int32_t* valid_len;           // [n_q] written: pos(i)+1 (0 for rows outside any sequence)
  int32_t bt_stride, num_seqs, n_q, num_heads, num_blocks, max_new_len, max_total_len;
  int32_t score_stride;
};

struct TopkArgs {
  const float* scores;          // [n_rows][row_stride]
  const int32_t* valid_len;     // [n_rows]
  int32_t* out;                 // [n_rows][k]
  int32_t n_rows, row_stride, k, max_valid;
};

struct GatherArgs {
  const void* k;
  const void* v;
  const uint8_t* sbase;         // FP8 / packed views: scale of row r of block b at
  int64_t blk_bytes, sblk_bytes;  // sbase + b * sblk_bytes + 4 r; row at k + b * blk_bytes + r * row_bytes
  const int32_t* bt_row;
  void* k_out;
  void* v_out;
  float* scale_out;
  int32_t n_tokens, num_blocks, block_size, num_kv_heads, row_bytes;  // row_bytes: one token of one head
  int32_t is_fp8;
};

struct AppendArgs {
  const uint16_t* k_new;        // bf16 [n_tokens][Hkv][d] (GQA) or [n_tokens][D] (FP8 pools)
  const uint16_t* v_new;        // bf16 [n_tokens][Hkv][d] (GQA) or null
  const int32_t* bt;
  const int32_t* cached_len;
  const int32_t* new_len;
  const int32_t* q_start;
  uint16_t* k_out;              // GQA pool K / V [NB][Hkv][bs][d]
  uint16_t* v_out;
  uint8_t* fp8_out;             // FP8 / packed rows: row r of block b at fp8_out + b * blk_bytes + r * row_bytes
  uint8_t* scale_out;           // its scale (fp32, or 4 E8M0 codes) at scale_out + b * sblk_bytes + 4 r
  int64_t blk_bytes, sblk_bytes;
  int32_t mxfp4;                // 1: MXFP4 rows (the packed layout's index keys), else FP8
  int32_t bt_stride, num_seqs, n_tokens, max_new_len, num_blocks, block_size, num_kv_heads;
  int32_t head_dim;             // d (GQA) or D (FP8)
  int32_t is_fp8;
};

hipError_t launch_gqa_prefill(const GqaPrefillArgs& a, hipStream_t s);
// GQA decode = plan (pass lists, numbering) then the attention grid of one workgroup per CU.
hipError_t launch_gqa_decode_plan(const GqaDecodeArgs& a, hipStream_t s);
hipError_t launch_gqa_decode(const GqaDecodeArgs& a, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
// MLA: the fixed-reference kernel, then the exact kernel over the units it marked
hipError_t launch_mla_decode(const MlaDecodeArgs& a, hipStream_t s);
hipError_t launch_sparse_mla(const SparseMlaArgs& a, hipStream_t s);
hipError_t launch_mla_decode_exact(const MlaDecodeArgs& a, hipStream_t s);
hipError_t launch_sparse_mla_exact(const SparseMlaArgs& a, hipStream_t s);
hipError_t launch_indexer_scores(const IndexerArgs& a, hipStream_t s);
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
hipError_t launch_gather(const GatherArgs& a, hipStream_t s);
hipError_t launch_append(const AppendArgs& a, hipStream_t s);

}  // namespace pa
