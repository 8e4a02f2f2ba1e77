// C ABI of the paged-attention library: argument validation, workspace layout, launch.
// Every check happens before anything is enqueued; on error nothing is launched.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <cmath>
#include <mutex>
#include <vector>

#include "../../include/pa.h"
#include "pa_internal.h"

namespace {

thread_local char g_detail[512];

pa_status fail(pa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
  va_end(ap);
  return st;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

bool is_gqa_pool(const pa_kv_pool* p) { return p->kv_dtype == PA_BF16; }

pa_status check_gqa_pool(const pa_kv_pool* p) {
  if (p == nullptr) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
  if (p->kv_dtype != PA_BF16) return fail(PA_ERR_UNSUPPORTED, "GQA pool must be PA_BF16");
  if (p->block_size != 16) return fail(PA_ERR_UNSUPPORTED, "GQA pool block_size must be 16 (got %d)", p->block_size);
  if (p->head_dim_qk != p->head_dim_v || (p->head_dim_qk != 64 && p->head_dim_qk != 128))
    return fail(PA_ERR_UNSUPPORTED, "GQA head_dim must be 64 or 128 with head_dim_qk == head_dim_v");
  if (p->num_kv_heads < 1 || p->num_blocks < 1) return fail(PA_ERR_INVALID_ARG, "num_kv_heads and num_blocks must be >= 1");
  if (p->k == nullptr || p->v == nullptr) return fail(PA_ERR_INVALID_ARG, "pool k/v is NULL");
  if (!aligned(p->k, 16) || !aligned(p->v, 16)) return fail(PA_ERR_INVALID_ARG, "pool k/v must be 16-byte aligned");
  return PA_OK;
}

bool is_packed_pool(const pa_kv_pool* p) { return p->kv_dtype == PA_PACKED_MLA; }

pa_status check_fp8_pool(const pa_kv_pool* p, int d_qk, int d_v, const char* what) {
  if (p == nullptr) return fail(PA_ERR_INVALID_ARG, "%s pool is NULL", what);
  if (is_packed_pool(p)) {
    if (p->block_size != 64 || p->num_kv_heads != 1 || p->head_dim_qk != d_qk || p->head_dim_v != d_v)
      return fail(PA_ERR_UNSUPPORTED, "%s view of a packed pool must be block 64, one head, dims %d/%d", what,
                  d_qk, d_v);
    if (p->num_blocks < 1) return fail(PA_ERR_INVALID_ARG, "num_blocks must be >= 1");
    if (p->num_blocks > INT32_MAX / 64) return fail(PA_ERR_UNSUPPORTED, "%s pool: num_blocks * 64 rows must fit in int32", what);
    if (p->k == nullptr) return fail(PA_ERR_INVALID_ARG, "%s packed pool k is NULL", what);
    if (!aligned(p->k, 16)) return fail(PA_ERR_INVALID_ARG, "%s packed pool must be 16-byte aligned", what);
    return PA_OK;
  }
  if (p->kv_dtype != PA_FP8_E4M3) return fail(PA_ERR_UNSUPPORTED, "%s pool must be PA_FP8_E4M3 or PA_PACKED_MLA", what);
  if (p->block_size != 64) return fail(PA_ERR_UNSUPPORTED, "%s pool block_size must be 64 (got %d)", what, p->block_size);
  if (p->num_kv_heads != 1) return fail(PA_ERR_UNSUPPORTED, "%s pool must have num_kv_heads == 1", what);
  if (p->head_dim_qk != d_qk || p->head_dim_v != d_v)
    return fail(PA_ERR_UNSUPPORTED, "%s pool head dims must be %d/%d (got %d/%d)", what, d_qk, d_v,
                p->head_dim_qk, p->head_dim_v);
  if (p->num_blocks < 1) return fail(PA_ERR_INVALID_ARG, "num_blocks must be >= 1");
  if (p->num_blocks > INT32_MAX / 64) return fail(PA_ERR_UNSUPPORTED, "%s pool: num_blocks * 64 rows must fit in int32", what);
  if (p->k == nullptr || p->scale == nullptr) return fail(PA_ERR_INVALID_ARG, "%s pool k/scale is NULL", what);
  if (!aligned(p->k, 16) || !aligned(p->scale, 4)) return fail(PA_ERR_INVALID_ARG, "%s pool must be 16-byte aligned", what);
  return PA_OK;
}

// Rows of one cache group of an FP8 pool or of a view of a packed pool: row r of block b
// at rows + b * blk + r * row_bytes, its 4 scale bytes at scales + b * sblk + 4 r.
struct RowView {
  const uint8_t* rows;
  const uint8_t* scales;
  int64_t blk, sblk;
  int32_t row_bytes, fp4;
};

constexpr int64_t kPackedBlock = 41472, kPackedLatentScale = 36864, kPackedKeys = 37120, kPackedKeyScales = 41216;

RowView row_view(const pa_kv_pool* p) {
  RowView v{};
  const uint8_t* base = static_cast<const uint8_t*>(p->k);
  if (is_packed_pool(p)) {
    v.blk = v.sblk = kPackedBlock;
    if (p->head_dim_qk == 576) {
      v.rows = base;
      v.scales = base + kPackedLatentScale;
      v.row_bytes = 576;
    } else {
      v.rows = base + kPackedKeys;
      v.scales = base + kPackedKeyScales;
      v.row_bytes = 64;
      v.fp4 = 1;
    }
    return v;
  }
  v.rows = base;
  v.scales = reinterpret_cast<const uint8_t*>(p->scale);
  v.blk = (int64_t)p->block_size * p->head_dim_qk;
  v.sblk = (int64_t)p->block_size * 4;
  v.row_bytes = p->head_dim_qk;
  return v;
}

pa_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return PA_OK;
}

// ---- optional per-launch timing (pa_profile_*): events recorded on the call's stream
struct ProfRec {
  const char* name;
  int slot;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
char g_prof_only[64] = "";                // empty: every launch is recorded
std::vector<hipEvent_t> g_prof_events;   // 2 per record slot
std::vector<ProfRec> g_prof_recs;

template <class F>
hipError_t timed(const char* name, hipStream_t stream, F&& launch) {
  int slot = -1;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (g_prof_on && g_prof_recs.size() * 2 < g_prof_events.size() &&
        (g_prof_only[0] == 0 || strcmp(g_prof_only, name) == 0)) {
      slot = (int)g_prof_recs.size();
      g_prof_recs.push_back({name, slot});
    }
  }
  if (slot >= 0) hipEventRecord(g_prof_events[2 * slot], stream);
  const hipError_t e = launch();
  if (slot >= 0) hipEventRecord(g_prof_events[2 * slot + 1], stream);
  return e;
}

#define PA_TRY(x)                       \
  do {                                  \
    const pa_status st_ = (x);          \
    if (st_ != PA_OK) return st_;       \
  } while (0)

// ---- decode workspace layouts
// MLA: partial outputs [S][max_splits][rows][512] then partial log2-sum-exp.
// GQA: piece partials, partial log2-sum-exp, the pass lists, pass counts, region starts
// and piece starts (each part 256-byte aligned).
struct DecodeLayout {
  int max_splits, rows, d_v, split;
  pa::GqaDecodeDims dims;
  size_t o_bytes, lse_bytes, pass_bytes, npass_bytes, rstart_bytes, pstart_bytes;
  size_t total() const { return o_bytes + lse_bytes + pass_bytes + npass_bytes + rstart_bytes + pstart_bytes; }
};

DecodeLayout decode_layout(int num_seqs, int q_per_seq, int num_q_heads, int max_context_len,
                           const pa_kv_pool* pool) {
  DecodeLayout l{};
  l.rows = q_per_seq * num_q_heads;
  l.d_v = pool->head_dim_v;
  if (!is_gqa_pool(pool)) {
    l.split = pa::kDecodeSplitMla;
    l.max_splits = max_context_len > 0 ? ceil_div(max_context_len, l.split) : 0;
    l.o_bytes = round_up((size_t)num_seqs * l.max_splits * l.rows * l.d_v * sizeof(float), 256);
    l.lse_bytes = round_up((size_t)num_seqs * l.max_splits * l.rows * sizeof(float), 256);
    return l;
  }
  const int hkv = pool->num_kv_heads;
  l.dims = pa::gqa_decode_dims(num_seqs, q_per_seq, num_q_heads, hkv, max_context_len);
  const size_t regions = (size_t)l.dims.n_groups * l.dims.n_chunks;
  const size_t slots = (size_t)l.dims.pieces_cap * l.dims.subs * hkv * 32;
  l.o_bytes = round_up(slots * l.d_v * sizeof(float), 256);
  l.lse_bytes = round_up(slots * sizeof(float), 256);
  l.pass_bytes = round_up(regions * l.dims.region_cap * 16, 256);
  l.npass_bytes = round_up(regions * sizeof(int32_t), 256);
  l.rstart_bytes = round_up((regions + 1) * sizeof(int32_t), 256);
  l.pstart_bytes = round_up(((size_t)l.dims.n_groups + 1) * sizeof(int32_t), 256);
  return l;
}

}  // namespace

extern "C" {

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    default: return "PA_ERR_UNKNOWN";
  }
}

const char* pa_last_error_detail(void) { return g_detail; }

int32_t pa_version(void) { return 1; }

// ------------------------------------------------------------------------- prefill
// Split-K prefill workspace: partial o [num_seqs * max_new_len][max_splits][num_q_heads][d]
// fp32, then the partial log2-sum-exp (each part 256-byte aligned).
struct PrefillLayout {
  int split_len, max_splits;
  size_t o_bytes, lse_bytes;
  size_t total() const { return o_bytes + lse_bytes; }
};

PrefillLayout prefill_layout(int32_t num_seqs, int32_t num_q_heads, int32_t max_new_len,
                             int32_t max_total_len, const pa_kv_pool* pool) {
  PrefillLayout l{};
  if (pool == nullptr || pool->num_kv_heads < 1 || num_q_heads < 1 || num_seqs < 1 || max_new_len < 1) return l;
  l.split_len = pa::prefill_split_len(num_seqs, num_q_heads, pool->num_kv_heads, max_new_len, max_total_len);
  if (l.split_len == 0) return l;
  l.max_splits = ceil_div(max_total_len, l.split_len);
  const size_t rows = (size_t)num_seqs * max_new_len * l.max_splits * num_q_heads;
  l.o_bytes = round_up(rows * pool->head_dim_v * sizeof(float), 256);
  l.lse_bytes = round_up(rows * sizeof(float), 256);
  return l;
}

size_t paged_attn_prefill_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t max_new_len,
                                         int32_t max_total_len, const pa_kv_pool* pool) {
  return prefill_layout(num_seqs, num_q_heads, max_new_len, max_total_len, pool).total();
}

pa_status paged_attn_prefill(const void* q, const pa_kv_pool* pool, const int32_t* block_table,
                             int32_t bt_stride, const int32_t* cached_len, const int32_t* new_len,
                             const int32_t* q_start, int32_t num_seqs, int32_t num_q_heads,
                             int32_t max_new_len, int32_t max_total_len, float scale, void* out,
                             float* lse, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  g_detail[0] = 0;
  PA_TRY(check_gqa_pool(pool));
  if (q == nullptr || out == nullptr || block_table == nullptr || cached_len == nullptr ||
      new_len == nullptr || q_start == nullptr)
    return fail(PA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(PA_ERR_INVALID_ARG, "q/out must be 16-byte aligned");
  if (num_seqs < 0 || max_new_len < 0 || max_total_len < 0 || bt_stride < 1)
    return fail(PA_ERR_INVALID_ARG, "negative size or bt_stride < 1");
  if (num_q_heads < 1 || num_q_heads % pool->num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads must be a positive multiple of num_kv_heads");
  const int G = num_q_heads / pool->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(PA_ERR_UNSUPPORTED, "group size %d not in {1,2,4,8}", G);
  if ((long)bt_stride * pool->block_size < max_total_len)
    return fail(PA_ERR_INVALID_ARG, "bt_stride * block_size < max_total_len");
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (num_seqs == 0 || max_new_len == 0) return PA_OK;
  const PrefillLayout l = prefill_layout(num_seqs, num_q_heads, max_new_len, max_total_len, pool);
  if (l.total() > 0) {
    if (workspace == nullptr || workspace_bytes < l.total())
      return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", l.total(), workspace_bytes);
    if (!aligned(workspace, 16)) return fail(PA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  pa::GqaPrefillArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(pool->k);
  a.v = static_cast<const uint16_t*>(pool->v);
  a.bt = block_table;
  a.cached_len = cached_len;
  a.new_len = new_len;
  a.q_start = q_start;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.bt_stride = bt_stride;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.head_dim = pool->head_dim_qk;
  a.num_blocks = pool->num_blocks;
  a.max_new_len = max_new_len;
  a.max_total_len = max_total_len;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.split_len = l.split_len;
  a.max_splits = l.max_splits;
  if (l.split_len > 0) {
    a.part_o = static_cast<float*>(workspace);
    a.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + l.o_bytes);
  }
  (void)hipGetLastError();
  PA_TRY(launched(timed("prefill_gqa", stream, [&] { return pa::launch_gqa_prefill(a, stream); }), "prefill launch"));
  if (l.split_len == 0) return PA_OK;
  pa::CombineArgs c{};
  c.part_o = a.part_o;
  c.part_lse = a.part_lse;
  c.out = a.out;
  c.lse = lse;
  c.num_seqs = num_seqs;
  c.rows = num_q_heads;
  c.head_dim = pool->head_dim_v;
  c.max_splits = l.max_splits;
  c.split = l.split_len;
  c.max_context_len = max_total_len;
  c.pf_q_start = q_start;
  c.pf_cached = cached_len;
  c.pf_new_len = new_len;
  c.pf_max_new = max_new_len;
  c.pf_max_total = max_total_len;
  return launched(timed("combine", stream, [&] { return pa::launch_combine(c, stream); }), "prefill combine launch");
}

// ------------------------------------------------------------------------- decode
static pa_status check_decode(const pa_kv_pool* pool, int32_t num_seqs, int32_t q_per_seq,
                              int32_t num_q_heads, int32_t max_context_len, int32_t bt_stride) {
  if (pool == nullptr) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
  if (num_seqs < 0 || max_context_len < 0 || bt_stride < 1)
    return fail(PA_ERR_INVALID_ARG, "negative size or bt_stride < 1");
  if (q_per_seq < 1 || q_per_seq > 4) return fail(PA_ERR_UNSUPPORTED, "q_per_seq must be 1..4");
  if (is_gqa_pool(pool)) {
    PA_TRY(check_gqa_pool(pool));
    if (num_q_heads < 1 || num_q_heads % pool->num_kv_heads != 0)
      return fail(PA_ERR_INVALID_ARG, "num_q_heads must be a positive multiple of num_kv_heads");
    const int G = num_q_heads / pool->num_kv_heads;
    if (G > 16 || q_per_seq * G > 16)
      return fail(PA_ERR_UNSUPPORTED, "q_per_seq * group size must be <= 16 (got %d)", q_per_seq * G);
  } else {
    PA_TRY(check_fp8_pool(pool, 576, 512, "MLA"));
    if (num_q_heads < 1 || num_q_heads > 128 || num_q_heads % 16 != 0)
      return fail(PA_ERR_UNSUPPORTED, "MLA num_q_heads must be a multiple of 16 up to 128");
  }
  if ((long)bt_stride * pool->block_size < max_context_len)
    return fail(PA_ERR_INVALID_ARG, "bt_stride * block_size < max_context_len");
  return PA_OK;
}

size_t paged_attn_decode_workspace_size(int32_t num_seqs, int32_t q_per_seq, int32_t num_q_heads,
                                        int32_t max_context_len, const pa_kv_pool* pool) {
  if (pool == nullptr || num_seqs < 0 || q_per_seq < 1 || num_q_heads < 1 || max_context_len < 0) return 0;
  if (is_gqa_pool(pool) && (pool->num_kv_heads < 1 || num_q_heads % pool->num_kv_heads != 0)) return 0;
  return decode_layout(num_seqs, q_per_seq, num_q_heads, max_context_len, pool).total();
}

static pa_status decode_impl(const void* q, const pa_kv_pool* pool, const int32_t* block_table,
                             int32_t bt_stride, const int32_t* context_len, int32_t num_seqs,
                             int32_t q_per_seq, int32_t num_q_heads, int32_t max_context_len,
                             float scale, void* out, float* lse, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  PA_TRY(check_decode(pool, num_seqs, q_per_seq, num_q_heads, max_context_len, bt_stride));
  if (q == nullptr || out == nullptr || block_table == nullptr || context_len == nullptr)
    return fail(PA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(PA_ERR_INVALID_ARG, "q/out must be 16-byte aligned");
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale must be finite and > 0");
  const bool mla = !is_gqa_pool(pool);
  const DecodeLayout l = decode_layout(num_seqs, q_per_seq, num_q_heads, max_context_len, pool);
  if (num_seqs == 0 || max_context_len == 0) return PA_OK;
  if (workspace == nullptr || workspace_bytes < l.total())
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", l.total(), workspace_bytes);
  if (!aligned(workspace, 16)) return fail(PA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  char* ws = static_cast<char*>(workspace);
  float* part_o = reinterpret_cast<float*>(ws);
  float* part_lse = reinterpret_cast<float*>(ws + l.o_bytes);
  pa::CombineArgs c{};
  (void)hipGetLastError();
  if (!mla) {
    pa::GqaDecodeArgs a{};
    size_t off = l.o_bytes + l.lse_bytes;
    a.passes = reinterpret_cast<uint32_t*>(ws + off);
    off += l.pass_bytes;
    a.n_passes = reinterpret_cast<int32_t*>(ws + off);
    off += l.npass_bytes;
    a.region_start = reinterpret_cast<int32_t*>(ws + off);
    off += l.rstart_bytes;
    a.piece_start = reinterpret_cast<int32_t*>(ws + off);
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(pool->k);
    a.v = static_cast<const uint16_t*>(pool->v);
    a.bt = block_table;
    a.context_len = context_len;
    a.part_o = part_o;
    a.part_lse = part_lse;
    a.bt_stride = bt_stride;
    a.num_seqs = num_seqs;
    a.q_per_seq = q_per_seq;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = pool->num_kv_heads;
    a.head_dim = pool->head_dim_qk;
    a.num_blocks = pool->num_blocks;
    a.max_context_len = max_context_len;
    a.dims = l.dims;
    a.scale_log2 = scale * 1.4426950408889634f;
    PA_TRY(launched(timed("decode_plan", stream, [&] { return pa::launch_gqa_decode_plan(a, stream); }), "decode plan launch"));
    PA_TRY(launched(timed("decode_gqa", stream, [&] { return pa::launch_gqa_decode(a, stream); }), "decode launch"));
    c.piece_start = a.piece_start;
    c.subs = l.dims.subs;
    c.members = l.dims.members;
    c.num_kv_heads = pool->num_kv_heads;
    c.q_per_seq = q_per_seq;
  } else {
    pa::MlaDecodeArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    const RowView rv = row_view(pool);
    a.kv = rv.rows;
    a.kv_sbase = rv.scales;
    a.blk_bytes = rv.blk;
    a.sblk_bytes = rv.sblk;
    a.bt = block_table;
    a.context_len = context_len;
    a.part_o = part_o;
    a.part_lse = part_lse;
    a.bt_stride = bt_stride;
    a.num_seqs = num_seqs;
    a.q_per_seq = q_per_seq;
    a.num_q_heads = num_q_heads;
    a.num_blocks = pool->num_blocks;
    a.max_context_len = max_context_len;
    a.max_splits = l.max_splits;
    a.scale_log2 = scale * 1.4426950408889634f;
    PA_TRY(launched(timed("decode_mla", stream, [&] { return pa::launch_mla_decode(a, stream); }), "MLA decode launch"));
  }
  c.part_o = part_o;
  c.part_lse = part_lse;
  c.context_len = context_len;
  c.out = static_cast<uint16_t*>(out);
  c.lse = lse;
  c.num_seqs = num_seqs;
  c.rows = l.rows;
  c.head_dim = pool->head_dim_v;
  c.max_splits = l.max_splits;
  c.split = l.split;
  c.max_context_len = max_context_len;
  return launched(timed("combine", stream, [&] { return pa::launch_combine(c, stream); }), "combine launch");
}

pa_status paged_attn_decode(const void* q, const pa_kv_pool* pool, const int32_t* block_table,
                            int32_t bt_stride, const int32_t* context_len, int32_t num_seqs,
                            int32_t q_per_seq, int32_t num_q_heads, int32_t max_context_len,
                            float scale, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  g_detail[0] = 0;
  return decode_impl(q, pool, block_table, bt_stride, context_len, num_seqs, q_per_seq, num_q_heads,
                     max_context_len, scale, out, lse, workspace, workspace_bytes, stream);
}

// Decode without a caller workspace: the same kernels run on a fixed scratch array that
// the library keeps in device memory, one copy per GPU (a __device__ variable exists
// once in every device's copy of the code object).  The host-side name `scratch` is not a
// device address; the address of the current device's copy comes from
// hipGetSymbolAddress, looked up once per device (with that device current) and kept.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

static pa_status device_scratch(void** ptr) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(PA_ERR_UNSUPPORTED, "device %d beyond the scratch table", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t g = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (g != hipSuccess || p == nullptr)
      return fail(PA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(g));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PA_OK;
}

size_t paged_attn_decode_noalloc_max_bytes(void) { return PA_NOALLOC_SCRATCH_BYTES; }

pa_status paged_attn_decode_noalloc(const void* q, const pa_kv_pool* pool, const int32_t* block_table,
                                    int32_t bt_stride, const int32_t* context_len, int32_t num_seqs,
                                    int32_t q_per_seq, int32_t num_q_heads, int32_t max_context_len,
                                    float scale, void* out, float* lse, hipStream_t stream) {
  g_detail[0] = 0;
  PA_TRY(check_decode(pool, num_seqs, q_per_seq, num_q_heads, max_context_len, bt_stride));
  const size_t need = decode_layout(num_seqs, q_per_seq, num_q_heads, max_context_len, pool).total();
  if (need > (size_t)PA_NOALLOC_SCRATCH_BYTES)
    return fail(PA_ERR_WORKSPACE,
                "paged_attn_decode_noalloc: these sizes need %zu bytes of scratch, more than the %zu the "
                "library holds; use paged_attn_decode with a caller workspace",
                need, (size_t)PA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  PA_TRY(device_scratch(&ws));
  return decode_impl(q, pool, block_table, bt_stride, context_len, num_seqs, q_per_seq, num_q_heads,
                     max_context_len, scale, out, lse, ws, (size_t)PA_NOALLOC_SCRATCH_BYTES, stream);
}

// ------------------------------------------------------------------------- indexer + top-k
static size_t idx_scores_bytes(int32_t n_q, int32_t max_total_len) {
  return round_up((size_t)n_q * max_total_len * sizeof(float), 256);
}

size_t mla_indexer_topk_workspace_size(int32_t n_q, int32_t num_idx_heads, int32_t max_total_len,
                                       int32_t k) {
  (void)num_idx_heads;
  (void)k;
  if (n_q < 0 || max_total_len < 0) return 0;
  return idx_scores_bytes(n_q, max_total_len) + round_up((size_t)n_q * sizeof(int32_t), 256);
}

pa_status mla_indexer_topk(const void* q_idx, const float* w, const pa_kv_pool* idx_pool,
                           const int32_t* block_table, int32_t bt_stride,
                           const int32_t* cached_len, const int32_t* new_len,
                           const int32_t* q_start, int32_t num_seqs, int32_t n_q,
                           int32_t num_idx_heads, int32_t max_new_len, int32_t max_total_len,
                           int32_t k, int32_t* topk_idx, float* scores_out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  g_detail[0] = 0;
  PA_TRY(check_fp8_pool(idx_pool, 128, 0, "indexer"));
  if (q_idx == nullptr || w == nullptr || block_table == nullptr || cached_len == nullptr ||
      new_len == nullptr || q_start == nullptr || topk_idx == nullptr)
    return fail(PA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(q_idx, 16) || !aligned(w, 4) || (scores_out && !aligned(scores_out, 4)))
    return fail(PA_ERR_INVALID_ARG, "misaligned pointer");
  if (num_seqs < 0 || n_q < 0 || max_new_len < 0 || max_total_len < 0 || bt_stride < 1)
    return fail(PA_ERR_INVALID_ARG, "negative size or bt_stride < 1");
  if (num_idx_heads < 16 || num_idx_heads > 64 || num_idx_heads % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "num_idx_heads must be 16, 32, 48 or 64");
  if (k < 1 || k > 4096) return fail(PA_ERR_UNSUPPORTED, "k must be 1..4096");
  if ((long)bt_stride * idx_pool->block_size < max_total_len)
    return fail(PA_ERR_INVALID_ARG, "bt_stride * block_size < max_total_len");
  const size_t need = mla_indexer_topk_workspace_size(n_q, num_idx_heads, max_total_len, k);
  if (n_q == 0 || num_seqs == 0) return PA_OK;
  if (workspace == nullptr || workspace_bytes < need)
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  if (!aligned(workspace, 16)) return fail(PA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  float* scores = scores_out ? scores_out : static_cast<float*>(workspace);
  int32_t* valid = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + idx_scores_bytes(n_q, max_total_len));
  (void)hipGetLastError();
  pa::IndexerArgs a{};
  a.q_idx = static_cast<const uint16_t*>(q_idx);
  a.w = w;
  const RowView rv = row_view(idx_pool);
  a.keys = rv.rows;
  a.key_sbase = rv.scales;
  a.blk_bytes = rv.blk;
  a.sblk_bytes = rv.sblk;
  a.fp4 = rv.fp4;
  a.bt = block_table;
  a.cached_len = cached_len;
  a.new_len = new_len;
  a.q_start = q_start;
  a.scores = scores;
  a.valid_len = valid;
  a.bt_stride = bt_stride;
  a.num_seqs = num_seqs;
  a.n_q = n_q;
  a.num_heads = num_idx_heads;
  a.num_blocks = idx_pool->num_blocks;
  a.max_new_len = max_new_len;
  a.max_total_len = max_total_len;
  a.score_stride = max_total_len;
  PA_TRY(launched(timed("indexer", stream, [&] { return pa::launch_indexer_scores(a, stream); }), "indexer launch"));
  pa::TopkArgs t{};
  t.scores = scores;
  t.valid_len = valid;
  t.out = topk_idx;
  t.n_rows = n_q;
  t.row_stride = max_total_len;
  t.k = k;
  t.max_valid = max_total_len;
  return launched(timed("topk", stream, [&] { return pa::launch_topk(t, stream); }), "top-k launch");
}

// ------------------------------------------------------------------------- sparse MLA
size_t sparse_mla_attn_workspace_size(int32_t, int32_t, int32_t) { return 0; }

pa_status sparse_mla_attn(const void* q, const pa_kv_pool* pool, const int32_t* block_table,
                          int32_t bt_stride, const int32_t* q_seq, const int32_t* topk_idx,
                          int32_t n_q, int32_t k, int32_t num_q_heads, float scale, void* out,
                          float* lse, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  (void)workspace;
  (void)workspace_bytes;
  g_detail[0] = 0;
  PA_TRY(check_fp8_pool(pool, 576, 512, "MLA"));
  if (q == nullptr || out == nullptr || block_table == nullptr || q_seq == nullptr || topk_idx == nullptr)
    return fail(PA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(PA_ERR_INVALID_ARG, "q/out must be 16-byte aligned");
  if (n_q < 0 || bt_stride < 1) return fail(PA_ERR_INVALID_ARG, "negative size or bt_stride < 1");
  if (k < 1 || k > 8192) return fail(PA_ERR_UNSUPPORTED, "k must be 1..8192");
  if (num_q_heads < 16 || num_q_heads > 128 || num_q_heads % 16 != 0 || (num_q_heads > 64 && num_q_heads % 64 != 0))
    return fail(PA_ERR_UNSUPPORTED, "num_q_heads must be 16..64 in steps of 16, or 128");
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (n_q == 0) return PA_OK;
  (void)hipGetLastError();
  pa::SparseMlaArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  const RowView rv = row_view(pool);
  a.kv = rv.rows;
  a.kv_sbase = rv.scales;
  a.blk_bytes = rv.blk;
  a.sblk_bytes = rv.sblk;
  a.bt = block_table;
  a.q_seq = q_seq;
  a.topk = topk_idx;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.bt_stride = bt_stride;
  a.n_q = n_q;
  a.k = k;
  a.num_q_heads = num_q_heads;
  a.num_blocks = pool->num_blocks;
  a.scale_log2 = scale * 1.4426950408889634f;
  return launched(timed("sparse_mla", stream, [&] { return pa::launch_sparse_mla(a, stream); }), "sparse MLA launch");
}

// ------------------------------------------------------------------------- KV append
pa_status paged_kv_append(const pa_kv_pool* pool, const int32_t* block_table, int32_t bt_stride,
                          const int32_t* cached_len, const int32_t* new_len, const int32_t* q_start,
                          int32_t num_seqs, int32_t n_tokens, int32_t max_new_len, const void* k_new,
                          const void* v_new, hipStream_t stream) {
  g_detail[0] = 0;
  if (pool == nullptr) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
  const bool fp8 = pool->kv_dtype == PA_FP8_E4M3 || is_packed_pool(pool);
  if (fp8) {
    if (pool->head_dim_qk == 576)
      PA_TRY(check_fp8_pool(pool, 576, 512, "MLA"));
    else
      PA_TRY(check_fp8_pool(pool, 128, 0, "indexer"));
  } else {
    PA_TRY(check_gqa_pool(pool));
    if (v_new == nullptr) return fail(PA_ERR_INVALID_ARG, "v_new is NULL for a bf16 pool");
    if (!aligned(v_new, 16)) return fail(PA_ERR_INVALID_ARG, "v_new must be 16-byte aligned");
  }
  if (num_seqs < 0 || n_tokens < 0 || max_new_len < 0) return fail(PA_ERR_INVALID_ARG, "negative size");
  if (num_seqs == 0 || n_tokens == 0 || max_new_len == 0) return PA_OK;
  if (bt_stride < 1) return fail(PA_ERR_INVALID_ARG, "bt_stride must be >= 1");
  if (block_table == nullptr || cached_len == nullptr || new_len == nullptr || q_start == nullptr ||
      k_new == nullptr)
    return fail(PA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(k_new, 16)) return fail(PA_ERR_INVALID_ARG, "k_new must be 16-byte aligned");
  if (num_seqs > 65535) return fail(PA_ERR_UNSUPPORTED, "num_seqs must be <= 65535");
  (void)hipGetLastError();
  pa::AppendArgs a{};
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.bt = block_table;
  a.cached_len = cached_len;
  a.new_len = new_len;
  a.q_start = q_start;
  // the pool descriptor's pointers are const for the attention calls; the append is the
  // one call that writes through them
  if (fp8) {
    const RowView rv = row_view(pool);
    a.fp8_out = const_cast<uint8_t*>(rv.rows);
    a.scale_out = const_cast<uint8_t*>(rv.scales);
    a.blk_bytes = rv.blk;
    a.sblk_bytes = rv.sblk;
    a.mxfp4 = rv.fp4;
  } else {
    a.k_out = static_cast<uint16_t*>(const_cast<void*>(pool->k));
    a.v_out = static_cast<uint16_t*>(const_cast<void*>(pool->v));
  }
  a.bt_stride = bt_stride;
  a.num_seqs = num_seqs;
  a.n_tokens = n_tokens;
  a.max_new_len = max_new_len;
  a.num_blocks = pool->num_blocks;
  a.block_size = pool->block_size;
  a.num_kv_heads = pool->num_kv_heads;
  a.head_dim = pool->head_dim_qk;
  a.is_fp8 = fp8 ? 1 : 0;
  const char* tname = !fp8 ? "append_gqa" : (a.mxfp4 ? "append_mxfp4" : "append_fp8");
  return launched(timed(tname, stream, [&] { return pa::launch_append(a, stream); }), "append launch");
}

// ------------------------------------------------------------------------- test hooks
pa_status pa_test_gather_kv(const pa_kv_pool* pool, const int32_t* block_table, int32_t bt_stride,
                            int32_t seq, int32_t n_tokens, void* k_out, void* v_out,
                            float* scale_out, hipStream_t stream) {
  g_detail[0] = 0;
  if (pool == nullptr || block_table == nullptr || k_out == nullptr)
    return fail(PA_ERR_INVALID_ARG, "a required pointer is NULL");
  const bool fp8 = pool->kv_dtype == PA_FP8_E4M3 || is_packed_pool(pool);
  if (fp8) {
    if (is_packed_pool(pool)) {
      PA_TRY(check_fp8_pool(pool, pool->head_dim_qk == 576 ? 576 : 128, pool->head_dim_qk == 576 ? 512 : 0, "gather"));
      if (scale_out == nullptr) return fail(PA_ERR_INVALID_ARG, "scale_out is NULL");
    } else if (pool->k == nullptr || pool->scale == nullptr || scale_out == nullptr || pool->num_kv_heads != 1 ||
               pool->head_dim_qk % 16 != 0 || pool->block_size < 1) {
      return fail(PA_ERR_INVALID_ARG, "bad FP8 pool for gather");
    }
  } else {
    PA_TRY(check_gqa_pool(pool));
    if (v_out == nullptr) return fail(PA_ERR_INVALID_ARG, "v_out is NULL");
  }
  if (seq < 0 || n_tokens < 0 || bt_stride < 1 || (long)bt_stride * pool->block_size < n_tokens)
    return fail(PA_ERR_INVALID_ARG, "bad seq / n_tokens / bt_stride");
  if (!aligned(k_out, 16) || (v_out && !aligned(v_out, 16))) return fail(PA_ERR_INVALID_ARG, "outputs must be 16-byte aligned");
  (void)hipGetLastError();
  pa::GatherArgs a{};
  a.k = pool->k;
  a.v = pool->v;
  if (fp8) {
    const RowView rv = row_view(pool);
    a.k = rv.rows;
    a.sbase = rv.scales;
    a.blk_bytes = rv.blk;
    a.sblk_bytes = rv.sblk;
  }
  a.bt_row = block_table + (size_t)seq * bt_stride;
  a.k_out = k_out;
  a.v_out = v_out;
  a.scale_out = scale_out;
  a.n_tokens = n_tokens;
  a.num_blocks = pool->num_blocks;
  a.block_size = pool->block_size;
  a.num_kv_heads = pool->num_kv_heads;
  a.row_bytes = fp8 ? row_view(pool).row_bytes : pool->head_dim_qk * 2;
  a.is_fp8 = fp8 ? 1 : 0;
  return launched(pa::launch_gather(a, stream), "gather launch");
}

size_t pa_test_topk_workspace_size(int32_t, int32_t) { return 0; }

pa_status pa_test_topk_from_scores(const float* scores, const int32_t* valid_len, int32_t n_rows,
                                   int32_t row_stride, int32_t k, int32_t* out_idx, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  (void)workspace;
  (void)workspace_bytes;
  g_detail[0] = 0;
  if (scores == nullptr || valid_len == nullptr || out_idx == nullptr)
    return fail(PA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (n_rows < 0 || row_stride < 0) return fail(PA_ERR_INVALID_ARG, "negative size");
  if (k < 1 || k > 4096) return fail(PA_ERR_UNSUPPORTED, "k must be 1..4096");
  (void)hipGetLastError();
  pa::TopkArgs t{};
  t.scores = scores;
  t.valid_len = valid_len;
  t.out = out_idx;
  t.n_rows = n_rows;
  t.row_stride = row_stride;
  t.k = k;
  t.max_valid = row_stride;
  return launched(timed("topk", stream, [&] { return pa::launch_topk(t, stream); }), "top-k launch");
}

// ------------------------------------------------------------------------- profiling
pa_status pa_profile_enable(int32_t max_records) {
  g_detail[0] = 0;
  if (max_records < 1 || max_records > (1 << 20)) return fail(PA_ERR_INVALID_ARG, "max_records must be 1..2^20");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (hipEvent_t e : g_prof_events) (void)hipEventDestroy(e);
  g_prof_events.assign(2 * (size_t)max_records, nullptr);
  // Timing-only events: without the system-scope fence a record neither writes back nor
  // invalidates the caches, so the instrumentation does not slow the launches it brackets.
  for (auto& e : g_prof_events)
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) {
      g_prof_events.clear();
      return fail(PA_ERR_HIP, "hipEventCreate failed");
    }
  g_prof_recs.clear();
  g_prof_on = true;
  return PA_OK;
}

pa_status pa_profile_select(const char* name) {
  g_detail[0] = 0;
  if (name != nullptr && strlen(name) >= sizeof(g_prof_only))
    return fail(PA_ERR_INVALID_ARG, "kernel name longer than %zu characters", sizeof(g_prof_only) - 1);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  snprintf(g_prof_only, sizeof(g_prof_only), "%s", name != nullptr ? name : "");
  return PA_OK;
}

int32_t pa_profile_count(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  return (int32_t)g_prof_recs.size();
}

pa_status pa_profile_record(int32_t i, char* name_out, int32_t name_cap, float* ms_out) {
  g_detail[0] = 0;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (i < 0 || i >= (int32_t)g_prof_recs.size() || ms_out == nullptr)
    return fail(PA_ERR_INVALID_ARG, "no profile record %d", i);
  const ProfRec& r = g_prof_recs[i];
  if (name_out && name_cap > 0) snprintf(name_out, (size_t)name_cap, "%s", r.name);
  if (hipEventSynchronize(g_prof_events[2 * r.slot + 1]) != hipSuccess ||
      hipEventElapsedTime(ms_out, g_prof_events[2 * r.slot], g_prof_events[2 * r.slot + 1]) != hipSuccess)
    return fail(PA_ERR_HIP, "event timing failed");
  return PA_OK;
}

pa_status pa_profile_disable(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = false;
  g_prof_only[0] = 0;
  for (hipEvent_t e : g_prof_events) (void)hipEventDestroy(e);
  g_prof_events.clear();
  g_prof_recs.clear();
  return PA_OK;
}

}  // extern "C"
