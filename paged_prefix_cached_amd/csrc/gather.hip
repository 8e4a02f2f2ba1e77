// Test hook: copy one sequence's KV out of the paged pool into contiguous buffers with
// the same block-table walk (phys_block) the attention kernels use.  Bit-exact.
//
// Source: vLLM AgentX article (news.ainew.jp), "Hybrid KV cache management": one shared
// block pool; logical token t of a sequence is row t % block_size of physical block
// block_table[t / block_size].
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

// One thread per (token, head, 16-byte chunk).  GQA pools are [blocks][heads][bs][row];
// FP8 and packed views have one head: row r of block b at k + b * blk_bytes + r * row_bytes.
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  const int chunks = a.row_bytes / 16;
  const long total = (long)a.n_tokens * a.num_kv_heads * chunks;
  const long n_lblocks = (a.n_tokens + a.block_size - 1) / a.block_size;
  for (long idx = (long)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (long)gridDim.x * blockDim.x) {
    const int c = (int)(idx % chunks);
    const int h = (int)((idx / chunks) % a.num_kv_heads);
    const int t = (int)(idx / ((long)chunks * a.num_kv_heads));
    const int pb = phys_block(a.bt_row, t / a.block_size, (int)n_lblocks, a.num_blocks);
    const size_t b = (size_t)(pb < 0 ? 0 : pb), r = (size_t)(t % a.block_size);
    const size_t src = a.is_fp8 ? b * a.blk_bytes + r * a.row_bytes + 16 * c
                                : ((b * a.num_kv_heads + h) * a.block_size + r) * a.row_bytes + 16 * c;
    const size_t dst = ((size_t)t * a.num_kv_heads + h) * a.row_bytes + 16 * c;
    const u32x4 zero = {0, 0, 0, 0};
    st16(static_cast<uint8_t*>(a.k_out) + dst,
         pb >= 0 ? ld16(static_cast<const uint8_t*>(a.k) + src) : zero);
    if (!a.is_fp8)
      st16(static_cast<uint8_t*>(a.v_out) + dst,
           pb >= 0 ? ld16(static_cast<const uint8_t*>(a.v) + src) : zero);
    if (a.is_fp8 && c == 0)   // the row's 4 scale bytes (fp32, or 4 E8M0 codes), bit for bit
      a.scale_out[t] = pb >= 0 ? *reinterpret_cast<const float*>(a.sbase + b * a.sblk_bytes + 4 * r) : 0.f;
  }
}

}  // namespace

hipError_t launch_gather(const GatherArgs& a, hipStream_t stream) {
  const long total = (long)a.n_tokens * a.num_kv_heads * (a.row_bytes / 16);
  if (total == 0) return hipSuccess;
  const long blocks = (total + 255) / 256;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace pa
