// KV-cache write on gfx950: stores this step's new key and value rows in the paged cache, where the
// attention kernels read them.
//
// Token t is row j of request s; its absolute position is pos = ctx - q_len + j (context_lens counts
// the request's cached tokens including this step's, as in the attention). Logical block pos / BS of
// the request is physical block block_tables[s][pos / BS], slot pos % BS ("Continuous batching: a
// paradigm shift in inference throughput", section 2.2: the block table; "PagedAttention memory paging
// and continuous batching in practice", logical and physical blocks: a new token fills the next slot
// of a block allocated on demand). The slot row [num_kv_heads][head_dim] of k_new[t] and v_new[t] is
// copied with 16-byte lane loads and stores. A token whose position or block id falls outside the pool
// is skipped (a write is never clamped onto another block).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kCacheThreads = 256;

// One work-group per token; `chunks` 16-byte pieces per slot row of K (and as many of V).
__global__ __launch_bounds__(kCacheThreads) void cache_write_kernel(CacheWriteArgs a, int chunks) {
  const int t = blockIdx.x;
  int s = t, q0 = t, q_len = 1;
  if (a.query_start_loc != nullptr) {
    s = dev::find_request(a.query_start_loc, a.num_seqs, t);
    q0 = a.query_start_loc[s];
    q_len = a.query_start_loc[s + 1] - q0;
    if (t < q0 || t >= q0 + q_len) return;
  }
  const int pos = a.context_lens[s] - q_len + (t - q0);
  if (pos < 0 || pos >= a.max_blocks * a.block_size) return;
  const int blk = a.block_tables[(int64_t)s * a.max_blocks + pos / a.block_size];
  if (blk < 0 || blk >= a.num_blocks) return;
  const int64_t slot_row = (int64_t)blk * a.block_size + pos % a.block_size;
  const int64_t row_bytes = (int64_t)chunks * 16;
  for (int c = threadIdx.x; c < 2 * chunks; c += kCacheThreads) {
    const bool is_v = c >= chunks;
    const int64_t off = (int64_t)(is_v ? c - chunks : c) * 16;
    const char* src = static_cast<const char*>(is_v ? a.v_new : a.k_new) + (int64_t)t * row_bytes + off;
    char* dst = static_cast<char*>(is_v ? a.v_cache : a.k_cache) + slot_row * row_bytes + off;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteArgs& a, int row_bytes, hipStream_t s) {
  if (a.num_tokens <= 0) return hipSuccess;
  if (row_bytes % 16 != 0) return hipErrorInvalidValue;
  cache_write_kernel<<<dim3((unsigned)a.num_tokens), dim3(kCacheThreads), 0, s>>>(a, row_bytes / 16);
  return hipGetLastError();
}

}  // namespace pa
