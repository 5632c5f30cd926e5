// KV-cache write and block copy on gfx950.
//
// The cache write stores this step's new key and value rows in the paged cache, where the attention
// kernels read them.
//
// Token t is row j of request s; its absolute position is pos = ctx - q_len + j (context_lens counts
// the request's cached tokens including this step's, as in the attention). Logical block pos / BS of
// the request is physical block block_tables[s][pos / BS], slot pos % BS ("Continuous batching: a
// paradigm shift in inference throughput", section 2.2: the block table; "PagedAttention memory paging
// and continuous batching in practice", logical and physical blocks: a new token fills the next slot
// of a block allocated on demand). The row [num_kv_heads][head_dim] of k_new[t] and v_new[t] is
// copied with 16-byte lane loads and stores into the slot's rows, of either cache layout (one run in a
// token-major block, one run per kv head in a head-major block). A token whose position or block id
// falls outside the pool is skipped (a write is never clamped onto another block).
//
// The block copy moves whole physical blocks (K and V) from a source pool to a destination pool:
// copy-on-write of a shared block within one pool ("PagedAttention memory paging and continuous batching
// in practice", comparison table: copy-on-write and shared blocks; "Continuous batching", section 4.2),
// and swap of a preempted request's blocks between the GPU pool and a pinned host pool ("Continuous
// batching", section 3.3; "The PagedAttention mechanism in vLLM and memory optimisation practice",
// section 2.1, block-granular swap). Host memory is read and written by the kernel itself across the host
// link, so a scattered list of blocks is one launch. A pair with an id outside its pool is skipped.
#include <hip/hip_ext.h>
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
  // the slot's rows: at slot_bytes steps within the block, one kv head's row every head_bytes
  const int64_t slot_base = (int64_t)blk * a.block_bytes + (int64_t)(pos % a.block_size) * a.slot_bytes;
  const int64_t row_bytes = (int64_t)chunks * 16;
  for (int c = threadIdx.x; c < 2 * chunks; c += kCacheThreads) {
    const bool is_v = c >= chunks;
    const int off = (is_v ? c - chunks : c) * 16;  // within the token's [kv head][head_dim] row (< 2^31 bytes)
    const int h = off / a.head_bytes_len;
    const char* src = static_cast<const char*>(is_v ? a.v_new : a.k_new) + (int64_t)t * row_bytes + off;
    char* dst = static_cast<char*>(is_v ? a.v_cache : a.k_cache) + slot_base + (int64_t)h * a.head_bytes +
                (off - h * a.head_bytes_len);
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }
}

// Block copy: work-group (pair, cache, slice) moves up to kCopyChunks 16-byte pieces of one block of
// one cache; every lane issues all of its loads before its first store, so a work-group keeps 16 KB in
// flight (the host link's latency is a few microseconds, HBM's about one).
constexpr int kCopyPerLane = 4;
constexpr int kCopyChunks = kCacheThreads * kCopyPerLane;

__global__ __launch_bounds__(kCacheThreads) void copy_blocks_kernel(CopyBlocksArgs a, int slices) {
  const int slice = blockIdx.x % slices;
  const int pc = blockIdx.x / slices;
  const int pair = pc >> 1;
  const bool is_v = pc & 1;
  const int2 m = reinterpret_cast<const int2*>(a.mapping)[pair];
  if (m.x < 0 || m.x >= a.src_num_blocks || m.y < 0 || m.y >= a.dst_num_blocks) return;
  const int64_t chunks = a.block_bytes / 16;
  const uint4* src = reinterpret_cast<const uint4*>(static_cast<const char*>(is_v ? a.src_v : a.src_k) +
                                                    (int64_t)m.x * a.block_bytes);
  uint4* dst = reinterpret_cast<uint4*>(static_cast<char*>(is_v ? a.dst_v : a.dst_k) + (int64_t)m.y * a.block_bytes);
  const int64_t first = (int64_t)slice * kCopyChunks;
  if (first + kCopyChunks <= chunks) {  // a whole slice: unguarded, so the loads stay in flight together
    const uint4* sp = src + first + threadIdx.x;
    uint4* dp = dst + first + threadIdx.x;
    static_assert(kCopyPerLane == 4, "four named registers per lane");
    const uint4 x0 = sp[0], x1 = sp[kCacheThreads], x2 = sp[2 * kCacheThreads], x3 = sp[3 * kCacheThreads];
    dp[0] = x0;
    dp[kCacheThreads] = x1;
    dp[2 * kCacheThreads] = x2;
    dp[3 * kCacheThreads] = x3;
  } else {  // the block's last, partial slice
    for (int64_t c = first + threadIdx.x; c < chunks; c += kCacheThreads) dst[c] = src[c];
  }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t s, KernelTiming tm) {
  if (a.num_pairs <= 0) return hipSuccess;
  if (a.block_bytes <= 0 || a.block_bytes % 16 != 0) return hipErrorInvalidValue;
  const int64_t slices = (a.block_bytes / 16 + kCopyChunks - 1) / kCopyChunks;
  const int64_t grid = (int64_t)a.num_pairs * 2 * slices;
  if (slices > INT32_MAX || grid > INT32_MAX) return hipErrorInvalidValue;
  hipExtLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)grid), dim3(kCacheThreads), 0, s, tm.start, tm.stop, 0, a,
                        (int)slices);
  return hipGetLastError();
}

hipError_t launch_cache_write(const CacheWriteArgs& a, int row_bytes, hipStream_t s, KernelTiming tm) {
  if (a.num_tokens <= 0) return hipSuccess;
  if (row_bytes % 16 != 0) return hipErrorInvalidValue;
  hipExtLaunchKernelGGL(cache_write_kernel, dim3((unsigned)a.num_tokens), dim3(kCacheThreads), 0, s, tm.start, tm.stop,
                        0, a, row_bytes / 16);
  return hipGetLastError();
}

}  // namespace pa
