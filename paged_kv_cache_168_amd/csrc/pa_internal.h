// Launch descriptors shared by the C ABI (pa_api.cpp) and the gfx950 kernels (pa_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_host.h"

namespace pa {

// How a kernel's row item maps to a query row.
enum RowMode : int32_t {
  kDecodeSeqs = 0,       // item = request s, query row t = s, sees context_lens[s] keys
  kMixedDecodeSeqs = 1,  // item = request s; only requests with q_len == 1; t = query_start_loc[s]
  kAllTokens = 2,        // item = query row t; request found from query_start_loc; causal horizon
  kPrefillTokens = 3,    // as kAllTokens, but only rows of requests with q_len > 1
};


struct AttnArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start_loc;
  float* part_o;   // [T][Hq][P_max][D] un-normalised partition sums
  float* part_ml;  // [T][Hq][P_max][2] (reference max in log2 units, sum of weights)
  int32_t* seg_piece;        // balanced decode: [request][head group][partition] (first piece's partial slot, last
                             // piece's wave)
  const int32_t* tiles;      // prefill work list: (request, first row) pairs
  const int32_t* tile_count; // number of valid entries in `tiles`
  // element offset of (block b, slot o, kv head h, dim d) in either cache: b * block_stride + o * slot_stride +
  // h * head_stride + d (token-major: slot_stride = Hkv * D, head_stride = D; head-major: D and BS * D)
  int64_t block_stride, slot_stride, head_stride;
  int32_t head_major;  // 1: head-major layout
  int32_t num_seqs, num_tokens;
  int32_t num_q_heads, num_kv_heads, group;  // group = Hq / Hkv
  int32_t heads_per_wave, subgroups;         // group = heads_per_wave * subgroups
  int32_t block_size, num_blocks, max_blocks;
  int32_t partition_tokens, max_partitions;
  int32_t chunk_partition_tokens;  // MFMA chunk rows: keys per partition, 0 = one partition per row tile
  int32_t chunk_partitions;        // partitions in the MFMA grid (1 when chunk_partition_tokens == 0)
  int32_t mode;       // RowMode
  int32_t num_items;  // row items in the grid (requests or query rows)
  int32_t tile_capacity;
  int32_t num_waves;  // balanced decode: waves sharing the global tile sequence
  // balanced decode cut into context partitions (caller-set partition_tokens): 16-token tiles per partition
  // (0: no partitions); the softmax restarts at every partition start
  int32_t bal_part_tiles;
  float scale_log2;   // scale * log2(e)
  int32_t cache_kv;   // 1: cached K/V loads (blocks shared between requests); 0: streaming loads
  // shared-prefix decode (all null / 0 otherwise)
  const int32_t* group_start;   // [num_groups + 1]: requests group_start[g] .. group_start[g+1]-1 form group g
  const int32_t* group_prefix;  // [num_groups]: leading tokens whose blocks the group's requests share
  int32_t* item_prefix;         // [num_seqs]: shared-prefix tokens of each request (0: none)
  // partials of the shared-prefix pass, one per partition of prefix_part_tokens prefix keys:
  float* prefix_o;              // [num_seqs][Hq][prefix_parts][D] un-normalised
  float* prefix_ml;             // [num_seqs][Hq][prefix_parts][2] (reference max in log2 units, sum of weights)
  int32_t prefix_parts, prefix_part_tokens;
  float* seg_o;                 // [num_seqs][Hq][D] partials of suffix segments held by one wave
  float* seg_ml;                // [num_seqs][Hq][2]
  int32_t num_groups;
};

// KV-cache write: the new rows of num_tokens tokens into the caches.
struct CacheWriteArgs {
  void* k_cache;
  void* v_cache;
  const void* k_new;
  const void* v_new;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start_loc;  // nullptr: one token per request (token t of request t)
  int64_t block_bytes, slot_bytes, head_bytes;  // the cache strides of AttnArgs, in bytes
  int32_t head_bytes_len;                        // bytes of one kv head's row (head_dim * element size)
  int32_t num_seqs, num_tokens;
  int32_t block_size, num_blocks, max_blocks;
};

// Block copy: pair i copies block mapping[2i] of the source pools to block mapping[2i+1] of the
// destination pools (device addresses; a pinned host pool is passed by its device address).
struct CopyBlocksArgs {
  void* dst_k;
  void* dst_v;
  const void* src_k;
  const void* src_v;
  const int32_t* mapping;
  int64_t block_bytes;  // bytes of one block of one cache, a multiple of 16
  int32_t num_pairs, src_num_blocks, dst_num_blocks;
};

// All launchers return the HIP error of their launch (hipSuccess if nothing to do).
// Kernel timing: when start/stop events are given, the dominant kernels are launched with them
// attached (hipExtLaunchKernel), so the events carry the kernel's own start and end times.
struct KernelTiming {
  hipEvent_t start = nullptr, stop = nullptr;
};
hipError_t launch_decode(const AttnArgs& a, int dtype, int head_dim, bool uniform_blocks, hipStream_t s,
                         KernelTiming timing = {});
hipError_t launch_merge(const AttnArgs& a, int dtype, int head_dim, hipStream_t s);
// Balanced (stream-K) decode over requests whose blocks hold a multiple of 16 tokens, and the merge
// of segments that several waves shared (also writes zero rows).
hipError_t launch_decode_balanced(const AttnArgs& a, int dtype, int head_dim, hipStream_t s, KernelTiming timing = {});
hipError_t launch_merge_balanced(const AttnArgs& a, int dtype, int head_dim, hipStream_t s);
// Whether the balanced decode of bf16 (dtype 1) groups of heads_per_wave heads runs on the matrix cores:
// groups of eight always, groups of four when blocks are shared (cached loads); otherwise the vector ALUs.
inline bool balanced_uses_mfma(int dtype, int heads_per_wave, bool shared) {
  return dtype == 1 && (heads_per_wave == 8 || (shared && heads_per_wave >= 4));
}
// Bytes of partial results the balanced decode needs for a.num_waves waves.
size_t balanced_partial_bytes(int num_waves, int heads_per_wave, int head_dim, size_t* ml_bytes);
hipError_t launch_plan(const AttnArgs& a, int32_t* tiles, int32_t* tile_count, int rows_per_tile,
                       hipStream_t s);
// Shared-prefix decode: work list of the prefix pass (one (group, first row) entry per block of
// rows_per_tile requests of every group with a prefix) and the per-request prefix lengths.
hipError_t launch_prefix_plan(const AttnArgs& a, int32_t* tiles, int32_t* tile_count, int rows_per_tile,
                              hipStream_t s);
// beside_decode: the chunk tiles run concurrently with the balanced decode kernel; work-groups of one
// 4-wave half then fit next to the decode waves (one wave per SIMD each).
hipError_t launch_prefill(const AttnArgs& a, int head_dim, bool beside_decode, hipStream_t s,
                          KernelTiming timing = {});
// The shared-prefix pass: every request of a group against the group's prefix keys, as partials.
hipError_t launch_prefix_pass(const AttnArgs& a, int head_dim, hipStream_t s);
// block_bytes: bytes of one cache block, block_size * num_kv_heads * head_dim * element size.
bool prefill_supported(int dtype, int head_dim, int group, int64_t block_bytes);
int prefill_rows_per_tile(int group);
// row_bytes: bytes of one slot row, num_kv_heads * head_dim * element size (a multiple of 16).
hipError_t launch_cache_write(const CacheWriteArgs& a, int row_bytes, hipStream_t s, KernelTiming timing = {});
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t s, KernelTiming timing = {});
// Streaming-read reference: `chunks` 16-byte chunks at buf, over num_waves waves.
hipError_t launch_stream_read(const void* buf, int64_t chunks, int num_waves, uint32_t* sink, hipStream_t s,
                              KernelTiming timing = {});

}  // namespace pa
