// C ABI of the paged-attention library: argument validation, path selection, workspace layout and
// kernel launches. Every check here runs on host scalars before the first HIP call, so invalid
// calls return a status without touching the device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "pa.h"
#include "pa_probe.h"
#include "pa_internal.h"

// Scratch memory of pa_decode_noalloc, for callers that cannot allocate: one copy per GPU the library
// runs on, held until the process ends. In host code `scratch` names a host-side stand-in, not device
// memory: kernels and copies are only ever given the device address that hipGetSymbolAddress returns
// for the current device, kept per device in g_scratch_ptr below.
static constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

using pa::fail;
using pa::validate_params;

thread_local hipEvent_t g_timing_start = nullptr;
thread_local hipEvent_t g_timing_stop = nullptr;

constexpr int kDefaultPartitionTokens = 512;
// Balanced decode: waves sharing the tile sequence. Private blocks (streaming loads): one wave per
// SIMD (256 CUs x 4) with a 3-tile prefetch ring; on the 8B-layer decode shape this reads as fast as
// 2048 waves (6.3 TB/s incremental at 2.4 GB per call) and splits fewer segments. Blocks shared
// between requests (cached loads): two waves per SIMD, which keeps more readers of a shared block in
// flight together (11% faster than 1024 waves on the 256-request prefix-shared batch).
constexpr int kBalancedMaxWaves = 1024;
constexpr int kBalancedMaxWavesShared = 2048;
// Groups of eight bf16 heads on private blocks run on the matrix cores with K and V staged in LDS (24 KB
// per wave): six waves per CU fit, and on the 8 x 32768 batch 1536 waves read faster than 1024 (kernel
// 165 vs 175 us). A step with chunk rows keeps 1024, so that the chunk tiles fit beside the decode waves.
constexpr int kBalancedMaxWavesMfma = 1536;
// Balanced decode requires contexts up to this many tokens (per-chunk tile sums stay in int32).
constexpr int64_t kBalancedMaxContext = int64_t(1) << 24;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// bytes of one cache block (either layout)
int64_t block_bytes(const pa_params* p) {
  return (int64_t)p->block_size * p->num_kv_heads * p->head_dim * (p->dtype == PA_DTYPE_BF16 ? 2 : 4);
}

// Everything the launches need, derived from host scalars only.
struct Plan {
  int group = 0, heads_per_wave = 0, subgroups = 0;
  int partition_tokens = 0, max_partitions = 0;
  bool uniform_blocks = false;
  size_t part_ml_bytes = 0, part_o_bytes = 0;
  // balanced decode
  bool balanced = false;
  int num_waves = 0;
  int bal_part_tiles = 0;  // caller-set partitions: tiles per partition (0: none)
  size_t bal_ml_bytes = 0, bal_part_bytes = 0, bal_range_bytes = 0, bal_bytes = 0;
};

Plan make_plan(const pa_params* p, int64_t rows) {
  Plan pl;
  pl.group = p->num_q_heads / p->num_kv_heads;
  const int g = pl.group;
  pl.heads_per_wave = (g == 1 || g == 2 || g == 4 || g == 8) ? g : (g % 8 == 0) ? 8 : (g % 4 == 0) ? 4 : (g % 2 == 0) ? 2 : 1;
  pl.subgroups = g / pl.heads_per_wave;
  pl.partition_tokens = p->partition_tokens ? p->partition_tokens : kDefaultPartitionTokens;
  const int64_t max_ctx = (int64_t)p->max_blocks_per_seq * p->block_size;
  pl.max_partitions = (int)((max_ctx + pl.partition_tokens - 1) / pl.partition_tokens);
  const int bs = p->block_size;
  pl.uniform_blocks = bs % pa::kTileTokens == 0 && pl.partition_tokens % bs == 0 && pl.partition_tokens / bs <= 64;
  if (pl.max_partitions > 1) {
    const int64_t slots = rows * p->num_q_heads * (int64_t)pl.max_partitions;
    pl.part_ml_bytes = align_up((size_t)slots * 2 * sizeof(float));
    pl.part_o_bytes = align_up((size_t)slots * p->head_dim * sizeof(float));
  }
  return pl;
}

// Balanced decode over `items` decode rows: eligible when a 16-token tile never straddles a block.
void plan_balanced(const pa_params* p, int64_t items, int64_t rows, Plan& pl) {
  const int64_t max_ctx = (int64_t)p->max_blocks_per_seq * p->block_size;
  // the tile descriptors hold a pool row in int32: block * block_size + slot (token-major), or
  // (block * num_kv_heads + kv head) * block_size + slot (head-major)
  const int64_t pool_rows = (int64_t)p->num_blocks * p->block_size *
                            (p->layout == PA_LAYOUT_HEAD_MAJOR ? p->num_kv_heads : 1);
  pl.balanced = p->block_size % pa::kTileTokens == 0 && max_ctx <= kBalancedMaxContext && pool_rows <= INT32_MAX &&
                items > 0;
  if (!pl.balanced) return;
  const int64_t max_tiles = items * ((max_ctx + pa::kTileTokens - 1) / pa::kTileTokens) *
                            p->num_kv_heads * pl.subgroups;
  const bool shared = (p->flags & PA_FLAG_SHARED_BLOCKS) != 0;
  const bool mfma_lds = !shared && pa::balanced_uses_mfma(p->dtype, pl.heads_per_wave, false);
  const int max_waves = shared ? kBalancedMaxWavesShared : (mfma_lds && rows == items) ? kBalancedMaxWavesMfma
                                                                                        : kBalancedMaxWaves;
  pl.num_waves = (int)std::max<int64_t>(1, std::min<int64_t>(max_waves, max_tiles));
  pl.bal_part_bytes = align_up(pa::balanced_partial_bytes(pl.num_waves, pl.heads_per_wave, p->head_dim, &pl.bal_ml_bytes));
  // A caller-set partition size restarts the softmax at every multiple of partition_tokens keys; the kernel
  // folds the partitions a wave holds in registers, and the merge folds the pieces of the waves.
  if (p->partition_tokens > 0 && pl.max_partitions > 1) pl.bal_part_tiles = p->partition_tokens / pa::kTileTokens;
  // one piece record per (request, head group)
  const int64_t groups = items * (p->num_q_heads / pl.heads_per_wave);
  pl.bal_range_bytes = align_up((size_t)groups * 2 * sizeof(int32_t));
  pl.bal_bytes = pl.bal_part_bytes + pl.bal_range_bytes;
}

// Balanced-decode arguments at the start of `ws`: the waves' partials and the piece records.
void set_balanced(pa::AttnArgs& d, const Plan& pl, void* ws) {
  char* w = static_cast<char*>(ws);
  d.part_ml = reinterpret_cast<float*>(w);
  d.part_o = reinterpret_cast<float*>(w + pl.bal_ml_bytes);
  d.seg_piece = reinterpret_cast<int32_t*>(w + pl.bal_part_bytes);
  d.num_waves = pl.num_waves;
  d.bal_part_tiles = pl.bal_part_tiles;
}

pa::AttnArgs base_args(const pa_params* p, const Plan& pl, int32_t num_seqs, int32_t num_tokens, void* out,
                       const void* q, const void* k, const void* v, const int32_t* bt, const int32_t* cl,
                       const int32_t* qsl, void* ws) {
  pa::AttnArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k;
  a.v_cache = v;
  a.block_tables = bt;
  a.context_lens = cl;
  a.query_start_loc = qsl;
  char* w = static_cast<char*>(ws);
  a.part_ml = pl.max_partitions > 1 ? reinterpret_cast<float*>(w) : nullptr;
  a.part_o = pl.max_partitions > 1 ? reinterpret_cast<float*>(w + pl.part_ml_bytes) : nullptr;
  const int64_t D = p->head_dim, Hkv = p->num_kv_heads, BS = p->block_size;
  a.head_major = p->layout == PA_LAYOUT_HEAD_MAJOR ? 1 : 0;
  a.block_stride = BS * Hkv * D;
  a.slot_stride = a.head_major ? D : Hkv * D;
  a.head_stride = a.head_major ? BS * D : D;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.num_q_heads = p->num_q_heads;
  a.num_kv_heads = p->num_kv_heads;
  a.group = pl.group;
  a.heads_per_wave = pl.heads_per_wave;
  a.subgroups = pl.subgroups;
  a.block_size = p->block_size;
  a.num_blocks = p->num_blocks;
  a.max_blocks = p->max_blocks_per_seq;
  a.partition_tokens = pl.partition_tokens;
  a.max_partitions = pl.max_partitions;
  a.chunk_partition_tokens = p->partition_tokens;  // 0: a chunk row tile covers all its keys
  a.chunk_partitions = p->partition_tokens > 0 ? pl.max_partitions : 1;
  a.scale_log2 = p->scale * 1.4426950408889634f;
  a.cache_kv = (p->flags & PA_FLAG_SHARED_BLOCKS) ? 1 : 0;
  return a;
}

bool grid_fits(int64_t blocks) { return blocks <= (int64_t)INT32_MAX; }

pa_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return PA_OK;
  std::snprintf(pa::error_detail(), pa::kDetailBytes, "%s: %s", where, hipGetErrorString(e));
  return PA_ERR_HIP;
}

// The caller's timing events for the next dominant launch (one-shot): they are attached to that
// launch (hipExtLaunchKernel), so they record the kernel's own start and end.
pa::KernelTiming take_timing() {
  pa::KernelTiming t;
  t.start = g_timing_start;
  t.stop = g_timing_stop;
  g_timing_start = g_timing_stop = nullptr;
  return t;
}

// Auxiliary stream of a mixed step, one per (calling thread, device), created on first use and kept
// until the process ends (never destroyed: a thread-exit destructor could run after the runtime is
// gone). Default priority; non-blocking, so it never synchronises implicitly with the null stream.
struct AuxStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxAuxDevices = 64;
thread_local AuxStream g_aux[kMaxAuxDevices];

// Sets *out to the auxiliary stream of the device `s` runs on, or to NULL when `s` belongs to a device
// other than the current one (the caller then stays on `s` alone).
pa_status aux_stream_for(hipStream_t s, AuxStream** out) {
  *out = nullptr;
  int cur = 0;
  pa_status st = hip_status(hipGetDevice(&cur), "hipGetDevice");
  if (st != PA_OK) return st;
  if (s != nullptr) {
    int dev = cur;
    st = hip_status(hipStreamGetDevice(s, &dev), "hipStreamGetDevice");
    if (st != PA_OK) return st;
    if (dev != cur) return PA_OK;
  }
  if (cur < 0 || cur >= kMaxAuxDevices) return PA_OK;
  AuxStream& x = g_aux[cur];
  if (x.stream == nullptr) {
    AuxStream n;
    st = hip_status(hipStreamCreateWithFlags(&n.stream, hipStreamNonBlocking), "auxiliary stream");
    // The events only order the two streams on one device (no host waits on them, and the caller's own
    // synchronisation on its stream covers the host's view), so they go without timing and without the
    // system-scope fence at each record.
    const unsigned ev_flags = hipEventDisableTiming | hipEventDisableSystemFence;
    if (st == PA_OK) st = hip_status(hipEventCreateWithFlags(&n.fork, ev_flags), "fork event");
    if (st == PA_OK) st = hip_status(hipEventCreateWithFlags(&n.join, ev_flags), "join event");
    if (st != PA_OK) {
      if (n.join) (void)hipEventDestroy(n.join);
      if (n.fork) (void)hipEventDestroy(n.fork);
      if (n.stream) (void)hipStreamDestroy(n.stream);
      return st;
    }
    x = n;
  }
  *out = &x;
  return PA_OK;
}

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxAuxDevices] = {};

// Device address of `scratch` on the current device (looked up once per device, with it current). The
// stream must belong to the current device.
pa_status scratch_for(hipStream_t s, void** out) {
  *out = nullptr;
  int cur = 0;
  pa_status st = hip_status(hipGetDevice(&cur), "hipGetDevice");
  if (st != PA_OK) return st;
  if (s != nullptr) {
    int dev = cur;
    st = hip_status(hipStreamGetDevice(s, &dev), "hipStreamGetDevice");
    if (st != PA_OK) return st;
    if (dev != cur) return fail(PA_ERR_INVALID_ARGUMENT, "stream belongs to a device other than the current one");
  }
  if (cur < 0 || cur >= kMaxAuxDevices) return fail(PA_ERR_UNSUPPORTED, "device index beyond the library's table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[cur] == nullptr) {
    void* p = nullptr;
    st = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (st != PA_OK) return st;
    g_scratch_ptr[cur] = p;
  }
  *out = g_scratch_ptr[cur];
  return PA_OK;
}

// The auxiliary stream and events of a call: the caller's (pa_varlen_mixed_ex / pa_decode_shared_ex), or the
// library's own for the calling thread and the stream's device (aux_stream_for).
pa_status resolve_aux(const pa_aux* user, hipStream_t s, AuxStream& tmp, AuxStream** out) {
  *out = nullptr;
  if (user == nullptr) return aux_stream_for(s, out);
  if (!user->stream || !user->fork_event || !user->join_event)
    return fail(PA_ERR_NULL_POINTER, "pa_aux needs a stream and both events");
  tmp.stream = static_cast<hipStream_t>(user->stream);
  tmp.fork = static_cast<hipEvent_t>(user->fork_event);
  tmp.join = static_cast<hipEvent_t>(user->join_event);
  *out = &tmp;
  return PA_OK;
}

// Mixed-step workspace: [balanced decode partials][chunk-row partition partials][prefill work list].
struct MixedLayout {
  Plan plan;
  bool use_prefill = false;  // MFMA tiles for q_len > 1 requests
  int rows_per_tile = 0;
  int64_t tile_capacity = 0;
  size_t rows_offset = 0, list_offset = 0, total = 0;
};

MixedLayout mixed_layout(const pa_params* p, int32_t num_seqs, int32_t num_tokens, int32_t max_query_len) {
  MixedLayout m;
  m.plan = make_plan(p, num_tokens);
  plan_balanced(p, num_seqs, num_tokens, m.plan);
  m.use_prefill = max_query_len > 1 && pa::prefill_supported(p->dtype, p->head_dim, m.plan.group, block_bytes(p));
  m.rows_offset = m.plan.balanced ? m.plan.bal_bytes : 0;
  m.list_offset = m.rows_offset;
  // partition partials: rows on the partition kernel, chunk rows cut into caller-set partitions
  if (!m.plan.balanced || (max_query_len > 1 && (p->partition_tokens > 0 || !m.use_prefill)))
    m.list_offset += m.plan.part_ml_bytes + m.plan.part_o_bytes;
  m.total = m.list_offset;
  if (m.use_prefill) {
    m.rows_per_tile = pa::prefill_rows_per_tile(m.plan.group);
    const int64_t bm = m.rows_per_tile;
    // tiles <= sum over prefill requests of ceil(q_len / bm); prefill requests <= min(S, T/2)
    const int64_t nreq = std::min<int64_t>(num_seqs, num_tokens / 2);
    const int64_t by_tokens = (num_tokens + nreq * (bm - 1)) / bm;
    const int64_t by_len = nreq * ((max_query_len + bm - 1) / bm);
    m.tile_capacity = std::max<int64_t>(1, std::min(by_tokens, by_len));
    m.total += align_up(sizeof(int32_t) * 4 + sizeof(int32_t) * 2 * (size_t)m.tile_capacity);
  }
  return m;
}

// A decode batch whose table holds at most one partition of keys per request can go to the partition kernel:
// one wave per (request, KV head, head subgroup) holds a whole context and writes its output directly, with no
// merge launch. That pays when every context is at most four tiles (the balanced split would cut them into
// pieces and merge them in a second launch: 6.2 against 8.8 us for 4 requests of up to 48 tokens), or when
// those waves alone fill the GPU four times over (2048 requests of up to 512 tokens, 8 KV heads: 405 against
// 436 us); in between the balanced split is faster (64 and 256 such requests: 23.3 and 56.8 us against 42.4
// and 60.3 us).
Plan decode_plan(const pa_params* params, int32_t num_seqs) {
  Plan pl = make_plan(params, num_seqs);
  const int64_t max_ctx = (int64_t)params->max_blocks_per_seq * params->block_size;
  const int64_t ctx_tiles = (max_ctx + pa::kTileTokens - 1) / pa::kTileTokens;
  const int64_t context_waves = (int64_t)num_seqs * params->num_kv_heads * pl.subgroups;
  const bool one_wave_per_context = pl.max_partitions == 1 && (ctx_tiles <= 4 || context_waves >= 4 * kBalancedMaxWaves);
  if (!one_wave_per_context) plan_balanced(params, num_seqs, num_seqs, pl);
  return pl;
}

size_t decode_workspace(const Plan& pl) { return pl.balanced ? pl.bal_bytes : pl.part_ml_bytes + pl.part_o_bytes; }

// Decode rows of a mixed step on the balanced kernel and its merge.
pa_status launch_balanced_rows(const pa::AttnArgs& d, const pa_params* p, hipStream_t s) {
  pa_status st;
  st = hip_status(pa::launch_decode_balanced(d, p->dtype, p->head_dim, s, take_timing()), "balanced decode kernel");
  if (st != PA_OK) return st;
  return hip_status(pa::launch_merge_balanced(d, p->dtype, p->head_dim, s), "balanced merge kernel");
}

// Rows of chunked-prefill slices on the MFMA kernel: the device work list (on `plan_stream`), then the
// tiles and the merge of partitions (on `s`, which must be ordered after `plan_stream`).
void set_work_list(pa::AttnArgs& a, const MixedLayout& m, char* ws) {
  int32_t* list = reinterpret_cast<int32_t*>(ws + m.list_offset);
  a.tile_count = list;
  a.tiles = list + 4;
  a.tile_capacity = (int32_t)m.tile_capacity;
}

pa_status launch_work_list(const pa::AttnArgs& a, const MixedLayout& m, hipStream_t s) {
  return hip_status(pa::launch_plan(a, const_cast<int32_t*>(a.tiles), const_cast<int32_t*>(a.tile_count),
                                    m.rows_per_tile, s),
                    "plan kernel");
}

pa_status launch_chunk_tiles(pa::AttnArgs a, const pa_params* p, bool beside_decode, hipStream_t s,
                             pa::KernelTiming tm = {}) {
  pa_status st = hip_status(pa::launch_prefill(a, p->head_dim, beside_decode, s, tm), "prefill kernel");
  if (st != PA_OK || a.chunk_partitions <= 1) return st;
  a.mode = pa::kPrefillTokens;  // partials of chunk rows whose keys span several partitions
  a.num_items = a.num_tokens;
  return hip_status(pa::launch_merge(a, p->dtype, p->head_dim, s), "merge kernel");
}

// Shared-prefix decode workspace: [balanced decode][prefix partials (max, sum), (outputs)][whole-segment
// partials, the same][per-request prefix lengths][prefix-pass work list].
// The prefix pass cuts a group's prefix keys into partitions of this many keys (more when a context could
// hold more than kMaxPrefixParts of them): the work-groups of a long prefix then run side by side instead of
// one walking all its keys, and the merge folds a row's prefix partitions in order. On the prefix-shared
// batch described by its beam groups (shared prefixes up to 2480 keys) the step took 170.5 us with 1024-key
// partitions, 172.3 with 512, 178.6 with 256 and 183 without partitions.
constexpr int kPrefixPartitionTokens = 1024;
constexpr int kMaxPrefixParts = 16;

struct SharedLayout {
  Plan plan;
  bool prefix_pass = false;  // false: the batch runs as a plain decode (same results)
  int prefix_parts = 1, prefix_part_tokens = 0;
  int rows_per_tile = 0;
  int64_t tile_capacity = 0;
  size_t prefix_ml = 0, prefix_o = 0, seg_ml = 0, seg_o = 0, item_prefix = 0, list = 0, total = 0;
};

SharedLayout shared_layout(const pa_params* p, int32_t num_seqs, int32_t num_groups) {
  SharedLayout m;
  m.plan = decode_plan(p, num_seqs);
  m.prefix_pass = m.plan.balanced && num_groups > 0 && pa::prefill_supported(p->dtype, p->head_dim, m.plan.group, block_bytes(p));
  if (!m.prefix_pass) {
    m.total = decode_workspace(m.plan);
    return m;
  }
  const size_t rows = (size_t)num_seqs * p->num_q_heads;
  const int64_t max_ctx = (int64_t)p->max_blocks_per_seq * p->block_size;
  int64_t ppt = kPrefixPartitionTokens;
  if ((max_ctx + ppt - 1) / ppt > kMaxPrefixParts)
    ppt = ((max_ctx + kMaxPrefixParts - 1) / kMaxPrefixParts + pa::kTileTokens - 1) / pa::kTileTokens * pa::kTileTokens;
  m.prefix_part_tokens = (int)ppt;
  m.prefix_parts = (int)std::max<int64_t>(1, (max_ctx + ppt - 1) / ppt);
  size_t off = m.plan.bal_bytes;
  m.prefix_ml = off;
  off += align_up(rows * m.prefix_parts * 2 * sizeof(float));
  m.prefix_o = off;
  off += align_up(rows * m.prefix_parts * p->head_dim * sizeof(float));
  m.seg_ml = off;
  off += align_up(rows * 2 * sizeof(float));
  m.seg_o = off;
  off += align_up(rows * p->head_dim * sizeof(float));
  m.item_prefix = off;
  off += align_up((size_t)num_seqs * sizeof(int32_t));
  // tiles = sum over groups of ceil(size / rows_per_tile) <= ceil(S / rows_per_tile) + non-empty groups
  m.rows_per_tile = pa::prefill_rows_per_tile(m.plan.group);
  m.tile_capacity = (num_seqs + m.rows_per_tile - 1) / m.rows_per_tile + std::min(num_groups, num_seqs);
  m.list = off;
  off += align_up(sizeof(int32_t) * 4 + sizeof(int32_t) * 2 * (size_t)m.tile_capacity);
  m.total = off;
  return m;
}

}  // namespace

extern "C" {

size_t pa_decode_workspace_size(const pa_params* params, int32_t num_seqs) {
  if (validate_params(params) != PA_OK || num_seqs < 0) return 0;
  return decode_workspace(decode_plan(params, num_seqs));
}

pa_status pa_decode(const pa_params* params, int32_t num_seqs, void* out, const void* q, const void* k_cache,
                    const void* v_cache, const int32_t* block_tables, const int32_t* context_lens, void* workspace,
                    size_t workspace_bytes, void* stream) {
  pa::error_detail()[0] = '\0';
  pa_status st = validate_params(params);
  if (st != PA_OK) return st;
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_seqs must be >= 0");
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PA_ERR_NULL_POINTER, "a tensor pointer is NULL");
  const Plan pl = decode_plan(params, num_seqs);
  const size_t need = decode_workspace(pl);
  if (need > 0 && workspace == nullptr) return fail(PA_ERR_NULL_POINTER, "workspace is NULL but required");
  if (workspace_bytes < need) return fail(PA_ERR_WORKSPACE_TOO_SMALL, "workspace smaller than pa_decode_workspace_size");
  if (!grid_fits((int64_t)pl.max_partitions * num_seqs * params->num_kv_heads * pl.subgroups) ||
      !grid_fits((int64_t)num_seqs * params->num_q_heads))
    return fail(PA_ERR_UNSUPPORTED, "launch grid too large");

  hipStream_t s = static_cast<hipStream_t>(stream);
  pa::AttnArgs a = base_args(params, pl, num_seqs, num_seqs, out, q, k_cache, v_cache, block_tables, context_lens,
                             nullptr, workspace);
  a.mode = pa::kDecodeSeqs;
  a.num_items = num_seqs;
  if (pl.balanced) {
    set_balanced(a, pl, workspace);
    st = hip_status(pa::launch_decode_balanced(a, params->dtype, params->head_dim, s, take_timing()),
                      "balanced decode kernel");
    if (st != PA_OK) return st;
    return hip_status(pa::launch_merge_balanced(a, params->dtype, params->head_dim, s), "balanced merge kernel");
  }
  st = hip_status(pa::launch_decode(a, params->dtype, params->head_dim, pl.uniform_blocks, s, take_timing()),
                    "decode kernel");
  if (st != PA_OK) return st;
  return hip_status(pa::launch_merge(a, params->dtype, params->head_dim, s), "merge kernel");
}

pa_status pa_decode_noalloc(const pa_params* params, int32_t num_seqs, void* out, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                            void* stream) {
  pa::error_detail()[0] = '\0';
  pa_status st = validate_params(params);
  if (st != PA_OK) return st;
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_seqs must be >= 0");
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PA_ERR_NULL_POINTER, "a tensor pointer is NULL");
  const size_t need = decode_workspace(decode_plan(params, num_seqs));
  if (need > kScratchBytes) {
    std::snprintf(pa::error_detail(), pa::kDetailBytes, "the call needs %zu bytes of scratch, more than the %zu of "
                  "pa_decode_noalloc (use pa_decode with a workspace)", need, kScratchBytes);
    return PA_ERR_WORKSPACE_TOO_SMALL;
  }
  void* ws = nullptr;
  st = scratch_for(static_cast<hipStream_t>(stream), &ws);
  if (st != PA_OK) return st;
  return pa_decode(params, num_seqs, out, q, k_cache, v_cache, block_tables, context_lens, ws, kScratchBytes, stream);
}

size_t pa_decode_shared_workspace_size(const pa_params* params, int32_t num_seqs, int32_t num_groups) {
  if (validate_params(params) != PA_OK || num_seqs < 0 || num_groups < 0) return 0;
  return shared_layout(params, num_seqs, num_groups).total;
}

pa_status pa_decode_shared_ex(const pa_params* params, int32_t num_seqs, int32_t num_groups, void* out, const void* q,
                              const void* k_cache, const void* v_cache, const int32_t* block_tables,
                              const int32_t* context_lens, const int32_t* group_start, const int32_t* group_prefix,
                              void* workspace, size_t workspace_bytes, void* stream, const pa_aux* aux) {
  pa::error_detail()[0] = '\0';
  pa_status st = validate_params(params);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_groups < 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_seqs and num_groups must be >= 0");
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PA_ERR_NULL_POINTER, "a tensor pointer is NULL");
  if (num_groups > 0 && (!group_start || !group_prefix)) return fail(PA_ERR_NULL_POINTER, "a group array is NULL");
  const SharedLayout m = shared_layout(params, num_seqs, num_groups);
  if (!m.prefix_pass)  // no prefix pass for this shape: a plain decode gives the same result
    return pa_decode(params, num_seqs, out, q, k_cache, v_cache, block_tables, context_lens, workspace,
                     workspace_bytes, stream);
  if (workspace == nullptr) return fail(PA_ERR_NULL_POINTER, "workspace is NULL but required");
  if (workspace_bytes < m.total)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "workspace smaller than pa_decode_shared_workspace_size");
  if (!grid_fits(m.tile_capacity * m.prefix_parts * params->num_kv_heads) ||
      !grid_fits((int64_t)num_seqs * params->num_q_heads))
    return fail(PA_ERR_UNSUPPORTED, "launch grid too large");

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  pa::AttnArgs a = base_args(params, m.plan, num_seqs, num_seqs, out, q, k_cache, v_cache, block_tables,
                             context_lens, nullptr, workspace);
  a.mode = pa::kDecodeSeqs;
  a.num_items = num_seqs;
  set_balanced(a, m.plan, workspace);
  a.group_start = group_start;
  a.group_prefix = group_prefix;
  a.num_groups = num_groups;
  a.item_prefix = reinterpret_cast<int32_t*>(ws + m.item_prefix);
  a.prefix_ml = reinterpret_cast<float*>(ws + m.prefix_ml);
  a.prefix_o = reinterpret_cast<float*>(ws + m.prefix_o);
  a.prefix_parts = m.prefix_parts;
  a.prefix_part_tokens = m.prefix_part_tokens;
  a.seg_ml = reinterpret_cast<float*>(ws + m.seg_ml);
  a.seg_o = reinterpret_cast<float*>(ws + m.seg_o);
  int32_t* list = reinterpret_cast<int32_t*>(ws + m.list);
  a.tile_count = list;
  a.tiles = list + 4;
  a.tile_capacity = (int32_t)m.tile_capacity;
  // the prefix pass: group rows against their prefix keys, cut into partitions, partials into prefix_*
  pa::AttnArgs pre = a;
  pre.part_ml = a.prefix_ml;
  pre.part_o = a.prefix_o;
  pre.max_partitions = m.prefix_parts;
  pre.chunk_partitions = m.prefix_parts;
  pre.chunk_partition_tokens = m.prefix_part_tokens;

  // The prefix pass (MFMA, on L2-resident shared blocks) runs on an auxiliary stream beside the decode of
  // the private suffixes; the merge waits for both.
  AuxStream user_aux, *x = nullptr;
  st = resolve_aux(aux, s, user_aux, &x);
  if (st != PA_OK) return st;
  st = hip_status(pa::launch_prefix_plan(a, list + 4, list, m.rows_per_tile, s), "prefix plan kernel");
  if (st != PA_OK) return st;
  hipStream_t ps = x != nullptr ? x->stream : s;
  if (x != nullptr) {
    st = hip_status(hipEventRecord(x->fork, s), "fork event");
    if (st == PA_OK) st = hip_status(hipStreamWaitEvent(x->stream, x->fork, 0), "fork wait");
    if (st != PA_OK) return st;
  }
  st = hip_status(pa::launch_prefix_pass(pre, params->head_dim, ps), "prefix kernel");
  if (st == PA_OK && x != nullptr) st = hip_status(hipEventRecord(x->join, x->stream), "join event");
  if (st != PA_OK) return st;
  st = hip_status(pa::launch_decode_balanced(a, params->dtype, params->head_dim, s, take_timing()),
                  "balanced decode kernel");
  if (st == PA_OK && x != nullptr) st = hip_status(hipStreamWaitEvent(s, x->join, 0), "join wait");
  if (st != PA_OK) return st;
  return hip_status(pa::launch_merge_balanced(a, params->dtype, params->head_dim, s), "balanced merge kernel");
}

pa_status pa_decode_shared(const pa_params* params, int32_t num_seqs, int32_t num_groups, void* out, const void* q,
                           const void* k_cache, const void* v_cache, const int32_t* block_tables,
                           const int32_t* context_lens, const int32_t* group_start, const int32_t* group_prefix,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return pa_decode_shared_ex(params, num_seqs, num_groups, out, q, k_cache, v_cache, block_tables, context_lens,
                             group_start, group_prefix, workspace, workspace_bytes, stream, nullptr);
}

size_t pa_varlen_mixed_workspace_size(const pa_params* params, int32_t num_seqs, int32_t num_tokens,
                                      int32_t max_query_len) {
  if (validate_params(params) != PA_OK || num_seqs < 0 || num_tokens < 0 || max_query_len < 0) return 0;
  return mixed_layout(params, num_seqs, num_tokens, max_query_len).total;
}

pa_status pa_varlen_mixed_ex(const pa_params* params, int32_t num_seqs, int32_t num_tokens, int32_t max_query_len,
                             void* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start_loc,
                             void* workspace, size_t workspace_bytes, void* stream, const pa_aux* aux) {
  pa::error_detail()[0] = '\0';
  pa_status st = validate_params(params);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_tokens < 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_seqs and num_tokens must be >= 0");
  if (num_seqs == 0 || num_tokens == 0) return PA_OK;
  if (max_query_len < 1 || max_query_len > num_tokens)
    return fail(PA_ERR_INVALID_ARGUMENT, "max_query_len must be in [1, num_tokens]");
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start_loc)
    return fail(PA_ERR_NULL_POINTER, "a tensor pointer is NULL");
  const MixedLayout m = mixed_layout(params, num_seqs, num_tokens, max_query_len);
  if (m.total > 0 && workspace == nullptr) return fail(PA_ERR_NULL_POINTER, "workspace is NULL but required");
  if (workspace_bytes < m.total)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "workspace smaller than pa_varlen_mixed_workspace_size");
  const Plan& pl = m.plan;
  if (!grid_fits((int64_t)pl.max_partitions * num_tokens * params->num_kv_heads * pl.subgroups) ||
      !grid_fits((int64_t)m.tile_capacity * pl.max_partitions * params->num_kv_heads) ||
      !grid_fits((int64_t)num_tokens * params->num_q_heads))
    return fail(PA_ERR_UNSUPPORTED, "launch grid too large");

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  pa::AttnArgs a = base_args(params, pl, num_seqs, num_tokens, out, q, k_cache, v_cache, block_tables, context_lens,
                             query_start_loc, ws + m.rows_offset);
  pa::AttnArgs d = a;  // decode rows (q_len == 1)
  d.mode = pa::kMixedDecodeSeqs;
  d.num_items = num_seqs;
  if (pl.balanced) set_balanced(d, pl, ws);

  if (m.use_prefill) set_work_list(a, m, ws);
  if (pl.balanced && m.use_prefill && num_seqs > 1) {
    // Chunk rows (MFMA, compute-bound) and decode rows (HBM-bound) touch disjoint rows of `out` and
    // disjoint workspace regions: the work-list kernel and the chunk tiles go to an auxiliary stream
    // forked from `s` and joined back into it, so they run concurrently with the decode rows (which need
    // no work list and start at once), in work-groups small enough to sit next to the decode waves. (A
    // single request has no decode rows to overlap with: it takes the serial path and the larger
    // work-groups.)
    AuxStream user_aux, *x = nullptr;
    st = resolve_aux(aux, s, user_aux, &x);
    if (st != PA_OK) return st;
    if (x != nullptr) {
      st = hip_status(hipEventRecord(x->fork, s), "fork event");
      if (st == PA_OK) st = hip_status(hipStreamWaitEvent(x->stream, x->fork, 0), "fork wait");
      if (st == PA_OK) st = launch_work_list(a, m, x->stream);
      if (st == PA_OK) st = launch_chunk_tiles(a, params, true, x->stream);
      if (st != PA_OK) return st;
      st = hip_status(hipEventRecord(x->join, x->stream), "join event");
      if (st != PA_OK) return st;
      st = launch_balanced_rows(d, params, s);
      const pa_status sj = hip_status(hipStreamWaitEvent(s, x->join, 0), "join wait");
      return st != PA_OK ? st : sj;
    }
  }
  // serial order on `s`: decode rows, then chunk rows. A batch of one request with several query rows has no
  // decode rows: its chunk kernel is then the call's dominant kernel.
  const bool no_decode_rows = num_seqs == 1 && num_tokens > 1;
  if (pl.balanced && !no_decode_rows) {
    st = launch_balanced_rows(d, params, s);
    if (st != PA_OK || max_query_len <= 1) return st;
  } else if (m.use_prefill && !no_decode_rows) {  // decode rows on the partition kernel, then their merge
    st = hip_status(pa::launch_decode(d, params->dtype, params->head_dim, pl.uniform_blocks, s, take_timing()),
                      "decode kernel");
    if (st != PA_OK) return st;
    st = hip_status(pa::launch_merge(d, params->dtype, params->head_dim, s), "merge kernel");
    if (st != PA_OK) return st;
  }
  if (m.use_prefill) {
    st = launch_work_list(a, m, s);
    return st != PA_OK ? st : launch_chunk_tiles(a, params, false, s, no_decode_rows ? take_timing() : pa::KernelTiming{});
  }
  // no MFMA kernel for this shape: rows of chunks (every row when the balanced kernel is not eligible) on the
  // partition kernel
  a.mode = pl.balanced ? pa::kPrefillTokens : pa::kAllTokens;
  a.num_items = num_tokens;
  // the partition kernel is the dominant kernel unless balanced decode rows ran
  st = hip_status(pa::launch_decode(a, params->dtype, params->head_dim, pl.uniform_blocks, s,
                                    pl.balanced && !no_decode_rows ? pa::KernelTiming{} : take_timing()),
                  "decode kernel");
  if (st != PA_OK) return st;
  return hip_status(pa::launch_merge(a, params->dtype, params->head_dim, s), "merge kernel");
}

pa_status pa_varlen_mixed(const pa_params* params, int32_t num_seqs, int32_t num_tokens, int32_t max_query_len,
                          void* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start_loc,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return pa_varlen_mixed_ex(params, num_seqs, num_tokens, max_query_len, out, q, k_cache, v_cache, block_tables,
                            context_lens, query_start_loc, workspace, workspace_bytes, stream, nullptr);
}

pa_status pa_cache_write(const pa_params* params, int32_t num_seqs, int32_t num_tokens, void* k_cache, void* v_cache,
                         const void* k_new, const void* v_new, const int32_t* block_tables,
                         const int32_t* context_lens, const int32_t* query_start_loc, void* stream) {
  pa::error_detail()[0] = '\0';
  pa_status st = validate_params(params);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_tokens < 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_seqs and num_tokens must be >= 0");
  if (query_start_loc == nullptr && num_tokens != num_seqs)
    return fail(PA_ERR_INVALID_ARGUMENT, "without query_start_loc num_tokens must equal num_seqs");
  if (num_seqs == 0 || num_tokens == 0) return PA_OK;
  if (!k_cache || !v_cache || !k_new || !v_new || !block_tables || !context_lens)
    return fail(PA_ERR_NULL_POINTER, "a tensor pointer is NULL");
  pa::CacheWriteArgs a{};
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_new = k_new;
  a.v_new = v_new;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start_loc = query_start_loc;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.block_size = params->block_size;
  a.num_blocks = params->num_blocks;
  a.max_blocks = params->max_blocks_per_seq;
  const int elem = params->dtype == PA_DTYPE_BF16 ? 2 : 4;
  if ((int64_t)params->num_kv_heads * params->head_dim * elem > INT32_MAX)
    return fail(PA_ERR_UNSUPPORTED, "slot row too large");
  const int row_bytes = params->num_kv_heads * params->head_dim * elem;
  const bool hm = params->layout == PA_LAYOUT_HEAD_MAJOR;
  a.head_bytes_len = params->head_dim * elem;
  a.block_bytes = (int64_t)params->block_size * row_bytes;
  a.slot_bytes = hm ? a.head_bytes_len : row_bytes;
  a.head_bytes = hm ? (int64_t)params->block_size * a.head_bytes_len : a.head_bytes_len;
  return hip_status(pa::launch_cache_write(a, row_bytes, static_cast<hipStream_t>(stream), take_timing()),
                    "cache write kernel");
}

namespace {

// Address under which a kernel reaches caller memory [p, p + bytes): device memory of the current device,
// or pinned host memory (through its device mapping). Pageable host memory, another device's memory, a
// range that runs past its allocation or a misaligned pointer is rejected, so the copy kernel can never
// touch memory it cannot reach.
pa_status kernel_address(const void* p, int64_t bytes, int align, void** dev, const char* what) {
  static thread_local char msg[160];
  if (reinterpret_cast<uintptr_t>(p) % align != 0) {
    std::snprintf(msg, sizeof msg, "%s must be %d-byte aligned", what, align);
    return fail(PA_ERR_INVALID_ARGUMENT, msg);
  }
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess ||
      (at.type != hipMemoryTypeDevice && at.type != hipMemoryTypeHost)) {
    (void)hipGetLastError();
    std::snprintf(msg, sizeof msg, "%s is neither device memory nor pinned host memory", what);
    return fail(PA_ERR_INVALID_ARGUMENT, msg);
  }
  if (at.type == hipMemoryTypeDevice) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || at.device != cur) {
      (void)hipGetLastError();
      std::snprintf(msg, sizeof msg, "%s is memory of another device", what);
      return fail(PA_ERR_INVALID_ARGUMENT, msg);
    }
  }
  void* base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, const_cast<void*>(p)) != hipSuccess ||
      static_cast<const char*>(p) + bytes > static_cast<const char*>(base) + size) {
    (void)hipGetLastError();
    std::snprintf(msg, sizeof msg, "%s does not hold %lld bytes in one allocation", what, (long long)bytes);
    return fail(PA_ERR_INVALID_ARGUMENT, msg);
  }
  *dev = at.type == hipMemoryTypeHost && at.devicePointer != nullptr ? at.devicePointer : const_cast<void*>(p);
  return PA_OK;
}

}  // namespace

pa_status pa_copy_blocks(const pa_params* params, int32_t num_pairs, void* dst_k, void* dst_v, int32_t dst_num_blocks,
                         const void* src_k, const void* src_v, int32_t src_num_blocks, const int32_t* mapping,
                         void* stream) {
  pa::error_detail()[0] = '\0';
  pa_status st = validate_params(params);
  if (st != PA_OK) return st;
  if (num_pairs < 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_pairs must be >= 0");
  if (src_num_blocks < 1 || dst_num_blocks < 1) return fail(PA_ERR_INVALID_ARGUMENT, "a pool holds no block");
  if (num_pairs == 0) return PA_OK;
  if (!dst_k || !dst_v || !src_k || !src_v || !mapping) return fail(PA_ERR_NULL_POINTER, "a pointer is NULL");
  const int64_t elem = params->dtype == PA_DTYPE_BF16 ? 2 : 4;
  const int64_t block_bytes = (int64_t)params->block_size * params->num_kv_heads * params->head_dim * elem;
  const int64_t slices = (block_bytes / 16 + 1023) / 1024;
  if ((int64_t)num_pairs * 2 * slices > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "too many pairs for one launch");
  pa::CopyBlocksArgs a{};
  void* m = nullptr;
  const void* src[2] = {src_k, src_v};
  void* dst[2] = {dst_k, dst_v};
  void* src_dev[2] = {nullptr, nullptr};
  void* dst_dev[2] = {nullptr, nullptr};
  const char* src_name[2] = {"src_k", "src_v"};
  const char* dst_name[2] = {"dst_k", "dst_v"};
  for (int c = 0; c < 2 && st == PA_OK; ++c) {
    st = kernel_address(src[c], block_bytes * src_num_blocks, 16, &src_dev[c], src_name[c]);
    if (st == PA_OK) st = kernel_address(dst[c], block_bytes * dst_num_blocks, 16, &dst_dev[c], dst_name[c]);
  }
  if (st == PA_OK) st = kernel_address(mapping, (int64_t)num_pairs * 8, 8, &m, "mapping");
  if (st != PA_OK) return st;
  a.src_k = src_dev[0];
  a.src_v = src_dev[1];
  a.dst_k = dst_dev[0];
  a.dst_v = dst_dev[1];
  a.mapping = static_cast<const int32_t*>(m);
  a.block_bytes = block_bytes;
  a.num_pairs = num_pairs;
  a.src_num_blocks = src_num_blocks;
  a.dst_num_blocks = dst_num_blocks;
  return hip_status(pa::launch_copy_blocks(a, static_cast<hipStream_t>(stream), take_timing()), "block copy kernel");
}

pa_status pa_probe_stream_read(const void* buf, size_t bytes, int32_t num_waves, uint32_t* sink, void* stream) {
  pa::error_detail()[0] = '\0';
  if (!buf || !sink) return fail(PA_ERR_NULL_POINTER, "buf and sink are required");
  if (bytes == 0 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "buf must be 16-byte aligned and bytes a positive multiple of 16");
  if (num_waves < 1 || num_waves > 65536) return fail(PA_ERR_INVALID_ARGUMENT, "num_waves must be in [1, 65536]");
  return hip_status(pa::launch_stream_read(buf, (int64_t)(bytes / 16), num_waves, sink,
                                           static_cast<hipStream_t>(stream), take_timing()),
                    "stream read kernel");
}

pa_status pa_set_kernel_timing_events(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(PA_ERR_INVALID_ARGUMENT, "timing events must both be set or both be NULL");
  g_timing_start = static_cast<hipEvent_t>(start_event);
  g_timing_stop = static_cast<hipEvent_t>(stop_event);
  return PA_OK;
}

}  // extern "C"
