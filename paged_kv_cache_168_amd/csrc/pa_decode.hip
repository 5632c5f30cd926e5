// Paged-attention decode on gfx950 (CDNA4): context-partitioned single-wave kernel and the
// log-sum-exp merge of partitions.
//
// What is computed follows "Continuous batching: a paradigm shift in inference throughput"
// (guijiagi.com), section 4.1: for a query row, walk the request's logical blocks, translate each
// through the block table to a physical block, score the keys (scaled q.k), softmax over the
// visible keys and accumulate the weighted values, then normalise. The page's running sum is not
// rescaled when the maximum grows; here both the running sum and the accumulator are rescaled
// against one reference maximum, so the result is the exact softmax up to rounding.
//
// Work decomposition (one wave = one work item): (query row, kv head, head sub-group, context
// partition). A wave loads each 16-token tile of K and V once, straight from HBM into VGPRs with
// 16-byte lane loads, and uses it for every query head of its GQA group. The block table slice of
// the partition is held in one VGPR and read with v_readlane, so the address of tile i+1 never waits
// on a table load; tile i+1 is in flight while tile i is computed.
//
// The per-tile arithmetic (reduce-scatter of the partial dot products, online softmax per row
// group, PV accumulation) is DecodeState in pa_device.h.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

using namespace dev;

// ---------------------------------------------------------------------------------------------
// decode partition kernel
// ---------------------------------------------------------------------------------------------
template <typename T, int D, int GW, bool kUniform>
__global__ __launch_bounds__(64) void decode_partition_kernel(AttnArgs a) {
  using State = DecodeState<T, D, GW>;
  constexpr int EPL = State::EPL, TPL = State::TPL;
  __shared__ typename State::Shared sh;
  __shared__ int32_t s_tab[kUniform ? 1 : kMaxPartitionTokens + 1];

  State st;
  st.init(threadIdx.x);
  const int lane = threadIdx.x;

  int id = blockIdx.x;
  const int kv_slots = a.num_kv_heads * a.subgroups;
  const int kv_sub = id % kv_slots;
  id /= kv_slots;
  const int item = id % a.num_items;
  const int part = id / a.num_items;
  const int kvh = kv_sub / a.subgroups;
  const int sub = kv_sub % a.subgroups;

  Row row;
  if (!resolve_row(a, item, row)) return;
  const int h0 = kvh * a.group + sub * GW;
  T* out_row = static_cast<T*>(a.out) + ((int64_t)row.t * a.num_q_heads + h0) * D;
  if (row.nvis <= 0) {  // no visible key: the row is defined as zeros
    if (part == 0 && st.R == 0) {
#pragma unroll
      for (int g = 0; g < GW; ++g) *reinterpret_cast<uint4*>(out_row + g * D + st.r * EPL) = make_uint4(0, 0, 0, 0);
    }
    return;
  }
  const int PT = a.partition_tokens;
  const int start = part * PT;
  if (start >= row.nvis) return;
  const int end = min(start + PT, row.nvis);
  const int n_parts = ceil_div(row.nvis, PT);
  const int BS = a.block_size;
  const int64_t row_stride = a.slot_stride;  // elements between a kv head's rows of consecutive slots

  uint4 qv[GW];
  {
    const T* qp = static_cast<const T*>(a.q) + ((int64_t)row.t * a.num_q_heads + h0) * D + st.r * EPL;
#pragma unroll
    for (int g = 0; g < GW; ++g) qv[g] = *reinterpret_cast<const uint4*>(qp + g * D);
  }

  // block-table slice of the partition (one VGPR lane per block, or LDS for any block size)
  const int32_t* tab = a.block_tables + (int64_t)row.s * a.max_blocks;
  const int first_blk = start / BS;
  const int n_blk = (end - 1) / BS - first_blk + 1;
  int my_blk = 0;
  if constexpr (kUniform) {
    if (lane < n_blk) my_blk = clamp_block(tab[first_blk + lane], a.num_blocks);
  } else {
    for (int i = lane; i < n_blk; i += 64) s_tab[i] = clamp_block(tab[first_blk + i], a.num_blocks);
    __syncthreads();
  }

  const T* kbase = static_cast<const T*>(a.k_cache) + (int64_t)kvh * a.head_stride + st.r * EPL;
  const T* vbase = static_cast<const T*>(a.v_cache) + (int64_t)kvh * a.head_stride + st.r * EPL;

  // Uniform mode: a 16-token tile never straddles a block (block_size % 16 == 0).
  auto load_tile = [&](int tile_start, uint4 (&kt)[TPL], uint4 (&vt)[TPL]) {
    if constexpr (kUniform) {
      const int rel = tile_start - first_blk * BS;
      const int blk = __builtin_amdgcn_readlane(my_blk, rel / BS);
      const int64_t base = (int64_t)blk * a.block_stride + (int64_t)(rel % BS) * row_stride;
#pragma unroll
      for (int j = 0; j < TPL; ++j) {
        const int64_t off = base + (int64_t)st.row_of(j) * row_stride;
        kt[j] = a.cache_kv ? load_kv<false>(kbase + off) : load_kv<true>(kbase + off);
        vt[j] = a.cache_kv ? load_kv<false>(vbase + off) : load_kv<true>(vbase + off);
      }
    } else {
#pragma unroll
      for (int j = 0; j < TPL; ++j) {
        const int pos = tile_start + st.row_of(j);
        if (pos < end) {
          const int blk = s_tab[pos / BS - first_blk];
          const int64_t off = (int64_t)blk * a.block_stride + (int64_t)(pos % BS) * row_stride;
          kt[j] = a.cache_kv ? load_kv<false>(kbase + off) : load_kv<true>(kbase + off);
          vt[j] = a.cache_kv ? load_kv<false>(vbase + off) : load_kv<true>(vbase + off);
        } else {
          kt[j] = make_uint4(0, 0, 0, 0);
          vt[j] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  };

  st.reset();
  // main loop: tile i+1 is loaded while tile i is computed
  uint4 k0[TPL], v0[TPL], k1[TPL], v1[TPL];
  int tile = start;
  load_tile(tile, k0, v0);
  while (true) {
    const int next = tile + kTileTokens;
    if (next < end) load_tile(next, k1, v1);
    st.tile(qv, k0, v0, end - tile, a.scale_log2, sh);
    if (next >= end) break;
    tile = next + kTileTokens;
    if (tile < end) load_tile(tile, k0, v0);
    st.tile(qv, k1, v1, end - next, a.scale_log2, sh);
    if (tile >= end) break;
  }

  st.finish(sh);
  if (n_parts == 1) {
    st.store_output(out_row, sh);
  } else {
    const int64_t slot = ((int64_t)row.t * a.num_q_heads + h0) * a.max_partitions + part;
    st.store_partial(a.part_o + slot * D, (int64_t)a.max_partitions * D, a.part_ml + slot * 2,
                     (int64_t)a.max_partitions * 2, sh);
  }
}

// ---------------------------------------------------------------------------------------------
// log-sum-exp merge of context partitions: one wave per (query row, query head)
// ---------------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void merge_partitions_kernel(AttnArgs a) {
  constexpr int DPL = D / 64;
  const int lane = threadIdx.x;
  const int h = blockIdx.x % a.num_q_heads;
  const int item = blockIdx.x / a.num_q_heads;
  Row row;
  if (!resolve_row(a, item, row)) return;
  const int n_parts = ceil_div(row.nvis, a.partition_tokens);
  if (n_parts <= 1) return;
  const int64_t base = ((int64_t)row.t * a.num_q_heads + h) * a.max_partitions;
  const float* ml = a.part_ml + base * 2;

  float mx = kNegInf;
  for (int p = lane; p < n_parts; p += 64) mx = fmaxf(mx, ml[2 * p]);
  mx = allreduce_max<0, 6>(mx, lane);

  float acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.0f;
  float lsum = 0.0f;
  const float* po = a.part_o + base * D + lane * DPL;
  for (int p = 0; p < n_parts; ++p) {
    const float wgt = __builtin_amdgcn_exp2f(ml[2 * p] - mx);
    lsum = fmaf(wgt, ml[2 * p + 1], lsum);
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = fmaf(wgt, po[(int64_t)p * D + e], acc[e]);
  }
  const float inv = 1.0f / lsum;
  T* op = static_cast<T*>(a.out) + ((int64_t)row.t * a.num_q_heads + h) * D + lane * DPL;
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    if constexpr (sizeof(T) == 2) op[e] = __builtin_bit_cast(uint16_t, (__bf16)(acc[e] * inv));
    else op[e] = acc[e] * inv;
  }
}

template <typename T, int D, int GW>
hipError_t launch_decode_t(const AttnArgs& a, bool uniform, hipStream_t s, KernelTiming tm) {
  const int64_t grid = (int64_t)a.max_partitions * a.num_items * a.num_kv_heads * a.subgroups;
  if (grid <= 0) return hipSuccess;
  if (uniform)
    hipExtLaunchKernelGGL(decode_partition_kernel<T, D, GW, true>, dim3((unsigned)grid), dim3(64), 0, s, tm.start,
                          tm.stop, 0, a);
  else
    hipExtLaunchKernelGGL(decode_partition_kernel<T, D, GW, false>, dim3((unsigned)grid), dim3(64), 0, s, tm.start,
                          tm.stop, 0, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_decode_d(const AttnArgs& a, bool uniform, hipStream_t s, KernelTiming tm) {
  switch (a.heads_per_wave) {
    case 1: return launch_decode_t<T, D, 1>(a, uniform, s, tm);
    case 2: return launch_decode_t<T, D, 2>(a, uniform, s, tm);
    case 4: return launch_decode_t<T, D, 4>(a, uniform, s, tm);
    case 8: return launch_decode_t<T, D, 8>(a, uniform, s, tm);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const AttnArgs& a, int dtype, int head_dim, bool uniform, hipStream_t s, KernelTiming tm) {
  if (dtype == 1) {
    if (head_dim == 128) return launch_decode_d<uint16_t, 128>(a, uniform, s, tm);
    if (head_dim == 64) return launch_decode_d<uint16_t, 64>(a, uniform, s, tm);
  } else {
    if (head_dim == 128) return launch_decode_d<float, 128>(a, uniform, s, tm);
    if (head_dim == 64) return launch_decode_d<float, 64>(a, uniform, s, tm);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const AttnArgs& a, int dtype, int head_dim, hipStream_t s) {
  const int64_t grid = (int64_t)a.num_items * a.num_q_heads;
  if (grid <= 0 || a.max_partitions <= 1) return hipSuccess;
  if (dtype == 1) {
    if (head_dim == 128) merge_partitions_kernel<uint16_t, 128><<<dim3((unsigned)grid), dim3(64), 0, s>>>(a);
    else merge_partitions_kernel<uint16_t, 64><<<dim3((unsigned)grid), dim3(64), 0, s>>>(a);
  } else {
    if (head_dim == 128) merge_partitions_kernel<float, 128><<<dim3((unsigned)grid), dim3(64), 0, s>>>(a);
    else merge_partitions_kernel<float, 64><<<dim3((unsigned)grid), dim3(64), 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace pa
