// Chunked-prefill rows on MFMA (gfx950): attention of the query rows of requests with q_len > 1.
//
// What is computed is the same attention as the decode kernels ("Continuous batching: a paradigm
// shift in inference throughput", section 4.1: keys and values reached block by block through the
// block table, scaled dot products, softmax, weighted sum of V), with the causal horizon of a
// prefill slice: row j of a slice of q_len rows sees keys 0 .. ctx - q_len + j. The slice's own keys
// are already in the paged cache ("PagedAttention memory paging and continuous batching in
// practice", chunked-prefill section: prefill slices batched with the running decodes).
//
// A prefill slice is a dense contraction, so it runs on the matrix cores. One work-group of four
// waves takes 64 (query row, query head) pairs of one kv head (64 / G rows of all G heads of the
// GQA group) against one context partition, in 32-key steps:
//   * the 32 x D tiles of K and V are gathered through the block table into LDS once and used by
//     all 64 pairs;
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (A = K from LDS, B = the wave's 16 query rows kept in
//     registers), so each lane holds one pair and 8 of the 32 keys: the softmax row reductions are
//     two cross-lane swaps;
//   * O^T += V^T P^T on the same instruction: P^T is the lane's own 8 weights (no data movement),
//     split into a bf16 head and a bf16 tail so that the weights keep about 16 significant bits
//     (one bf16 rounding of the weights alone would cost up to 2^-9 of the output); V^T comes from
//     LDS with the transposing read ds_read_b64_tr_b16, which hands each lane 4 keys of one column;
//   * the next step's K/V are loaded into registers while the current step computes.
// Rows whose visible keys span several partitions write (max, sum, un-normalised output) partials
// that the log-sum-exp merge kernel combines; rows inside one partition are written directly.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

using namespace dev;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
#define PA_LDS __attribute__((address_space(3)))

constexpr int kPrefillThreads = 256;  // four waves
constexpr int kMaxTableSlice = kMaxPartitionTokens + 1;

__device__ __forceinline__ f32x4_t mfma_bf16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// Transposing LDS read of 4 bf16: within each 16-lane group g, lane g*16 + r receives, as element k,
// the element r % 4 of the 8-byte chunk addressed by lane g*16 + 4k + r / 4.
__device__ __forceinline__ uint2 lds_read_tr(const uint16_t* p) {
  PA_LDS bf16x4_t* lp = (PA_LDS bf16x4_t*)(const_cast<uint16_t*>(p));
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(lp));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

// Weights w0, w1 as two bf16 terms each: head = bf16(w), tail = bf16(w - head). head + tail carries
// about 16 significant bits, so P V on the matrix cores keeps the fp32 accuracy of the weights.
__device__ __forceinline__ void split_bf16x2(float w0, float w1, uint32_t& head, uint32_t& tail) {
  const __bf16 h0 = (__bf16)w0, h1 = (__bf16)w1;
  head = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
  tail = pack_bf16x2(w0 - (float)h0, w1 - (float)h1);
}

template <int D>
__global__ __launch_bounds__(kPrefillThreads) void prefill_mfma_kernel(AttnArgs a) {
  constexpr int KS = D / 32;                  // 32-wide steps of the q.k contraction
  constexpr int DT = D / 16;                  // 16-wide column tiles of the output
  constexpr int KT = kPrefillTileTokens;      // keys per step
  constexpr int CPR = D / 8;                  // 16-byte chunks per key row
  constexpr int NCH = KT * CPR / kPrefillThreads;  // chunks of K (and of V) each thread moves per step
  constexpr int KROW = D + 8;                 // LDS row strides (elements), padded against bank conflicts
  constexpr int VROW = D + 16;
  static_assert(NCH * kPrefillThreads == KT * CPR, "tile must split evenly over the threads");
  __shared__ __align__(16) uint16_t sk[KT * KROW];
  __shared__ __align__(16) uint16_t sv[KT * VROW];
  __shared__ int32_t s_tab[kMaxTableSlice];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = lane & 15;   // MFMA column: this lane's pair
  const int lg = lane >> 4;  // lane group: keys 4*lg.. of each 16-key half, d 8*lg.. of each 32-wide step

  int id = blockIdx.x;  // kv head fastest: work-groups sharing K/V land on the same XCD
  const int kvh = id % a.num_kv_heads;
  id /= a.num_kv_heads;
  const int part = id % a.max_partitions;
  const int tile = id / a.max_partitions;
  if (tile >= *a.tile_count) return;
  const int s = a.tiles[2 * tile];
  const int row0 = a.tiles[2 * tile + 1];
  const int q0 = a.query_start_loc[s];
  const int q_len = a.query_start_loc[s + 1] - q0;
  const int max_ctx = a.max_blocks * a.block_size;
  const int ctx = min(max(a.context_lens[s], 0), max_ctx);
  const int G = a.group;
  const int rows_here = min(kPrefillPairs / G, q_len - row0);
  const int PT = a.partition_tokens;
  const int kbeg = part * PT;

  // this lane's (query row, query head) pair
  const int pair = wave * 16 + c;
  const int rl = pair / G;
  const int j = row0 + rl;
  const int t = q0 + j;
  const bool live = rl < rows_here && t >= 0 && t < a.num_tokens;
  const int h = kvh * G + (pair - rl * G);
  const int nvis = live ? min(ctx - q_len + j + 1, ctx) : 0;
  const int64_t orow = ((int64_t)t * a.num_q_heads + h) * D;
  uint16_t* out = static_cast<uint16_t*>(a.out);

  if (part == 0 && live && nvis <= 0) {  // no visible key: the row is defined as zeros
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<uint2*>(out + orow + 16 * dt + 4 * lg) = make_uint2(0, 0);
  }
  // keys the last row of the tile sees bound what the work-group reads
  const int last_vis = min(ctx - q_len + row0 + rows_here, ctx);
  const int kend = min(kbeg + PT, last_vis);
  if (rows_here <= 0 || kbeg >= kend) return;
  const int lim = min(nvis, kbeg + PT);  // this pair's keys end here within the partition

  // block-table slice of the partition
  const int BS = a.block_size;
  const int first_blk = kbeg / BS;
  const int n_blk = (kend - 1) / BS - first_blk + 1;
  const int32_t* tab = a.block_tables + (int64_t)s * a.max_blocks;
  for (int i = tid; i < n_blk; i += kPrefillThreads) s_tab[i] = clamp_block(tab[first_blk + i], a.num_blocks);

  // queries: B operand of S^T = K Q^T (lane holds q[pair][32 ks + 8 lg .. + 7])
  uint4 qb[KS];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + orow + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[ks] = live ? *reinterpret_cast<const uint4*>(qp + 32 * ks) : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();  // table slice visible

  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache) + (int64_t)kvh * D;
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache) + (int64_t)kvh * D;
  const int64_t slot_stride = (int64_t)a.num_kv_heads * D;
  uint4 kr[NCH], vr[NCH];
  auto load_step = [&](int k0) {
#pragma unroll
    for (int n = 0; n < NCH; ++n) {
      const int ci = tid + n * kPrefillThreads;
      const int key = ci / CPR, dc = ci - key * CPR;
      const int pos = k0 + key;
      if (pos < kend) {  // keys past the work-group's horizon (stale or foreign data) are never read
        const int blk = s_tab[pos / BS - first_blk];
        const int64_t off = ((int64_t)blk * BS + pos % BS) * slot_stride + dc * 8;
        kr[n] = *reinterpret_cast<const uint4*>(kc + off);
        vr[n] = *reinterpret_cast<const uint4*>(vc + off);
      } else {
        kr[n] = make_uint4(0, 0, 0, 0);
        vr[n] = make_uint4(0, 0, 0, 0);
      }
    }
  };

  f32x4_t acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m = kNegInf, lsum = 0.0f;
  // transposing-read addresses of the V^T operand: rows 4 lg + c / 4 (and + 16), columns 4 (c % 4)
  const int vrow = 4 * lg + (c >> 2);
  const int vcol = 4 * (c & 3);

  load_step(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += KT) {
    __syncthreads();  // every wave is done with the previous step's tiles
#pragma unroll
    for (int n = 0; n < NCH; ++n) {
      const int ci = tid + n * kPrefillThreads;
      const int key = ci / CPR, dc = ci - key * CPR;
      *reinterpret_cast<uint4*>(sk + key * KROW + dc * 8) = kr[n];
      *reinterpret_cast<uint4*>(sv + key * VROW + dc * 8) = vr[n];
    }
    __syncthreads();
    if (k0 + KT < kend) load_step(k0 + KT);  // in flight while this step computes

    // S^T for keys k0 + 16 hf + (0..15): lane holds keys 16 hf + 4 lg + i of pair c
    f32x4_t st[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      st[hf] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 ka = *reinterpret_cast<const uint4*>(sk + (16 * hf + c) * KROW + 32 * ks + 8 * lg);
        st[hf] = mfma_bf16(ka, qb[ks], st[hf]);
      }
    }
    // causal / partition mask and online softmax (log2 units)
    float x[8];
    float tmax = kNegInf;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = k0 + 16 * hf + 4 * lg + i;
        const float v = pos < lim ? st[hf][i] * a.scale_log2 : kNegInf;
        x[4 * hf + i] = v;
        tmax = fmaxf(tmax, v);
      }
    }
    tmax = fmaxf(tmax, partner16(tmax, lane));
    tmax = fmaxf(tmax, partner32(tmax, lane));
    const float mn = fmaxf(m, tmax);
    const float base = mn == kNegInf ? 0.0f : mn;
    const float alpha = __builtin_amdgcn_exp2f(m - base);
    m = mn;
    float psum = 0.0f;
    uint32_t ph[4], pt[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float w0 = __builtin_amdgcn_exp2f(x[2 * i] - base), w1 = __builtin_amdgcn_exp2f(x[2 * i + 1] - base);
      psum += w0 + w1;
      split_bf16x2(w0, w1, ph[i], pt[i]);
    }
    lsum = lsum * alpha + psum;
    const uint4 pb_head = make_uint4(ph[0], ph[1], ph[2], ph[3]);
    const uint4 pb_tail = make_uint4(pt[0], pt[1], pt[2], pt[3]);
    // O^T += V^T P^T: A element e of lane (lg, c) is V[key e < 4 ? 4 lg + e : 12 + 4 lg + e][16 dt + c]
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint2 v0 = lds_read_tr(sv + vrow * VROW + 16 * dt + vcol);
      const uint2 v1 = lds_read_tr(sv + (16 + vrow) * VROW + 16 * dt + vcol);
      const uint4 va = make_uint4(v0.x, v0.y, v1.x, v1.y);
      acc[dt] = mfma_bf16(va, pb_tail, acc[dt] * alpha);
      acc[dt] = mfma_bf16(va, pb_head, acc[dt]);
    }
  }
  // the four lane groups of a pair hold partial sums against the same reference maximum
  lsum += partner16(lsum, lane);
  lsum += partner32(lsum, lane);

  if (!live || lim <= kbeg) return;  // this pair has no key in this partition
  const int n_parts = ceil_div(nvis, PT);
  if (n_parts == 1) {
    const float inv = 1.0f / lsum;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint32_t w0 = pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv);
      const uint32_t w1 = pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv);
      *reinterpret_cast<uint2*>(out + orow + 16 * dt + 4 * lg) = make_uint2(w0, w1);
    }
  } else {
    const int64_t slot = ((int64_t)t * a.num_q_heads + h) * a.max_partitions + part;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4*>(a.part_o + slot * D + 16 * dt + 4 * lg) =
          make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
    if (lg == 0) *reinterpret_cast<float2*>(a.part_ml + slot * 2) = make_float2(m, lsum);
  }
}

// Work list of the prefill kernel: one (request, first row) entry per block of rows_per_tile rows of
// every request with q_len > 1, in request order. One wave; the count is clamped to the capacity.
__global__ __launch_bounds__(64) void prefill_plan_kernel(AttnArgs a, int32_t* tiles, int32_t* count,
                                                         int rows_per_tile) {
  const int lane = threadIdx.x;
  int base = 0;
  for (int c0 = 0; c0 < a.num_seqs; c0 += 64) {
    const int s = c0 + lane;
    int n = 0;
    if (s < a.num_seqs) {
      const int q_len = a.query_start_loc[s + 1] - a.query_start_loc[s];
      if (q_len > 1) n = ceil_div(q_len, rows_per_tile);
    }
    const int incl = wave_inclusive_scan(n, lane);
    for (int i = 0; i < n; ++i) {
      const int idx = base + incl - n + i;
      if (idx < a.tile_capacity) {
        tiles[2 * idx] = s;
        tiles[2 * idx + 1] = i * rows_per_tile;
      }
    }
    base += __builtin_amdgcn_readlane(incl, 63);
  }
  if (lane == 0) *count = min(base, a.tile_capacity);
}

}  // namespace

bool prefill_supported(int dtype, int head_dim, int group) {
  return dtype == 1 && (head_dim == 64 || head_dim == 128) && group >= 1 && group <= kPrefillPairs &&
         kPrefillPairs % group == 0;
}

int prefill_rows_per_tile(int group) { return group > 0 && group <= kPrefillPairs ? kPrefillPairs / group : 1; }

hipError_t launch_plan(const AttnArgs& a, int32_t* tiles, int32_t* tile_count, int rows_per_tile, hipStream_t s) {
  prefill_plan_kernel<<<dim3(1), dim3(64), 0, s>>>(a, tiles, tile_count, rows_per_tile);
  return hipGetLastError();
}

hipError_t launch_prefill(const AttnArgs& a, int head_dim, hipStream_t s) {
  if (a.partition_tokens > kMaxPartitionTokens || a.partition_tokens < kTileTokens) return hipErrorInvalidValue;
  const int64_t grid = (int64_t)a.tile_capacity * a.max_partitions * a.num_kv_heads;
  if (grid <= 0) return hipSuccess;
  if (head_dim == 128) prefill_mfma_kernel<128><<<dim3((unsigned)grid), dim3(kPrefillThreads), 0, s>>>(a);
  else if (head_dim == 64) prefill_mfma_kernel<64><<<dim3((unsigned)grid), dim3(kPrefillThreads), 0, s>>>(a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
