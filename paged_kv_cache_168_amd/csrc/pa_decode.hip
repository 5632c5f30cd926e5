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
// Lane layout of a tile (EPL = elements per 16-byte load, LPR = lanes per K/V row):
//   lane = R * LPR + r;  row group R = lane / LPR, r = lane % LPR.
//   Register j of a lane holds elements [r*EPL, r*EPL+EPL) of token j*RPL + R of the tile.
// Partial dot products of the G heads are reduce-scattered across the LPR lanes of a row group
// (DPP butterflies, high lane bit first), so after the reduction a lane holds full scores
// for token j = r>>2 and heads picked by r&3. Each row group keeps its own online-softmax state
// (reference max and weight sum per head); the row groups are merged once per partition.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
// A tile only rescales the accumulators when its maximum exceeds the reference by more than this
// (log2 units): weights stay <= 2^8 and rescaling becomes rare after the first tiles.
constexpr float kRescaleSlack = 8.0f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <typename T>
struct Geometry {
  static constexpr int kEPL = 16 / int(sizeof(T));
};

template <int X>
struct Log2 {
  static constexpr int value = 1 + Log2<X / 2>::value;
};
template <>
struct Log2<1> {
  static constexpr int value = 0;
};

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------------------------
// cross-lane exchanges
// ---------------------------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor3 = 0x1B;        // quad_perm [3,2,1,0]
constexpr int kDppXor7 = 0x141;       // row_half_mirror
constexpr int kDppXor8 = 0x128;       // row_ror:8
constexpr int kDppRor4 = 0x124;       // row_ror:4

// Value of the lane whose index differs in bit 4 (resp. bit 5).
__device__ __forceinline__ float partner16(float x, int lane) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((lane & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ float partner32(float x, int lane) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((lane & 32) ? r[0] : r[1]);
}

// Partner for a reduce-scatter step on lane bit B: any lane index that differs in bit B and agrees
// on all higher bits (the lower bits may differ; they are reduced in later steps).
template <int B>
__device__ __forceinline__ float rs_partner(float x, int lane) {
  if constexpr (B == 0) return dpp<kDppXor1>(x);
  else if constexpr (B == 1) return dpp<kDppXor3>(x);
  else if constexpr (B == 2) return dpp<kDppXor7>(x);
  else if constexpr (B == 3) return dpp<kDppXor8>(x);
  else return partner16(x, lane);
}

// Exact-xor partner on lane bit B (keeps every other bit).
template <int B>
__device__ __forceinline__ float xor_partner(float x, int lane) {
  if constexpr (B == 0) return dpp<kDppXor1>(x);
  else if constexpr (B == 1) return dpp<0x4E>(x);  // quad_perm [2,3,0,1]
  else if constexpr (B == 2) return __shfl_xor(x, 4);
  else if constexpr (B == 3) return dpp<kDppXor8>(x);
  else if constexpr (B == 4) return partner16(x, lane);
  else return partner32(x, lane);
}

// Sum over lane bits [LO, HI): every lane of a group gets the same bits.
template <int LO, int HI>
__device__ __forceinline__ float allreduce_sum(float x, int lane) {
  if constexpr (LO < HI) {
    x = x + xor_partner<LO>(x, lane);
    return allreduce_sum<LO + 1, HI>(x, lane);
  } else {
    return x;
  }
}
template <int LO, int HI>
__device__ __forceinline__ float allreduce_max(float x, int lane) {
  if constexpr (LO < HI) {
    x = fmaxf(x, xor_partner<LO>(x, lane));
    return allreduce_max<LO + 1, HI>(x, lane);
  } else {
    return x;
  }
}
// Max over lane bits 2 and 3 of a 16-lane row with two row rotations (exact for max).
__device__ __forceinline__ float rowmax_bits23(float x) {
  x = fmaxf(x, dpp<kDppRor4>(x));
  return fmaxf(x, dpp<kDppXor8>(x));
}

// Reduce-scatter of N partial sums over the lanes of a row group (lane bits [0, L)).
// On return lane r holds in v[0..N/2^L) the full sums of value indexes r*N/2^L + i when
// N >= 2^L; otherwise v[0] holds value index r >> (L - log2 N) (replicated over the low bits).
template <int B, int N, int n>
__device__ __forceinline__ void reduce_scatter_step(float (&v)[N], int lane) {
  if constexpr (B >= 0) {
    if constexpr (n > 1) {
      const bool hi = (lane >> B) & 1;
#pragma unroll
      for (int i = 0; i < n / 2; ++i) {
        const float send = hi ? v[i] : v[i + n / 2];
        const float keep = hi ? v[i + n / 2] : v[i];
        v[i] = keep + rs_partner<B>(send, lane);
      }
      reduce_scatter_step<B - 1, N, n / 2>(v, lane);
    } else {
      v[0] = v[0] + xor_partner<B>(v[0], lane);
      reduce_scatter_step<B - 1, N, 1>(v, lane);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// element helpers
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <typename T>
__device__ __forceinline__ float dot_partial(const uint4& q, const uint4& k);
template <>
__device__ __forceinline__ float dot_partial<uint16_t>(const uint4& q, const uint4& k) {
  float d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.x), __builtin_bit_cast(bf16x2_t, k.x),
                                            0.0f, false);
  d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.y), __builtin_bit_cast(bf16x2_t, k.y), d, false);
  d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.z), __builtin_bit_cast(bf16x2_t, k.z), d, false);
  d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.w), __builtin_bit_cast(bf16x2_t, k.w), d, false);
  return d;
}
template <>
__device__ __forceinline__ float dot_partial<float>(const uint4& q, const uint4& k) {
  float d = __uint_as_float(q.x) * __uint_as_float(k.x);
  d = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), d);
  d = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), d);
  d = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), d);
  return d;
}

template <typename T>
__device__ __forceinline__ void unpack(const uint4& w, float (&f)[Geometry<T>::kEPL]);
template <>
__device__ __forceinline__ void unpack<uint16_t>(const uint4& w, float (&f)[8]) {
  f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
  f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
  f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z);
  f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}
template <>
__device__ __forceinline__ void unpack<float>(const uint4& w, float (&f)[4]) {
  f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
  f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
}

template <typename T>
__device__ __forceinline__ uint4 pack(const float (&f)[Geometry<T>::kEPL]);
template <>
__device__ __forceinline__ uint4 pack<uint16_t>(const float (&f)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)f[2 * i]);
    const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)f[2 * i + 1]);
    w[i] = lo | (hi << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}
template <>
__device__ __forceinline__ uint4 pack<float>(const float (&f)[4]) {
  return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
}

__device__ __forceinline__ int clamp_block(int b, int nb) { return (b >= 0 && b < nb) ? b : 0; }

// ---------------------------------------------------------------------------------------------
// row resolution
// ---------------------------------------------------------------------------------------------
struct Row {
  int t, s, nvis;
};

// Request that owns query row t: largest s with query_start_loc[s] <= t (binary search).
__device__ __forceinline__ int find_request(const int32_t* qsl, int num_seqs, int t) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (qsl[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Returns false when the item has no row for this kernel.
__device__ __forceinline__ bool resolve_row(const AttnArgs& a, int item, Row& row) {
  const int max_ctx = a.max_blocks * a.block_size;
  if (a.mode == kDecodeSeqs) {
    row.s = item;
    row.t = item;
    row.nvis = min(max(a.context_lens[item], 0), max_ctx);
    return true;
  }
  if (a.mode == kMixedDecodeSeqs) {
    const int q0 = a.query_start_loc[item], q1 = a.query_start_loc[item + 1];
    if (q1 - q0 != 1 || q0 < 0 || q0 >= a.num_tokens) return false;
    row.s = item;
    row.t = q0;
    row.nvis = min(max(a.context_lens[item], 0), max_ctx);
    return true;
  }
  // kAllTokens
  const int s = find_request(a.query_start_loc, a.num_seqs, item);
  const int q0 = a.query_start_loc[s], q1 = a.query_start_loc[s + 1];
  if (item < q0 || item >= q1) return false;
  const int ctx = min(max(a.context_lens[s], 0), max_ctx);
  row.s = s;
  row.t = item;
  row.nvis = min(ctx - (q1 - q0) + (item - q0) + 1, ctx);
  return true;
}

// ---------------------------------------------------------------------------------------------
// decode partition kernel
// ---------------------------------------------------------------------------------------------
template <typename T, int D, int GW, bool kUniform>
__global__ __launch_bounds__(64) void decode_partition_kernel(AttnArgs a) {
  constexpr int EPL = Geometry<T>::kEPL;
  constexpr int LPR = D / EPL;           // lanes per K/V row
  constexpr int L = Log2<LPR>::value;
  constexpr int RPL = 64 / LPR;          // rows per wave load = row groups
  constexpr int TPL = kTileTokens / RPL; // tokens per lane per tile
  constexpr int N = TPL * GW;            // partial scores per lane
  constexpr int VPL = GW >= 4 ? GW / 4 : 1;
  constexpr int DUP = GW >= 4 ? 1 : 4 / GW;  // lanes that share one reduced value
  static_assert(TPL * 4 == LPR, "token index of a reduced value is r >> 2");

  __shared__ float s_p[RPL][N];
  __shared__ float s_h[RPL][GW];
  __shared__ float s_ml[2][GW];
  __shared__ int32_t s_tab[kUniform ? 1 : kMaxPartitionTokens + 1];

  const int lane = threadIdx.x;
  const int r = lane % LPR;
  const int R = lane / LPR;
  const int j_own = r >> 2;

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
  if (row.nvis <= 0) {  // no visible key: the row is defined as zeros
    if (part == 0 && R == 0) {
      T* op = static_cast<T*>(a.out) + ((int64_t)row.t * a.num_q_heads + h0) * D + r * EPL;
#pragma unroll
      for (int g = 0; g < GW; ++g) *reinterpret_cast<uint4*>(op + g * D) = make_uint4(0, 0, 0, 0);
    }
    return;
  }
  const int PT = a.partition_tokens;
  const int start = part * PT;
  if (start >= row.nvis) return;
  const int end = min(start + PT, row.nvis);
  const int n_parts = ceil_div(row.nvis, PT);
  const int BS = a.block_size;
  const int64_t row_stride = (int64_t)a.num_kv_heads * D;  // elements between slots

  // query vectors of the GW heads, this lane's slice of the head dimension
  uint4 qv[GW];
  {
    const T* qp = static_cast<const T*>(a.q) + ((int64_t)row.t * a.num_q_heads + h0) * D + r * EPL;
#pragma unroll
    for (int g = 0; g < GW; ++g) qv[g] = *reinterpret_cast<const uint4*>(qp + g * D);
  }

  // block-table slice of the partition
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

  const T* kbase = static_cast<const T*>(a.k_cache) + (int64_t)kvh * D + r * EPL;
  const T* vbase = static_cast<const T*>(a.v_cache) + (int64_t)kvh * D + r * EPL;

  // Tile loads. Uniform mode: a 16-token tile never straddles a block (block_size % 16 == 0).
  auto load_tile = [&](int tile_start, uint4 (&kt)[TPL], uint4 (&vt)[TPL]) {
    if constexpr (kUniform) {
      const int rel = tile_start - first_blk * BS;
      const int blk = __builtin_amdgcn_readlane(my_blk, rel / BS);
      const int64_t base = ((int64_t)blk * BS + rel % BS) * row_stride;
#pragma unroll
      for (int j = 0; j < TPL; ++j) {
        const int64_t off = base + (int64_t)(j * RPL + R) * row_stride;
        kt[j] = *reinterpret_cast<const uint4*>(kbase + off);
        vt[j] = *reinterpret_cast<const uint4*>(vbase + off);
      }
    } else {
#pragma unroll
      for (int j = 0; j < TPL; ++j) {
        const int pos = tile_start + j * RPL + R;
        if (pos < end) {
          const int blk = s_tab[pos / BS - first_blk];
          const int64_t off = ((int64_t)blk * BS + pos % BS) * row_stride;
          kt[j] = *reinterpret_cast<const uint4*>(kbase + off);
          vt[j] = *reinterpret_cast<const uint4*>(vbase + off);
        } else {
          kt[j] = make_uint4(0, 0, 0, 0);
          vt[j] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  };

  // online-softmax state of this lane's row group
  float m_ref[VPL], l_sum[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    m_ref[i] = kNegInf;
    l_sum[i] = 0.0f;
  }
  float acc[GW][EPL];
#pragma unroll
  for (int g = 0; g < GW; ++g)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.0f;

  // head of reduced value i of this lane, and whether this lane is the writer of its value
  auto head_of = [&](int i) -> int {
    if constexpr (GW >= 4) return (r & 3) * VPL + i;
    else if constexpr (GW == 2) return (r >> 1) & 1;
    else return 0;
  };
  const bool dup_writer = (r & (DUP - 1)) == 0;

  auto compute_tile = [&](int tile_start, uint4 (&kt)[TPL], uint4 (&vt)[TPL]) {
    float sc[N];
#pragma unroll
    for (int j = 0; j < TPL; ++j)
#pragma unroll
      for (int g = 0; g < GW; ++g) sc[j * GW + g] = dot_partial<T>(qv[g], kt[j]);
    reduce_scatter_step<L - 1, N, N>(sc, lane);

    const bool valid = tile_start + j_own * RPL + R < end;
    float x[VPL], mt[VPL];
    bool need = false;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      x[i] = valid ? sc[i] * a.scale_log2 : kNegInf;
      float m = x[i];
      if constexpr (L == 3) m = fmaxf(m, xor_partner<2>(m, lane));
      else if constexpr (L == 4) m = rowmax_bits23(m);
      else m = allreduce_max<4, 5>(rowmax_bits23(m), lane);
      mt[i] = m;
      need |= m > m_ref[i] + kRescaleSlack;
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      float alpha[VPL];
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const float m_new = fmaxf(m_ref[i], mt[i]);
        alpha[i] = (m_new == m_ref[i]) ? 1.0f : __builtin_amdgcn_exp2f(m_ref[i] - m_new);
        l_sum[i] *= alpha[i];
        m_ref[i] = m_new;
        if (j_own == 0 && dup_writer) s_h[R][head_of(i)] = alpha[i];
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int g = 0; g < GW; ++g) {
        const float al = s_h[R][g];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] *= al;
      }
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const float p = valid ? __builtin_amdgcn_exp2f(x[i] - m_ref[i]) : 0.0f;
      l_sum[i] += p;
      if constexpr (GW >= 4) s_p[R][r * VPL + i] = p;
      else if (dup_writer) s_p[R][r / DUP] = p;
    }
    __builtin_amdgcn_wave_barrier();
    float pv[N];
#pragma unroll
    for (int i = 0; i < N; ++i) pv[i] = s_p[R][i];
    __builtin_amdgcn_wave_barrier();

    if (tile_start + kTileTokens > end) {  // tail: rows past the end may hold stale data or NaN
#pragma unroll
      for (int j = 0; j < TPL; ++j)
        if (tile_start + j * RPL + R >= end) vt[j] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < TPL; ++j) {
      float vf[EPL];
      unpack<T>(vt[j], vf);
#pragma unroll
      for (int g = 0; g < GW; ++g) {
        const float p = pv[j * GW + g];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(p, vf[e], acc[g][e]);
      }
    }
  };

  // main loop: tile i+1 is loaded while tile i is computed
  uint4 k0[TPL], v0[TPL], k1[TPL], v1[TPL];
  int tile = start;
  load_tile(tile, k0, v0);
  while (true) {
    const int next = tile + kTileTokens;
    if (next < end) load_tile(next, k1, v1);
    compute_tile(tile, k0, v0);
    if (next >= end) break;
    tile = next + kTileTokens;
    if (tile < end) load_tile(tile, k0, v0);
    compute_tile(next, k1, v1);
    if (tile >= end) break;
  }

  // merge the row groups: M = max over groups, w_R = 2^(m_R - M), L = sum_R w_R l_R
  float w[VPL], Mx[VPL], Ls[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const float lr = allreduce_sum<2, L>(l_sum[i], lane);
    Mx[i] = allreduce_max<L, 6>(m_ref[i], lane);
    w[i] = (m_ref[i] == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(m_ref[i] - Mx[i]);
    Ls[i] = allreduce_sum<L, 6>(lr * w[i], lane);
    if (j_own == 0 && dup_writer) {
      s_h[R][head_of(i)] = w[i];
      if (R == 0) {
        s_ml[0][head_of(i)] = Mx[i];
        s_ml[1][head_of(i)] = Ls[i];
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int g = 0; g < GW; ++g) {
    const float wg = s_h[R][g];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = allreduce_sum<L, 6>(acc[g][e] * wg, lane);
  }

  if (R != 0) return;
  if (n_parts == 1) {
    T* op = static_cast<T*>(a.out) + ((int64_t)row.t * a.num_q_heads + h0) * D + r * EPL;
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      const float inv = 1.0f / s_ml[1][g];
      float o[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = acc[g][e] * inv;
      *reinterpret_cast<uint4*>(op + g * D) = pack<T>(o);
    }
  } else {
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      const int64_t slot = ((int64_t)row.t * a.num_q_heads + h0 + g) * a.max_partitions + part;
      float* po = a.part_o + slot * D + r * EPL;
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        *reinterpret_cast<float4*>(po + e) = make_float4(acc[g][e], acc[g][e + 1], acc[g][e + 2], acc[g][e + 3]);
      if (r == 0) *reinterpret_cast<float2*>(a.part_ml + slot * 2) = make_float2(s_ml[0][g], s_ml[1][g]);
    }
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
hipError_t launch_decode_t(const AttnArgs& a, bool uniform, hipStream_t s) {
  const int64_t grid = (int64_t)a.max_partitions * a.num_items * a.num_kv_heads * a.subgroups;
  if (grid <= 0) return hipSuccess;
  if (uniform)
    decode_partition_kernel<T, D, GW, true><<<dim3((unsigned)grid), dim3(64), 0, s>>>(a);
  else
    decode_partition_kernel<T, D, GW, false><<<dim3((unsigned)grid), dim3(64), 0, s>>>(a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_decode_d(const AttnArgs& a, bool uniform, hipStream_t s) {
  switch (a.heads_per_wave) {
    case 1: return launch_decode_t<T, D, 1>(a, uniform, s);
    case 2: return launch_decode_t<T, D, 2>(a, uniform, s);
    case 4: return launch_decode_t<T, D, 4>(a, uniform, s);
    case 8: return launch_decode_t<T, D, 8>(a, uniform, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const AttnArgs& a, int dtype, int head_dim, bool uniform, hipStream_t s) {
  if (dtype == 1) {
    if (head_dim == 128) return launch_decode_d<uint16_t, 128>(a, uniform, s);
    if (head_dim == 64) return launch_decode_d<uint16_t, 64>(a, uniform, s);
  } else {
    if (head_dim == 128) return launch_decode_d<float, 128>(a, uniform, s);
    if (head_dim == 64) return launch_decode_d<float, 64>(a, uniform, s);
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
