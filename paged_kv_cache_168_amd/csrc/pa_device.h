// Device helpers shared by the decode kernels (gfx950, wave64): cross-lane exchanges, the
// reduce-scatter of partial dot products, bf16 packing and query-row resolution.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {
namespace dev {

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

// 16-byte load of data that one kernel reads exactly once (the K/V rows of a decode step): the
// non-temporal hint lets the caches evict these lines first, which keeps HBM streaming at a higher
// rate than ordinary loads on this part (measured on a paged gather: about 6.0 vs 5.3 TB/s).
__device__ __forceinline__ uint4 load_once(const void* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// K/V row load: streaming (kStream) for private blocks, cached when requests share blocks.
template <bool kStream>
__device__ __forceinline__ uint4 load_kv(const void* p) {
  if constexpr (kStream) return load_once(p);
  else return *static_cast<const uint4*>(p);
}

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
  // kAllTokens, kPrefillTokens
  const int s = find_request(a.query_start_loc, a.num_seqs, item);
  const int q0 = a.query_start_loc[s], q1 = a.query_start_loc[s + 1];
  if (item < q0 || item >= q1) return false;
  if (a.mode == kPrefillTokens && q1 - q0 == 1) return false;
  const int ctx = min(max(a.context_lens[s], 0), max_ctx);
  row.s = s;
  row.t = item;
  row.nvis = min(ctx - (q1 - q0) + (item - q0) + 1, ctx);
  return true;
}


// ---------------------------------------------------------------------------------------------
// One wave's attention state over a stream of 16-token tiles of one (query row, kv head) pair,
// for GW query heads of a GQA group.
//
// Lane layout of a tile (EPL = elements per 16-byte load, LPR = lanes per K/V row):
//   lane = R * LPR + r;  row group R = lane / LPR, r = lane % LPR.
//   Register j of a lane holds elements [r*EPL, r*EPL+EPL) of token j*RPL + R of the tile.
// Partial dot products of the GW heads are reduce-scattered across the LPR lanes of a row group
// (DPP butterflies, high lane bit first), so a lane ends with full scores for token j = r>>2 and
// the heads picked by r&3. Each row group keeps its own online-softmax state (reference maximum
// and weight sum per head, in log2 units); finish() merges the row groups.
// ---------------------------------------------------------------------------------------------
template <typename T, int D, int GW>
struct DecodeState {
  static constexpr int EPL = Geometry<T>::kEPL;
  static constexpr int LPR = D / EPL;            // lanes per K/V row
  static constexpr int L = Log2<LPR>::value;
  static constexpr int RPL = 64 / LPR;           // rows per wave load = row groups
  static constexpr int TPL = kTileTokens / RPL;  // tokens per lane per tile
  static constexpr int N = TPL * GW;             // partial scores per lane
  static constexpr int VPL = GW >= 4 ? GW / 4 : 1;
  static constexpr int DUP = GW >= 4 ? 1 : 4 / GW;  // lanes sharing one reduced value
  static_assert(TPL * 4 == LPR, "the token of a reduced value is r >> 2");

  struct Shared {
    float p[RPL][N];
    float h[RPL][GW];
    float ml[2][GW];
  };

  float m_ref[VPL], l_sum[VPL];
  float acc[GW][EPL];
  int lane, r, R, j_own;
  bool dup_writer;

  __device__ __forceinline__ void init(int lane_id) {
    lane = lane_id;
    r = lane % LPR;
    R = lane / LPR;
    j_own = r >> 2;
    dup_writer = (r & (DUP - 1)) == 0;
  }

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      m_ref[i] = kNegInf;
      l_sum[i] = 0.0f;
    }
#pragma unroll
    for (int g = 0; g < GW; ++g)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] = 0.0f;
  }

  // head of reduced value i of this lane
  __device__ __forceinline__ int head_of(int i) const {
    if constexpr (GW >= 4) return (r & 3) * VPL + i;
    else if constexpr (GW == 2) return (r >> 1) & 1;
    else return 0;
  }

  // Token (row of the tile) held in register j of this lane.
  __device__ __forceinline__ int row_of(int j) const { return j * RPL + R; }

  // One tile: tokens [0, valid) of the tile are visible; the rest are masked (and their V rows,
  // which may hold stale data or NaN, are replaced by zeros).
  __device__ __forceinline__ void tile(const uint4 (&qv)[GW], const uint4 (&kt)[TPL], const uint4 (&vt)[TPL], int valid,
                                       float scale_log2, Shared& sh) {
    float sc[N];
#pragma unroll
    for (int j = 0; j < TPL; ++j)
#pragma unroll
      for (int g = 0; g < GW; ++g) sc[j * GW + g] = dot_partial<T>(qv[g], kt[j]);
    reduce_scatter_step<L - 1, N, N>(sc, lane);

    const bool ok = j_own * RPL + R < valid;
    float x[VPL], mt[VPL];
    bool need = false;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      x[i] = ok ? sc[i] * scale_log2 : kNegInf;
      float m = x[i];
      if constexpr (L == 3) m = fmaxf(m, xor_partner<2>(m, lane));
      else if constexpr (L == 4) m = rowmax_bits23(m);
      else m = allreduce_max<4, 5>(rowmax_bits23(m), lane);
      mt[i] = m;
      need |= m > m_ref[i] + kRescaleSlack;
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const float m_new = fmaxf(m_ref[i], mt[i]);
        const float alpha = (m_new == m_ref[i]) ? 1.0f : __builtin_amdgcn_exp2f(m_ref[i] - m_new);
        l_sum[i] *= alpha;
        m_ref[i] = m_new;
        if (j_own == 0 && dup_writer) sh.h[R][head_of(i)] = alpha;
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int g = 0; g < GW; ++g) {
        const float al = sh.h[R][g];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] *= al;
      }
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const float p = ok ? __builtin_amdgcn_exp2f(x[i] - m_ref[i]) : 0.0f;
      l_sum[i] += p;
      if constexpr (GW >= 4) sh.p[R][r * VPL + i] = p;
      else if (dup_writer) sh.p[R][r / DUP] = p;
    }
    __builtin_amdgcn_wave_barrier();
    float pv[N];
#pragma unroll
    for (int i = 0; i < N; ++i) pv[i] = sh.p[R][i];
    __builtin_amdgcn_wave_barrier();

#pragma unroll
    for (int j = 0; j < TPL; ++j) {
      // rows past the visible end may hold stale data or NaN: select zeros, never multiply them
      const uint4 v = row_of(j) < valid ? vt[j] : make_uint4(0, 0, 0, 0);
      float vf[EPL];
      unpack<T>(v, vf);
#pragma unroll
      for (int g = 0; g < GW; ++g) {
        const float p = pv[j * GW + g];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(p, vf[e], acc[g][e]);
      }
    }
  }

  // Merge the row groups: M = max over groups, w_R = 2^(m_R - M), L = sum_R w_R l_R. Afterwards
  // lanes of row group 0 hold sum_R w_R acc_R in acc, and sh.ml[0][g] = M, sh.ml[1][g] = L.
  __device__ __forceinline__ void finish(Shared& sh) {
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const float lr = allreduce_sum<2, L>(l_sum[i], lane);
      const float mx = allreduce_max<L, 6>(m_ref[i], lane);
      const float w = (m_ref[i] == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(m_ref[i] - mx);
      const float ls = allreduce_sum<L, 6>(lr * w, lane);
      if (j_own == 0 && dup_writer) {
        sh.h[R][head_of(i)] = w;
        if (R == 0) {
          sh.ml[0][head_of(i)] = mx;
          sh.ml[1][head_of(i)] = ls;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      const float wg = sh.h[R][g];
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] = allreduce_sum<L, 6>(acc[g][e] * wg, lane);
    }
  }

  // Row group 0 writes out[h] = acc / L for the GW heads starting at `op` (head stride D).
  __device__ __forceinline__ void store_output(T* op, Shared& sh) const {
    if (R != 0) return;
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      const float inv = 1.0f / sh.ml[1][g];
      float o[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = acc[g][e] * inv;
      *reinterpret_cast<uint4*>(op + g * D + r * EPL) = pack<T>(o);
    }
  }

  // Row group 0 writes the un-normalised partial of head g to po + g * po_head_stride and
  // (M, L) to pml + g * 2.
  __device__ __forceinline__ void store_partial(float* po, int64_t po_head_stride, float* pml, int64_t pml_head_stride,
                                                Shared& sh) const {
    if (R != 0) return;
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      float* dst = po + g * po_head_stride + r * EPL;
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        *reinterpret_cast<float4*>(dst + e) = make_float4(acc[g][e], acc[g][e + 1], acc[g][e + 2], acc[g][e + 3]);
      if (r == 0) *reinterpret_cast<float2*>(pml + g * pml_head_stride) = make_float2(sh.ml[0][g], sh.ml[1][g]);
    }
  }
};

// Integer helpers for wave-wide bookkeeping.
__device__ __forceinline__ int wave_sum_int(int x) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) x += __shfl_xor(x, d);
  return x;
}
__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}
}  // namespace dev
}  // namespace pa
