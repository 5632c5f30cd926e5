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

// ---------------------------------------------------------------------------------------------
// matrix cores and LDS (bf16)
// ---------------------------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
#define PA_LDS __attribute__((address_space(3)))

// D += A B on a 16 x 16 tile, k = 32: lane l supplies A[l % 16][8 (l / 16) .. + 7] and
// B[8 (l / 16) .. + 7][l % 16] and holds D[4 (l / 16) + i][l % 16].
__device__ __forceinline__ f32x4_t mfma_16x16x32(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
// The same with k = 16: lane l supplies A[l % 16][4 (l / 16) .. + 3] and B[4 (l / 16) .. + 3][l % 16].
__device__ __forceinline__ f32x4_t mfma_16x16x16(const uint2& a, const uint2& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a), __builtin_bit_cast(i16x4_t, b), c,
                                                   0, 0, 0);
}

// Transposing LDS read of 4 bf16: within each 16-lane group g, lane g*16 + r receives, as element k,
// the element r % 4 of the 8-byte chunk addressed by lane g*16 + 4k + r / 4.
__device__ __forceinline__ uint2 lds_read_tr(const uint16_t* p) {
  PA_LDS bf16x4_t* lp = (PA_LDS bf16x4_t*)(const_cast<uint16_t*>(p));
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(lp));
}

// 16 bytes per lane from global memory into LDS at lds_base + 16 * lane (lds_base wave-uniform),
// with the non-temporal hint when kStream (data read once).
template <bool kStream>
__device__ __forceinline__ void load_to_lds(const void* g, uint16_t* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (PA_LDS void*)lds_base, 16, 0, kStream ? 2 : 0);
}

// Two floats to packed bf16 (round to nearest even), lo in the low half: one v_cvt_pk_bf16_f32, where two
// scalar casts would cost two conversions, a shift and an or.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Weights w0, w1 as two bf16 terms each: head = bf16(w), tail = bf16(w - head).
__device__ __forceinline__ void split_bf16x2(float w0, float w1, uint32_t& head, uint32_t& tail) {
  head = pack_bf16x2(w0, w1);
  tail = pack_bf16x2(w0 - __uint_as_float(head << 16), w1 - __uint_as_float(head & 0xFFFF0000u));
}

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
    float h2[RPL][GW];
    float ml[2][GW];
  };

  float m_ref[VPL], l_sum[VPL];
  float acc[GW][EPL];
  // context partitions of the current piece that have ended, folded together (caller-set partitions)
  float m_p[VPL], l_p[VPL];
  float acc_p[GW][EPL];
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

  __device__ __forceinline__ void reset_parts() {
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      m_p[i] = kNegInf;
      l_p[i] = 0.0f;
    }
#pragma unroll
    for (int g = 0; g < GW; ++g)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc_p[g][e] = 0.0f;
  }

  // Log-sum-exp fold of the current state with the kept one, per row group and head: into the kept state at a
  // partition's end (the current one then restarts), or into the current state at the piece's end.
  template <bool kIntoCurrent>
  __device__ __forceinline__ void fold_parts(Shared& sh) {
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const float mn = fmaxf(m_p[i], m_ref[i]);
      const float wp = m_p[i] == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(m_p[i] - mn);
      const float wc = m_ref[i] == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(m_ref[i] - mn);
      const float l = l_p[i] * wp + l_sum[i] * wc;
      if constexpr (kIntoCurrent) {
        m_ref[i] = mn;
        l_sum[i] = l;
      } else {
        m_p[i] = mn;
        l_p[i] = l;
      }
      if (j_own == 0 && dup_writer) {
        sh.h[R][head_of(i)] = wp;
        sh.h2[R][head_of(i)] = wc;
      }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      const float wp = sh.h[R][g], wc = sh.h2[R][g];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float v = acc_p[g][e] * wp + acc[g][e] * wc;
        if constexpr (kIntoCurrent) acc[g][e] = v;
        else acc_p[g][e] = v;
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // head of reduced value i of this lane
  __device__ __forceinline__ int head_of(int i) const {
    if constexpr (GW >= 4) return (r & 3) * VPL + i;
    else if constexpr (GW == 2) return (r >> 1) & 1;
    else return 0;
  }

  // Token (row of the tile) held in register j of this lane.
  __device__ __forceinline__ int row_of(int j) const { return j * RPL + R; }

  // Interface of the balanced decode kernel: the K and V rows of a tile in flight (registers), the
  // query registers, and the loads of both.
  static constexpr int kQRegs = GW;
  struct Tile {
    uint4 k[TPL], v[TPL];
  };
  // Loads of the tile whose first token row starts at element `base` of the caches (kv head included).
  template <bool kStream>
  __device__ __forceinline__ void issue(const T* kc, const T* vc, int64_t base, int64_t slot_stride, Tile& t, int,
                                        Shared&) const {
#pragma unroll
    for (int j = 0; j < TPL; ++j) {
      const int64_t off = base + (int64_t)row_of(j) * slot_stride + r * EPL;
      t.k[j] = load_kv<kStream>(kc + off);
      t.v[j] = load_kv<kStream>(vc + off);
    }
  }
  // Query registers of the GW heads whose first element is qp.
  __device__ __forceinline__ void load_q(const T* qp, float, uint4 (&qv)[kQRegs]) const {
#pragma unroll
    for (int g = 0; g < GW; ++g) qv[g] = *reinterpret_cast<const uint4*>(qp + g * D + r * EPL);
  }
  __device__ __forceinline__ void tile(const uint4 (&qv)[GW], const Tile& t, int, int valid, float scale_log2,
                                       Shared& sh) {
    tile(qv, t.k, t.v, valid, scale_log2, sh);
  }
  __device__ __forceinline__ void drain() const {}

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

// Decode of one query row on the matrix cores (bf16), for a GQA group of GW (4 or 8) query heads per
// wave: the GW heads are the 16 columns of the MFMA tiles (columns GW..15 hold zero queries and are
// never stored), the 16 tokens of a tile its rows.
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: lane (lg = lane / 16, c = lane % 16) supplies K row c
//     of the tile, 16-byte chunks lg, lg + 4, ... (the query chunks use the same order), and receives
//     the scores of keys 4 lg .. 4 lg + 3 for head c. The row maximum and sum take two cross-lane swaps.
//     KLDS: the K tile goes through LDS like V (every load instruction then reads 1 KB of whole rows);
//     otherwise each lane loads its chunks straight from HBM into registers.
//   * The online softmax rescales only when a head's maximum rises by more than kRescaleSlack.
//   * O^T += V^T P^T on v_mfma_f32_16x16x16bf16_1k: P^T is the lane's own weights (no data movement),
//     split into a bf16 head and a bf16 tail; V^T comes from LDS with the transposing read
//     ds_read_b64_tr_b16. The V tile goes from HBM straight into LDS (global_load_lds_dwordx4, the 16-byte
//     chunks of row r stored at position chunk ^ r so that the transposing reads hit distinct banks),
//     one ring slot per tile in flight.
// Keys past the visible end of a tile (stale or NaN data) get score -inf, weight 0 and zero V.
template <int D, int GW, int DEPTH, bool KLDS = false>
struct MfmaDecodeState {
  static constexpr int KS = D / 32;    // 32-wide steps of q.k = K registers per lane per tile
  static constexpr int DB = D / 16;    // 16-wide blocks of output dims
  static constexpr int CPR = D / 8;    // 16-byte chunks per row
  static constexpr int VL = 16 * CPR / 64;  // LDS-load instructions per V tile
  static constexpr int kQRegs = KS;
  static constexpr int kTileLoads = (KLDS ? VL : KS) + VL;  // vector-memory instructions per tile and lane
  static_assert(GW == 4 || GW == 8, "four or eight heads per wave");
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");

  struct Shared {
    uint16_t v[DEPTH][16 * D];
    uint16_t k[KLDS ? DEPTH : 1][16 * D];
  };
  struct Tile {
    uint4 k[KLDS ? 1 : KS];
  };

  f32x4_t acc[DB];
  float m_ref, l_sum, l_tot;
  // context partitions of the current piece that have ended, folded together (caller-set partitions)
  f32x4_t acc_p[DB];
  float m_p, l_p;
  int lane, lg, c;
  int v_off[DB];  // element offset of this lane's transposing-read chunk in a V tile

  __device__ __forceinline__ void init(int lane_id) {
    lane = lane_id;
    lg = lane >> 4;
    c = lane & 15;
    // lane (lg, c) addresses row 4 lg + c / 4, dims 16 db + 4 (c % 4) .. + 3: 16-byte chunk 2 db + (c % 4) / 2
    // (stored at position chunk ^ row), 8-byte half c % 2
    const int vr = 4 * lg + (c >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) v_off[db] = vr * D + (((2 * db + ((c & 3) >> 1)) ^ (vr % CPR)) * 8) + 4 * (c & 1);
  }

  __device__ __forceinline__ void reset() {
    m_ref = kNegInf;
    l_sum = 0.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  __device__ __forceinline__ void reset_parts() {
    m_p = kNegInf;
    l_p = 0.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc_p[db] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // Log-sum-exp fold of the current state with the kept one (a lane's maximum is its head's): into the kept
  // state at a partition's end (the current one then restarts), or into the current state at the piece's end.
  template <bool kIntoCurrent>
  __device__ __forceinline__ void fold_parts(Shared&) {
    const float mn = fmaxf(m_p, m_ref);
    const float wp = m_p == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(m_p - mn);
    const float wc = m_ref == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(m_ref - mn);
    const float l = l_p * wp + l_sum * wc;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const f32x4_t v = acc_p[db] * wp + acc[db] * wc;
      if constexpr (kIntoCurrent) acc[db] = v;
      else acc_p[db] = v;
    }
    if constexpr (kIntoCurrent) {
      m_ref = mn;
      l_sum = l;
    } else {
      m_p = mn;
      l_p = l;
    }
  }

  template <bool kStream>
  __device__ __forceinline__ void issue(const uint16_t* kc, const uint16_t* vc, int64_t base, int64_t slot_stride,
                                        Tile& t, int d, Shared& sh) const {
    // the slot's previous V fragments were read before its new tile may land
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if constexpr (KLDS) {
#pragma unroll
      for (int i = 0; i < VL; ++i) {
        const int p = i * 64 + lane;
        const int row = p / CPR;
        const int chunk = (p % CPR) ^ (row % CPR);
        load_to_lds<kStream>(kc + base + (int64_t)row * slot_stride + chunk * 8, sh.k[d] + i * 64 * 8);
      }
    } else {
      const uint16_t* kp = kc + base + (int64_t)c * slot_stride + lg * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) t.k[ks] = load_kv<kStream>(kp + ks * 32);
    }
    // V: instruction i fills LDS positions p = 64 i + lane: row p / CPR, position p % CPR, which holds the
    // row's chunk (p % CPR) ^ row
#pragma unroll
    for (int i = 0; i < VL; ++i) {
      const int p = i * 64 + lane;
      const int row = p / CPR;
      const int chunk = (p % CPR) ^ (row % CPR);
      load_to_lds<kStream>(vc + base + (int64_t)row * slot_stride + chunk * 8, sh.v[d] + i * 64 * 8);
    }
  }

  // Query registers: lane (lg, c) holds chunks lg + 4 ks of head c (zero for c >= GW). A negative scale
  // is applied as |scale| to sign-flipped queries, so the row maximum of the dot products is the one
  // of the scaled scores.
  __device__ __forceinline__ void load_q(const uint16_t* qp, float scale_log2, uint4 (&qv)[kQRegs]) const {
    const uint32_t flip = scale_log2 < 0.0f ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qv[ks] = make_uint4(0, 0, 0, 0);
    if (c < GW) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 v = *reinterpret_cast<const uint4*>(qp + c * D + (lg + 4 * ks) * 8);
        qv[ks] = make_uint4(v.x ^ flip, v.y ^ flip, v.z ^ flip, v.w ^ flip);
      }
    }
  }

  __device__ __forceinline__ void tile(const uint4 (&qv)[kQRegs], const Tile& t, int d, int valid, float scale_log2,
                                       Shared& sh) {
    const float c2 = fabsf(scale_log2);
    f32x4_t s = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (KLDS) {
      // the tile's loads into LDS have landed once at most the later tiles' loads are pending. (The compiler
      // tracks loads into LDS and adds a vmcnt(0) of its own before these reads, so in effect every tile waits
      // for all loads in flight; a build whose LDS loads it could not track, so that only this wait applied and
      // the later tiles stayed in flight, measured slower on the 8 x 32768 batch: 177.7 against 166.9 us.)
      static_assert((DEPTH - 1) * kTileLoads <= 63, "vmcnt range");
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((DEPTH - 1) * kTileLoads) : "memory");
      uint4 ka[KS];  // K row c, chunks lg + 4 ks (stored at position chunk ^ c)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        ka[ks] = *reinterpret_cast<const uint4*>(sh.k[d] + c * D + (((lg + 4 * ks) ^ (c % CPR)) * 8));
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s = mfma_16x16x32(ka[ks], qv[ks], s);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s = mfma_16x16x32(t.k[ks], qv[ks], s);
    }
    const bool partial = valid < kTileTokens;
    if (partial) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = (4 * lg + i < valid) ? s[i] : kNegInf;
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, partner16(mx, lane));
    mx = fmaxf(mx, partner32(mx, lane));
    const float tmax = mx == kNegInf ? kNegInf : mx * c2;  // log2 units
    if (__builtin_amdgcn_ballot_w64(tmax > m_ref + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m_ref, tmax);
      const float alpha = (m_new == m_ref) ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_sum *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    }
    const float nb = m_ref == kNegInf ? 0.0f : -m_ref;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c2, nb));
      if (partial) p[i] = (4 * lg + i < valid) ? p[i] : 0.0f;
    }
    l_sum += (p[0] + p[1]) + (p[2] + p[3]);
    uint2 w, u;
    split_bf16x2(p[0], p[1], w.x, u.x);
    split_bf16x2(p[2], p[3], w.y, u.y);

    // V^T fragments: the tile's loads into LDS have landed once at most the later tiles' loads are pending
    if constexpr (!KLDS) {
      static_assert((DEPTH - 1) * kTileLoads <= 63, "vmcnt range");
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((DEPTH - 1) * kTileLoads) : "memory");
    }
    uint2 va[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) va[db] = lds_read_tr(sh.v[d] + v_off[db]);
    if (partial) {  // element i of a fragment is key 4 lg + i
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        va[db].x &= (4 * lg + 0 < valid ? 0x0000FFFFu : 0u) | (4 * lg + 1 < valid ? 0xFFFF0000u : 0u);
        va[db].y &= (4 * lg + 2 < valid ? 0x0000FFFFu : 0u) | (4 * lg + 3 < valid ? 0xFFFF0000u : 0u);
      }
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      acc[db] = mfma_16x16x16(va[db], u, acc[db]);
      acc[db] = mfma_16x16x16(va[db], w, acc[db]);
    }
  }

  // Every lane group holds partial weight sums against the same reference maximum.
  __device__ __forceinline__ void finish(Shared&) {
    float l = l_sum;
    l += partner16(l, lane);
    l += partner32(l, lane);
    l_tot = l;
  }

  // out[h0 + c][16 db + 4 lg + i] = acc / L for the GW heads starting at `op` (head stride D).
  __device__ __forceinline__ void store_output(uint16_t* op, Shared&) const {
    if (c >= GW) return;
    const float inv = 1.0f / l_tot;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const uint32_t w0 = pack_bf16x2(acc[db][0] * inv, acc[db][1] * inv);
      const uint32_t w1 = pack_bf16x2(acc[db][2] * inv, acc[db][3] * inv);
      *reinterpret_cast<uint2*>(op + c * D + 16 * db + 4 * lg) = make_uint2(w0, w1);
    }
  }

  // The un-normalised partial of head c to po + c * po_head_stride and (M, L) to pml + c * pml_head_stride.
  __device__ __forceinline__ void store_partial(float* po, int64_t po_head_stride, float* pml, int64_t pml_head_stride,
                                                Shared&) const {
    if (c >= GW) return;
#pragma unroll
    for (int db = 0; db < DB; ++db)
      *reinterpret_cast<float4*>(po + c * po_head_stride + 16 * db + 4 * lg) =
          make_float4(acc[db][0], acc[db][1], acc[db][2], acc[db][3]);
    if (lg == 0) *reinterpret_cast<float2*>(pml + c * pml_head_stride) = make_float2(m_ref, l_tot);
  }

  // Before the wave ends: no load into LDS may still be in flight.
  __device__ __forceinline__ void drain() const { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
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
