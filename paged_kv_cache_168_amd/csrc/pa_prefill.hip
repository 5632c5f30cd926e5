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
// waves takes 64 * PB (query row, query head) pairs of one kv head (64 * PB / G rows of all G heads
// of the GQA group) and walks the keys in 64-key steps:
//   * each step's 64 x D tiles of K and V are gathered through the block table into one of two LDS
//     buffers and used by all pairs of the work-group; the next step's tiles and the block ids of the
//     step after it are loaded while the current step computes, so one barrier per step suffices;
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (A = K from LDS, B = the wave's query rows held in
//     registers): each lane holds one pair and 16 of the 64 keys, so the row maximum and sum need
//     only two cross-lane swaps;
//   * the online softmax rescales the accumulators only when a row maximum rises by more than 2^8
//     (weights stay <= 2^8); masking (causal horizon, end of the work-group's keys) is a select, and
//     only steps that reach a row's horizon evaluate it;
//   * O^T += V^T P^T on the same instruction: P^T is the lane's own weights (no data movement), split
//     into a bf16 head and a bf16 tail so that they keep about 16 significant bits (one bf16
//     rounding of the weights alone can cost 2^-8 of the largest |v|, which the bf16 error budget
//     cannot absorb); V^T comes from LDS with the transposing read ds_read_b64_tr_b16.
// By default a work-group covers all keys its rows see. With a caller-set partition size the keys
// are cut into partitions: rows whose keys span several partitions write (max, sum, un-normalised
// output) partials that the log-sum-exp merge kernel combines.
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
constexpr int kStepKeys = 64;         // keys per step

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

// Weights w0, w1 as two bf16 terms each: head = bf16(w), tail = bf16(w - head).
__device__ __forceinline__ void split_bf16x2(float w0, float w1, uint32_t& head, uint32_t& tail) {
  const __bf16 h0 = (__bf16)w0, h1 = (__bf16)w1;
  head = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
  tail = pack_bf16x2(w0 - (float)h0, w1 - (float)h1);
}

template <int D, int PB>
__global__ __launch_bounds__(kPrefillThreads) void prefill_mfma_kernel(AttnArgs a) {
  constexpr int KS = D / 32;                 // 32-wide steps of the q.k contraction
  constexpr int DB = D / 16;                 // 16-wide blocks of the output columns
  constexpr int KT = kStepKeys;              // keys per step
  constexpr int KB = KT / 16;                // 16-key blocks per step
  constexpr int CPR = D / 8;                 // 16-byte chunks per key row
  constexpr int NCH = KT * CPR / kPrefillThreads;  // chunks of K (and of V) each thread moves per step
  constexpr int KROW = D + 8;                // LDS row strides (elements), padded against bank conflicts
  constexpr int VROW = D + 16;
  constexpr int BUF = KT * (KROW + VROW);    // one buffer: K rows then V rows
  constexpr int PAIRS = 4 * 16 * PB;         // (row, head) pairs per work-group
  static_assert(NCH * kPrefillThreads == KT * CPR, "tile must split evenly over the threads");
  __shared__ __align__(16) uint16_t lds[2 * BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = lane & 15;   // MFMA column: this lane's pair within a 16-pair block
  const int lg = lane >> 4;  // lane group: keys 4*lg.. of each 16-key block, d 8*lg.. of each 32-wide step

  int id = blockIdx.x;  // kv head fastest: work-groups sharing K/V land on the same XCD
  const int kvh = id % a.num_kv_heads;
  id /= a.num_kv_heads;
  const int part = id % a.chunk_partitions;
  const int tile = id / a.chunk_partitions;
  if (tile >= *a.tile_count) return;
  const int s = a.tiles[2 * tile];
  const int row0 = a.tiles[2 * tile + 1];
  const int q0 = a.query_start_loc[s];
  const int q_len = a.query_start_loc[s + 1] - q0;
  const int max_ctx = a.max_blocks * a.block_size;
  const int ctx = min(max(a.context_lens[s], 0), max_ctx);
  const int G = a.group;
  const int rows_here = min(PAIRS / G, q_len - row0);
  const int PT = a.chunk_partition_tokens > 0 ? a.chunk_partition_tokens : max_ctx;
  const int kbeg = part * PT;

  // this lane's (query row, query head) pair in each of its PB pair blocks
  int lim[PB];
  bool live[PB];
  int64_t orow[PB];
  int nvis[PB];
  uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
  for (int pb = 0; pb < PB; ++pb) {
    const int pair = (wave * PB + pb) * 16 + c;
    const int rl = pair / G;
    const int j = row0 + rl;
    const int t = q0 + j;
    live[pb] = rl < rows_here && t >= 0 && t < a.num_tokens;
    const int h = kvh * G + (pair - rl * G);
    nvis[pb] = live[pb] ? min(ctx - q_len + j + 1, ctx) : 0;
    orow[pb] = ((int64_t)t * a.num_q_heads + h) * D;
    lim[pb] = min(nvis[pb], kbeg + PT);
    if (part == 0 && live[pb] && nvis[pb] <= 0) {  // no visible key: the row is defined as zeros
#pragma unroll
      for (int db = 0; db < DB; ++db) *reinterpret_cast<uint2*>(out + orow[pb] + 16 * db + 4 * lg) = make_uint2(0, 0);
    }
  }
  // keys the last row of the tile sees bound what the work-group reads
  const int last_vis = min(ctx - q_len + row0 + rows_here, ctx);
  const int kend = min(kbeg + PT, last_vis);
  if (rows_here <= 0 || kbeg >= kend) return;
  // keys every row of the tile sees: steps ending at or before this need no mask
  const int mask_from = min(max(ctx - q_len + row0 + 1, 0), kend);
  const int nsteps = ceil_div(kend - kbeg, KT);

  // queries: B operand of S^T = K Q^T (lane holds q[pair][32 ks + 8 lg .. + 7])
  uint4 qb[PB][KS];
#pragma unroll
  for (int pb = 0; pb < PB; ++pb) {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + orow[pb] + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qb[pb][ks] = live[pb] ? *reinterpret_cast<const uint4*>(qp + 32 * ks) : make_uint4(0, 0, 0, 0);
  }

  // gather: chunk n of this thread is key (tid + n * 256) / CPR of a step, 16-byte column (tid % CPR)
  const int BS = a.block_size;
  const bool bs_pow2 = (BS & (BS - 1)) == 0;
  const int bs_shift = __builtin_ctz(BS);
  const int32_t* tab = a.block_tables + (int64_t)s * a.max_blocks;
  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache) + (int64_t)kvh * D + (tid % CPR) * 8;
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache) + (int64_t)kvh * D + (tid % CPR) * 8;
  const int64_t slot_stride = (int64_t)a.num_kv_heads * D;
  auto key_of = [&](int n) { return (tid + n * kPrefillThreads) / CPR; };
  // Every load below is unconditional: a key past the work-group's keys is replaced by its last key
  // (a key of the request, inside the pool), and its data are replaced by zeros when they are written
  // to LDS. Block ids are kept as loaded and clamped only where an address is formed, so no load is
  // waited for before the next step needs it.
  auto load_ids = [&](int k0, int (&ids)[NCH]) {
#pragma unroll
    for (int n = 0; n < NCH; ++n) {
      const int pos = min(k0 + key_of(n), kend - 1);
      ids[n] = tab[bs_pow2 ? pos >> bs_shift : pos / BS];
    }
  };
  uint4 kr[NCH], vr[NCH];
  auto load_kv = [&](int k0, const int (&ids)[NCH]) {
#pragma unroll
    for (int n = 0; n < NCH; ++n) {
      const int pos = min(k0 + key_of(n), kend - 1);
      const int slot = bs_pow2 ? pos & (BS - 1) : pos % BS;
      const int64_t off = ((int64_t)clamp_block(ids[n], a.num_blocks) * BS + slot) * slot_stride;
      kr[n] = *reinterpret_cast<const uint4*>(kc + off);
      vr[n] = *reinterpret_cast<const uint4*>(vc + off);
    }
  };
  auto store_kv = [&](int buf, int k0) {
    uint16_t* sk = lds + buf * BUF;
    uint16_t* sv = sk + KT * KROW;
#pragma unroll
    for (int n = 0; n < NCH; ++n) {
      const int key = key_of(n), dc = tid % CPR;
      const uint32_t keep = k0 + key < kend ? 0xFFFFFFFFu : 0u;
      const uint4 kk = kr[n], vv = vr[n];
      *reinterpret_cast<uint4*>(sk + key * KROW + dc * 8) = make_uint4(kk.x & keep, kk.y & keep, kk.z & keep, kk.w & keep);
      *reinterpret_cast<uint4*>(sv + key * VROW + dc * 8) = make_uint4(vv.x & keep, vv.y & keep, vv.z & keep, vv.w & keep);
    }
  };

  f32x4_t acc[DB][PB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) acc[db][pb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_ref[PB], lsum[PB];
#pragma unroll
  for (int pb = 0; pb < PB; ++pb) {
    m_ref[pb] = kNegInf;
    lsum[pb] = 0.0f;
  }
  // transposing-read addresses of the V^T operand: rows 4 lg + c / 4 (and + 16), columns 4 (c % 4)
  const int vrow = 4 * lg + (c >> 2);
  const int vcol = 4 * (c & 3);

  // prologue: step 0 into buffer 0, block ids of step 1 in flight
  int ids[NCH];
  load_ids(kbeg, ids);
  load_kv(kbeg, ids);
  if (nsteps > 1) load_ids(kbeg + KT, ids);
  store_kv(0, kbeg);
  __syncthreads();

  for (int it = 0; it < nsteps; ++it) {
    const int k0 = kbeg + it * KT;
    const bool more = it + 1 < nsteps;
    if (more) {  // next step's K/V and the block ids of the step after it, in flight while this step computes
      load_kv(k0 + KT, ids);
      if (it + 2 < nsteps) load_ids(k0 + 2 * KT, ids);
    }
    const uint16_t* sk = lds + (it & 1) * BUF;
    const uint16_t* sv = sk + KT * KROW;

    // S^T for keys k0 + 16 kb + (0..15): lane holds keys 16 kb + 4 lg + i of its pairs
    f32x4_t st[KB][PB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int pb = 0; pb < PB; ++pb) st[kb][pb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const uint4 ka = *reinterpret_cast<const uint4*>(sk + (16 * kb + c) * KROW + 32 * ks + 8 * lg);
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) st[kb][pb] = mfma_bf16(ka, qb[pb][ks], st[kb][pb]);
      }
    }

    // scores in log2 units; masked keys (past a row's horizon or the work-group's keys) select -inf
    const bool masked = k0 + KT > mask_from;
    float tmax[PB];
    bool need = false;
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) {
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = st[kb][pb][i] * a.scale_log2;
          if (masked) x = (k0 + 16 * kb + 4 * lg + i < lim[pb]) ? x : kNegInf;
          st[kb][pb][i] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = fmaxf(mx, partner16(mx, lane));
      mx = fmaxf(mx, partner32(mx, lane));
      tmax[pb] = mx;
      need |= mx > m_ref[pb] + kRescaleSlack;
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int pb = 0; pb < PB; ++pb) {
        const float m_new = fmaxf(m_ref[pb], tmax[pb]);
        const float alpha = (m_new == m_ref[pb]) ? 1.0f : __builtin_amdgcn_exp2f(m_ref[pb] - m_new);
        m_ref[pb] = m_new;
        lsum[pb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db][pb] *= alpha;
      }
    }
    // weights (<= 2^8) as bf16 head + tail B operands of O^T += V^T P^T: for the 32-key half hf, lane
    // (lg, c) holds keys 4 lg + i of 16-key blocks 2 hf and 2 hf + 1
    uint4 pw[KB / 2][PB], pt[KB / 2][PB];
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) {
      const float base = m_ref[pb] == kNegInf ? 0.0f : m_ref[pb];
      float ps = 0.0f;
#pragma unroll
      for (int hf = 0; hf < KB / 2; ++hf) {
        uint32_t w[4], u[4];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const float p0 = __builtin_amdgcn_exp2f(st[2 * hf + b][pb][0] - base);
          const float p1 = __builtin_amdgcn_exp2f(st[2 * hf + b][pb][1] - base);
          const float p2 = __builtin_amdgcn_exp2f(st[2 * hf + b][pb][2] - base);
          const float p3 = __builtin_amdgcn_exp2f(st[2 * hf + b][pb][3] - base);
          ps += (p0 + p1) + (p2 + p3);
          split_bf16x2(p0, p1, w[2 * b], u[2 * b]);
          split_bf16x2(p2, p3, w[2 * b + 1], u[2 * b + 1]);
        }
        pw[hf][pb] = make_uint4(w[0], w[1], w[2], w[3]);
        pt[hf][pb] = make_uint4(u[0], u[1], u[2], u[3]);
      }
      lsum[pb] += ps;
    }
    // O^T += V^T P^T: A element e of lane (lg, c) is V[key e < 4 ? 4 lg + e : 12 + 4 lg + e][16 db + c]
    // (keys relative to the half's first key)
#pragma unroll
    for (int hf = 0; hf < KB / 2; ++hf) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint2 v0 = lds_read_tr(sv + (32 * hf + vrow) * VROW + 16 * db + vcol);
        const uint2 v1 = lds_read_tr(sv + (32 * hf + 16 + vrow) * VROW + 16 * db + vcol);
        const uint4 va = make_uint4(v0.x, v0.y, v1.x, v1.y);
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) {
          acc[db][pb] = mfma_bf16(va, pt[hf][pb], acc[db][pb]);
          acc[db][pb] = mfma_bf16(va, pw[hf][pb], acc[db][pb]);
        }
      }
    }
    if (more) store_kv((it + 1) & 1, k0 + KT);
    __syncthreads();
  }

#pragma unroll
  for (int pb = 0; pb < PB; ++pb) {
    // the four lane groups of a pair hold partial sums against the same reference maximum
    float l = lsum[pb];
    l += partner16(l, lane);
    l += partner32(l, lane);
    if (!live[pb] || lim[pb] <= kbeg) continue;  // this pair has no key in this partition
    const int n_parts = a.chunk_partition_tokens > 0 ? ceil_div(nvis[pb], PT) : 1;
    if (n_parts == 1) {
      const float inv = 1.0f / l;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint32_t w0 = pack_bf16x2(acc[db][pb][0] * inv, acc[db][pb][1] * inv);
        const uint32_t w1 = pack_bf16x2(acc[db][pb][2] * inv, acc[db][pb][3] * inv);
        *reinterpret_cast<uint2*>(out + orow[pb] + 16 * db + 4 * lg) = make_uint2(w0, w1);
      }
    } else {
      const int64_t slot = (orow[pb] / D) * a.max_partitions + part;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<float4*>(a.part_o + slot * D + 16 * db + 4 * lg) =
            make_float4(acc[db][pb][0], acc[db][pb][1], acc[db][pb][2], acc[db][pb][3]);
      if (lg == 0) *reinterpret_cast<float2*>(a.part_ml + slot * 2) = make_float2(m_ref[pb], l);
    }
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

constexpr int kPrefillPairBlocks = 1;  // 16-pair blocks per wave
constexpr int kPrefillPairs = 64 * kPrefillPairBlocks;

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
  if (a.chunk_partitions < 1) return hipErrorInvalidValue;
  const int64_t grid = (int64_t)a.tile_capacity * a.chunk_partitions * a.num_kv_heads;
  if (grid <= 0) return hipSuccess;
  if (head_dim == 128)
    prefill_mfma_kernel<128, kPrefillPairBlocks><<<dim3((unsigned)grid), dim3(kPrefillThreads), 0, s>>>(a);
  else if (head_dim == 64)
    prefill_mfma_kernel<64, kPrefillPairBlocks><<<dim3((unsigned)grid), dim3(kPrefillThreads), 0, s>>>(a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
