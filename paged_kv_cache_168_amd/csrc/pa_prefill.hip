// Chunked-prefill rows on MFMA (gfx950): attention of the query rows of requests with q_len > 1.
//
// What is computed is the same attention as the decode kernels ("Continuous batching: a paradigm
// shift in inference throughput", section 4.1: keys and values reached block by block through the
// block table, scaled dot products, softmax, weighted sum of V), with the causal horizon of a
// prefill slice: row j of a slice of q_len rows sees keys 0 .. ctx - q_len + j. The slice's own keys
// are already in the paged cache ("PagedAttention memory paging and continuous batching in
// practice", chunked-prefill section: prefill slices batched with the running decodes).
//
// A prefill slice is a dense contraction, so it runs on the matrix cores. A group of four waves (a
// "half") takes 64 * PB (query row, query head) pairs of one kv head (64 * PB / G rows of all G heads
// of the GQA group) and walks the keys in steps of KT keys; a work-group of several halves gives the
// steps to its halves in turn and folds their results at the end:
//   * each step's KT x D tiles of K and V go from global memory straight into one of two LDS buffers
//     (global_load_lds_dwordx4: no register staging, no LDS store instructions) and are used by all
//     pairs of the half. Each gather instruction's 1 KB of rows is followed by 64 bytes of padding and
//     the 16-byte chunks of a row are permuted by a two-bit XOR, so the fragment reads below hit distinct
//     banks and each of them is one base register plus an immediate offset. The next step's tiles and
//     the block ids of the step after it are in flight while the current step computes: one barrier per step;
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (A = K from LDS, B = the wave's query rows held in
//     registers): each lane holds one pair and four keys of each 16-key block, so the row maximum and
//     sum need only two cross-lane swaps;
//   * the online softmax rescales a pair's accumulators only when its own row maximum rises by more than 8 in
//     log2 units (weights stay <= 2^8); the scale is folded into one fma before the exponential (a negative
//     scale flips the sign of q instead); masking (causal horizon, end of the work-group's keys) is a
//     select, and only steps that reach a row's horizon evaluate it;
//   * O^T += V^T P^T on the same instruction: P^T is the lane's own weights (no data movement), split
//     into a bf16 head and a bf16 tail so that they keep about 16 significant bits (one bf16
//     rounding of the weights alone can cost 2^-8 of the largest |v|, which the bf16 error budget
//     cannot absorb); V^T comes from LDS with the transposing read ds_read_b64_tr_b16.
// By default a work-group covers all keys its rows see. With a caller-set partition size the keys
// are cut into partitions: rows whose keys span several partitions write (max, sum, un-normalised
// output) partials that the log-sum-exp merge kernel combines.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

using namespace dev;


// Chunk swizzle of row q of a group of key rows in LDS (see the tile layout in the kernel): two bits, so that
// rows 0-3 get 0-3 and rows 4-7 get 1, 0, 3, 2.
__device__ __forceinline__ int swz(int q) { return (q ^ (q >> 2)) & 3; }

// A wave-uniform address held in scalar registers, so that adding a lane's 32-bit offset gives a load with a
// scalar base and a vector offset (no 64-bit vector address arithmetic per load).
__device__ __forceinline__ const char* scalar_base(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

// Barrier after which the loads into LDS that any wave of the work-group issued before it have landed:
// each wave first waits for its own vector-memory operations (vmcnt(0); a work-group barrier alone
// does not wait for loads into LDS).
__device__ __forceinline__ void lds_loads_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt unconstrained
  __syncthreads();
}

// kPrefix: the shared-prefix pass of a decode batch. A tile is then (group g, first row): its rows are
// the decode requests group_start[g] + row (query row = request), which all read the group's prefix keys
// 0 .. P - 1 through the table of the group's first request; a request sees min(P, its context length)
// of them. The prefix keys are cut into partitions of a.chunk_partition_tokens keys, one work-group each; every
// row leaves its (max, sum, un-normalised output) partial of each partition it sees keys of in a.part_ml /
// a.part_o at slot (request * Hq + head) * max_partitions + partition, for the merge with the rest of its keys.
// A work-group is HALVES halves of WPH waves; each wave holds PB blocks of 16 (row, head) pairs, so a half holds
// 16 * WPH * PB pairs. Every wave reads a step's whole K and V tiles from LDS, so more pairs per wave (PB) means
// fewer LDS bytes per flop, at the cost of registers.
// KT: keys per step (a multiple of 32).
template <int D, int PB, int WPH, int HALVES, bool kPrefix, int KT = 64>
__global__ __launch_bounds__(64 * WPH * HALVES) void prefill_mfma_kernel(AttnArgs a) {
  constexpr int KS = D / 32;                 // 32-wide steps of the q.k contraction
  constexpr int DB = D / 16;                 // 16-wide blocks of the output columns
  static_assert(KT % 32 == 0, "a step is whole 32-key blocks");
  constexpr int KB = KT / 16;                // 16-key blocks per step
  constexpr int CPR = D / 8;                 // 16-byte chunks per key row
  constexpr int ROWB = D * 2;                // bytes per key row in LDS
  constexpr int HT = 64 * WPH;               // threads of one half
  constexpr int NI = KT * CPR / HT;          // wave instructions per tile (K or V) per wave of a half
  // LDS tile layout: one gather instruction writes 64 x 16 bytes = RPI key rows; such a group of rows is
  // followed by 64 bytes of padding, and within a group the 16-byte chunk j of row q sits at position
  // j ^ swz(q), swz(q) < 4. Padding and swizzle put the sixteen rows of a fragment read on distinct banks, and
  // since the swizzle only touches the two low bits of a chunk index, fragments that differ in the high bits
  // (another 32-wide step of the contraction, another pair of 16-wide output blocks, other rows) are a
  // constant byte offset apart: every fragment read is one base register plus an immediate.
  constexpr int RPI = 64 / CPR;              // key rows per gather instruction (one group)
  constexpr int GROUPB = 64 * 16 + 64;       // bytes per group of RPI rows, padding included
  constexpr int TILEB = KT / RPI * GROUPB;   // bytes of one K (or V) tile
  constexpr int TILE = TILEB / 2;            // the same in elements
  static_assert(16 % RPI == 0, "a fragment's 16 rows are whole groups");
  constexpr int ROWS16 = 16 / RPI * GROUPB;  // bytes between rows r and r + 16
  constexpr int PAIRS = WPH * 16 * PB;       // (row, head) pairs per work-group (each half holds all of them)
  static_assert(NI * HT == KT * CPR, "tile must split evenly over the threads of a half");
  // [half][buffer][K, V] tiles of TILEB bytes in the group layout above
  __shared__ __align__(16) uint16_t lds[HALVES * 2 * 2 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform indices, held in scalar registers (the LDS destinations of the tile loads derive from them)
  const int half = __builtin_amdgcn_readfirstlane(tid / HT);        // takes steps it = half, half + HALVES, ...
  const int wave = __builtin_amdgcn_readfirstlane((tid % HT) >> 6); // wave within the half
  const int c = lane & 15;   // MFMA column: this lane's pair within a 16-pair block
  const int lg = lane >> 4;  // lane group: keys 4*lg.. of each 16-key block, d 8*lg.. of each 32-wide step

  int id = blockIdx.x;  // kv head fastest: work-groups sharing K/V land on the same XCD
  const int kvh = id % a.num_kv_heads;
  id /= a.num_kv_heads;
  const int part = id % a.chunk_partitions;
  const int tile = id / a.chunk_partitions;
  if (tile >= *a.tile_count) return;
  const int row0 = a.tiles[2 * tile + 1];
  const int max_ctx = a.max_blocks * a.block_size;
  int s, q0, q_len, ctx;
  if constexpr (kPrefix) {  // s: the group's first request, whose table holds the shared blocks
    const int g = a.tiles[2 * tile];
    q0 = min(max(a.group_start[g], 0), a.num_seqs);
    q_len = min(max(a.group_start[g + 1], q0), a.num_seqs) - q0;
    s = q0;
    // the prefix keys: at most the first request's context, whole blocks (the same rule as the plan)
    ctx = min(min(max(a.group_prefix[g], 0), max_ctx), q_len > 0 ? max(a.context_lens[q0], 0) : 0);
    ctx -= ctx % a.block_size;
  } else {
    s = a.tiles[2 * tile];
    q0 = a.query_start_loc[s];
    q_len = a.query_start_loc[s + 1] - q0;
    ctx = min(max(a.context_lens[s], 0), max_ctx);
  }
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
    if constexpr (kPrefix) nvis[pb] = live[pb] ? min(ctx, max(a.context_lens[t], 0)) : 0;
    else nvis[pb] = live[pb] ? min(ctx - q_len + j + 1, ctx) : 0;
    orow[pb] = live[pb] ? ((int64_t)t * a.num_q_heads + h) * D : 0;
    lim[pb] = min(nvis[pb], kbeg + PT);
    if (!kPrefix && half == 0 && part == 0 && live[pb] && nvis[pb] <= 0) {  // no visible key: zeros
#pragma unroll
      for (int db = 0; db < DB; ++db) *reinterpret_cast<uint2*>(out + orow[pb] + 16 * db + 4 * lg) = make_uint2(0, 0);
    }
  }
  // keys the last row of the tile sees bound what the work-group reads
  const int last_vis = kPrefix ? ctx : min(ctx - q_len + row0 + rows_here, ctx);
  const int kend = min(kbeg + PT, last_vis);
  if (rows_here <= 0 || kbeg >= kend) return;
  // keys every row of the tile sees: steps ending at or before this need no mask
  int mask_from = min(max(ctx - q_len + row0 + 1, 0), kend);
  if constexpr (kPrefix) {  // a request shorter than the prefix sees fewer keys
    mask_from = kend;
    for (int r = 0; r < rows_here; ++r) mask_from = min(mask_from, max(a.context_lens[q0 + row0 + r], 0));
  }
  const int nsteps = ceil_div(kend - kbeg, KT);

  // queries: B operand of S^T = K Q^T (lane holds q[pair][32 ks + 8 lg .. + 7]); a negative scale is
  // applied as |scale| to sign-flipped queries, so that the row maximum of q.k * scale is the scale
  // times the row maximum of the (flipped) dot products
  const float c2 = fabsf(a.scale_log2);
  const uint32_t qflip = a.scale_log2 < 0.0f ? 0x80008000u : 0u;
  uint4 qb[PB][KS];
#pragma unroll
  for (int pb = 0; pb < PB; ++pb) {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + orow[pb] + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = *reinterpret_cast<const uint4*>(qp + 32 * ks);
      const uint32_t keep = live[pb] ? 0xFFFFFFFFu : 0u;
      qb[pb][ks] = make_uint4((v.x ^ qflip) & keep, (v.y ^ qflip) & keep, (v.z ^ qflip) & keep, (v.w ^ qflip) & keep);
    }
  }

  // Gather. Wave instruction i of wave w of a half fills group w * NI + i of a tile: lane l writes chunk
  // position l % CPR of the group's row l / CPR, which holds that row's chunk (l % CPR) ^ swz(l / CPR).
  // A key past the work-group's keys loads the last key instead (a key of the request, finite); its
  // scores are masked and its weights are zero.
  const int BS = a.block_size;
  const bool bs_pow2 = (BS & (BS - 1)) == 0;
  const int bs_shift = __builtin_ctz(BS);
  const int32_t* tab = a.block_tables + (int64_t)s * a.max_blocks;
  const char* kc = reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.k_cache) + (int64_t)kvh * a.head_stride);
  const char* vc = reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.v_cache) + (int64_t)kvh * a.head_stride);
  // byte strides; a block's bytes fit 32 bits (the host takes this kernel only then), so a key row's offset is one
  // 32 x 32 -> 64-bit multiply-add: block * block_bytes + (slot * slot_bytes + chunk offset)
  const uint32_t block_bytes = (uint32_t)(a.block_stride * 2);
  const uint32_t slot_bytes = (uint32_t)(a.slot_stride * 2);
  uint16_t* my_lds = lds + half * 2 * 2 * TILE;
  // A gather instruction covers RPI consecutive key rows. When blocks hold a power-of-two multiple of RPI rows
  // and the work-group's first key is a multiple of RPI, those rows lie in one block: on every step that ends
  // inside the work-group's keys (no row is clamped), the block id and the first row's slot are wave-uniform
  // (scalar arithmetic) and a lane adds only its fixed offset lane_off within the rows. Other steps, and other
  // block sizes, take each lane's row apart.
  const bool uni_rows = bs_pow2 && BS % RPI == 0 && kbeg % RPI == 0;
  const int lrow = lane / CPR;  // the lane's key row within its instruction's RPI rows
  // the lane's offset within those rows in the cache: it fills chunk position lane % CPR of row lrow
  const uint32_t lane_off = (uint32_t)lrow * slot_bytes + (uint32_t)(((lane % CPR) ^ swz(lrow)) * 16);
  // The block table through the constant address space: a wave-uniform entry is then a scalar load (the table
  // does not change while the kernel runs).
  typedef const __attribute__((address_space(4))) int32_t* const_table_t;
  const const_table_t ctab = (const_table_t)(tab);
  auto uni_step = [&](int k0) { return uni_rows && k0 + KT <= kend; };
  // block ids of the uniform path, loaded a step ahead into scalar registers
  int sids[NI];
  auto load_ids = [&](int k0) {
    if (uni_step(k0)) {
#pragma unroll
      for (int i = 0; i < NI; ++i) sids[i] = ctab[(k0 + (wave * NI + i) * RPI) >> bs_shift];
    }
  };
  auto issue_kv = [&](int k0, int buf) {
    uint16_t* sk = my_lds + buf * 2 * TILE;
    if (uni_step(k0)) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int rb = k0 + (wave * NI + i) * RPI;
        const uint64_t boff = (uint64_t)(uint32_t)clamp_block(sids[i], a.num_blocks) * block_bytes +
                              (uint32_t)(rb & (BS - 1)) * slot_bytes;
        uint16_t* dst = sk + (wave * NI + i) * (GROUPB / 2);
        load_to_lds<false>(scalar_base(kc + boff) + lane_off, dst);
        load_to_lds<false>(scalar_base(vc + boff) + lane_off, dst + TILE);
      }
      // (an empty statement that keeps the compiler from sharing the last loads' code with the path below,
      // which would move the uniform addresses into vector registers)
      asm volatile("");
      return;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int pos = min(k0 + (wave * NI + i) * RPI + lrow, kend - 1);
      const int slot = bs_pow2 ? pos & (BS - 1) : pos - (pos / BS) * BS;
      const int id = tab[bs_pow2 ? pos >> bs_shift : pos / BS];
      // the lane's slot in place of its unclamped row's (32-bit arithmetic modulo 2^32; the sum fits a block)
      const uint64_t off = (uint64_t)(uint32_t)clamp_block(id, a.num_blocks) * block_bytes +
                           ((uint32_t)slot * slot_bytes + lane_off - (uint32_t)lrow * slot_bytes);
      uint16_t* dst = sk + (wave * NI + i) * (GROUPB / 2);
      load_to_lds<false>(kc + off, dst);
      load_to_lds<false>(vc + off, dst + TILE);
    }
  };

  f32x4_t acc[DB][PB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) acc[db][pb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // per pair: reference maximum (log2 units), the rescale threshold m_ref + slack, the exponent bias -m_ref
  // (0 while m_ref is -inf), and the weights' sum
  float m_ref[PB], thr[PB], nb[PB], lsum[PB];
#pragma unroll
  for (int pb = 0; pb < PB; ++pb) {
    m_ref[pb] = kNegInf;
    thr[pb] = kNegInf;
    nb[pb] = 0.0f;
    lsum[pb] = 0.0f;
  }
  // LDS byte offsets of this lane's fragments within a buffer. K (A of S^T): row 16 kb + c, chunk
  // 4 ks + lg, at k_base + kb * ROWS16 + 64 ks. V^T (A of O^T, transposing read): row 32 hf + 16 h + 4 lg + c / 4,
  // elements 16 db + 4 (c % 4) .. + 3, i.e. chunk 2 db + (c % 4) / 2, byte 8 (c % 2) of it, at
  // v_base[db % 2] + 64 (db / 2) + (2 hf + h) * ROWS16.
  const int k_base = (c / RPI) * GROUPB + (c % RPI) * ROWB + 16 * (lg ^ swz(c % RPI));
  const int vr = 4 * lg + (c >> 2);
  int v_base[2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
    v_base[par] = TILEB + (vr / RPI) * GROUPB + (vr % RPI) * ROWB + 16 * ((2 * par + ((c & 3) >> 1)) ^ swz(vr % RPI)) +
                  8 * (c & 1);

  // prologue: this half's first step into its buffer 0, block ids of its second step in flight
  if (half < nsteps) {
    load_ids(kbeg + half * KT);
    issue_kv(kbeg + half * KT, 0);
    if (half + HALVES < nsteps) load_ids(kbeg + (half + HALVES) * KT);
  }
  lds_loads_barrier();

  // One step of this half. kMasked: the step reaches a row's horizon or the end of the work-group's
  // keys (only the last steps of a work-group), so scores and weights of keys a row may not see are
  // replaced.
  // buf: the LDS buffer of the step, (it / HALVES) & 1 (a constant in the unrolled hot loop, so that every
  // fragment read is an immediate offset from a fixed base).
  auto step = [&](int it, int buf, auto masked_tag) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    const int k0 = kbeg + it * KT;
    if (it + HALVES < nsteps) {  // this half's next step and the block ids of the one after, in flight meanwhile
      issue_kv(k0 + HALVES * KT, buf ^ 1);
      if (it + 2 * HALVES < nsteps) load_ids(k0 + 2 * HALVES * KT);
    }
    const char* bb = reinterpret_cast<const char*>(my_lds + buf * 2 * TILE);

    // S^T for keys k0 + 16 kb + (0..15): lane holds keys 16 kb + 4 lg + i of its pairs. All K fragments
    // of the step are read first, so the LDS reads are in flight together.
    uint4 ka[KS][KB];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) ka[ks][kb] = *reinterpret_cast<const uint4*>(bb + k_base + kb * ROWS16 + 64 * ks);
    f32x4_t st[KB][PB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int pb = 0; pb < PB; ++pb) st[kb][pb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) st[kb][pb] = mfma_16x16x32(ka[ks][kb], qb[pb][ks], st[kb][pb]);
    // V^T fragments of the step (A element e of lane (lg, c) is V[key e < 4 ? 4 lg + e : 12 + 4 lg + e]
    // [16 db + c], keys relative to the first key of the 32-key half): read now, used after the softmax
    uint4 va[KB / 2][DB];
#pragma unroll
    for (int hf = 0; hf < KB / 2; ++hf)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const char* vp = bb + v_base[db & 1] + 64 * (db >> 1) + 2 * hf * ROWS16;
        const uint2 v0 = lds_read_tr(reinterpret_cast<const uint16_t*>(vp));
        const uint2 v1 = lds_read_tr(reinterpret_cast<const uint16_t*>(vp + ROWS16));
        va[hf][db] = make_uint4(v0.x, v0.y, v1.x, v1.y);
      }

    // maxima of the dot products over the lane's own keys; masked keys (past a row's horizon or the
    // work-group's keys) select -inf. A pair's maximum exceeds the slack above its reference exactly when one
    // of its lanes' maxima does (the scale is not negative), so the cross-lane maximum is taken only then.
    float lmax[PB];
    bool need = false;
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) {
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (kMasked) st[kb][pb][i] = (k0 + 16 * kb + 4 * lg + i < lim[pb]) ? st[kb][pb][i] : kNegInf;
          mx = fmaxf(mx, st[kb][pb][i]);
        }
      }
      lmax[pb] = mx;
      need |= mx * c2 > thr[pb];
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      // Only a pair whose own maximum rose past the slack moves its reference: the others keep theirs (weights
      // stay <= 2^8 either way), so no pair's arithmetic depends on the other pairs of its wave, which may see
      // keys it does not.
#pragma unroll
      for (int pb = 0; pb < PB; ++pb) {
        float mx = lmax[pb];
        mx = fmaxf(mx, partner16(mx, lane));
        mx = fmaxf(mx, partner32(mx, lane));
        const float tmax = mx == kNegInf ? kNegInf : mx * c2;  // log2 units
        const float m_new = tmax > thr[pb] ? tmax : m_ref[pb];
        const float alpha = (m_new == m_ref[pb]) ? 1.0f : __builtin_amdgcn_exp2f(m_ref[pb] - m_new);
        m_ref[pb] = m_new;
        thr[pb] = m_new + kRescaleSlack;
        nb[pb] = m_new == kNegInf ? 0.0f : -m_new;
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
      float ps;
#pragma unroll
      for (int hf = 0; hf < KB / 2; ++hf) {
        uint32_t w[4], u[4];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          float p[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[i] = __builtin_amdgcn_exp2f(fmaf(st[2 * hf + b][pb][i], c2, nb[pb]));
            if constexpr (kMasked) p[i] = (k0 + 16 * (2 * hf + b) + 4 * lg + i < lim[pb]) ? p[i] : 0.0f;
          }
          const float g = (p[0] + p[1]) + (p[2] + p[3]);
          ps = hf == 0 && b == 0 ? g : ps + g;
          split_bf16x2(p[0], p[1], w[2 * b], u[2 * b]);
          split_bf16x2(p[2], p[3], w[2 * b + 1], u[2 * b + 1]);
        }
        pw[hf][pb] = make_uint4(w[0], w[1], w[2], w[3]);
        pt[hf][pb] = make_uint4(u[0], u[1], u[2], u[3]);
      }
      lsum[pb] += ps;
    }
    // O^T += V^T P^T
#pragma unroll
    for (int hf = 0; hf < KB / 2; ++hf)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) {
          acc[db][pb] = mfma_16x16x32(va[hf][db], pt[hf][pb], acc[db][pb]);
          acc[db][pb] = mfma_16x16x32(va[hf][db], pw[hf][pb], acc[db][pb]);
        }
  };
  // The halves advance together, one step each per round; a round ends with a barrier (the buffer a
  // half just used is free, the tiles it loads next have landed).
  // Rounds whose steps every row sees entirely run the unmasked step; the last rounds (a row's horizon, the end
  // of the work-group's keys) run the masked one, which is exact on any step. Separate loops keep the accumulators
  // in the same registers through the hot one, which takes two rounds per iteration (buffer 0, then buffer 1), with
  // a last unmasked round after it when their count is odd.
  const int n_full = min(nsteps, max(0, (mask_from - kbeg) / KT));  // steps every row sees entirely
  int r = 0;
  for (; r + 2 * HALVES <= n_full; r += 2 * HALVES) {
    step(r + half, 0, std::false_type{});
    lds_loads_barrier();
    step(r + HALVES + half, 1, std::false_type{});
    lds_loads_barrier();
  }
  if (r + HALVES <= n_full) {
    step(r + half, 0, std::false_type{});
    lds_loads_barrier();
    r += HALVES;
  }
  for (; r < nsteps; r += HALVES) {
    if (r + half < nsteps) step(r + half, (r / HALVES) & 1, std::true_type{});
    lds_loads_barrier();
  }

  // Combine the halves: halves 1 .. HALVES - 1 leave (reference maximum, sum, accumulators) in LDS, half 0 folds
  // them into its own in half order, lane by lane (every half holds the same pairs in the same lanes). The tiles'
  // LDS is free: every wave has passed the last round's barrier.
  if constexpr (HALVES > 1) {
    constexpr int XS = PB * (DB * 4 + 2);  // floats per lane
    static_assert((HALVES - 1) * WPH * 64 * XS * 4 <= (int)sizeof(lds), "the exchange fits the tiles' LDS");
    float* xch = reinterpret_cast<float*>(lds) + (wave * 64 + lane) * XS;
    if (half > 0) {
      float* xh = xch + (half - 1) * WPH * 64 * XS;
#pragma unroll
      for (int pb = 0; pb < PB; ++pb) {
        float* x = xh + pb * (DB * 4 + 2);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[db * 4 + i] = acc[db][pb][i];
        x[DB * 4] = m_ref[pb];
        x[DB * 4 + 1] = lsum[pb];
      }
    }
    __syncthreads();
    if (half > 0) return;
    for (int hh = 1; hh < HALVES; ++hh) {
      const float* xh = xch + (hh - 1) * WPH * 64 * XS;
#pragma unroll
      for (int pb = 0; pb < PB; ++pb) {
        const float* x = xh + pb * (DB * 4 + 2);
        const float mb = x[DB * 4], lb = x[DB * 4 + 1];
        const float mn = fmaxf(m_ref[pb], mb);
        const float wa = m_ref[pb] == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(m_ref[pb] - mn);
        const float wb = mb == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(mb - mn);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[db][pb][i] = acc[db][pb][i] * wa + x[db * 4 + i] * wb;
        m_ref[pb] = mn;
        lsum[pb] = lsum[pb] * wa + lb * wb;
      }
    }
  }

#pragma unroll
  for (int pb = 0; pb < PB; ++pb) {
    // the four lane groups of a pair hold partial sums against the same reference maximum
    float l = lsum[pb];
    l += partner16(l, lane);
    l += partner32(l, lane);
    if (!live[pb] || lim[pb] <= kbeg) continue;  // this pair has no key in this partition
    const int n_parts = kPrefix ? 2 : a.chunk_partition_tokens > 0 ? ceil_div(nvis[pb], PT) : 1;
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

// Shared-prefix pass: (group, first row) tiles of every group with a prefix, and each request's prefix
// length (0 outside such groups). One wave; the group arrays are read 64 groups per round trip and the
// request loop only stores. Group bounds are clamped to the batch; a prefix is cut to the context of the
// group's first request (whose table the prefix pass reads) and to whole blocks. Every request's length
// is stored by the lane that also cleared it, so the two stores keep their order.
__global__ __launch_bounds__(64) void prefix_plan_kernel(AttnArgs a, int32_t* tiles, int32_t* count,
                                                        int rows_per_tile) {
  const int lane = threadIdx.x;
  const int max_ctx = a.max_blocks * a.block_size;
  for (int s = lane; s < a.num_seqs; s += 64) a.item_prefix[s] = 0;
  int base = 0;
  for (int g0 = 0; g0 < a.num_groups; g0 += 64) {
    const int g = g0 + lane;
    int start = 0, size = 0, pre = 0;
    if (g < a.num_groups) {
      start = min(max(a.group_start[g], 0), a.num_seqs);
      size = min(max(a.group_start[g + 1], start), a.num_seqs) - start;
      pre = min(max(a.group_prefix[g], 0), max_ctx);
      if (size > 0) pre = min(pre, max(a.context_lens[start], 0));
      pre -= pre % a.block_size;
    }
    const int n = (pre > 0 && size > 0) ? ceil_div(size, rows_per_tile) : 0;
    const int incl = wave_inclusive_scan(n, lane);
    for (int i = 0; i < n; ++i) {
      const int idx = base + incl - n + i;
      if (idx < a.tile_capacity) {
        tiles[2 * idx] = g;
        tiles[2 * idx + 1] = i * rows_per_tile;
      }
    }
    base += __builtin_amdgcn_readlane(incl, 63);
    const int groups_here = min(64, a.num_groups - g0);
    for (int k = 0; k < groups_here; ++k) {
      const int st = __builtin_amdgcn_readlane(start, k);
      const int sz = __builtin_amdgcn_readlane(size, k);
      const int pk = __builtin_amdgcn_readlane(pre, k);
      for (int i = st + ((lane - st) & 63); i < st + sz; i += 64) a.item_prefix[i] = pk;
    }
  }
  if (lane == 0) *count = min(base, a.tile_capacity);
}

constexpr int kPrefillPairs = 64;  // (row, head) pairs per work-group, every launch shape

}  // namespace

bool prefill_supported(int dtype, int head_dim, int group, int64_t block_bytes) {
  return dtype == 1 && (head_dim == 64 || head_dim == 128) && group >= 1 && group <= kPrefillPairs &&
         kPrefillPairs % group == 0 && block_bytes <= UINT32_MAX;
}

int prefill_rows_per_tile(int group) { return group > 0 && group <= kPrefillPairs ? kPrefillPairs / group : 1; }

hipError_t launch_plan(const AttnArgs& a, int32_t* tiles, int32_t* tile_count, int rows_per_tile, hipStream_t s) {
  prefill_plan_kernel<<<dim3(1), dim3(64), 0, s>>>(a, tiles, tile_count, rows_per_tile);
  return hipGetLastError();
}

// Beside the decode kernel: one half of four waves of 16 pairs, 64-key steps (168 VGPRs, so a chunk wave fits on
// a SIMD next to a decode wave). Alone: four such halves taking 32-key steps in turn (120 VGPRs, four waves per
// SIMD, 136 KB of LDS for bf16 D 128). Measured alone on the 512-row chunk, same box: 41-43.5 us, against 47.5-48.7
// us for two halves of 64-key steps, 46.8-47.7 us for three halves and 53-54 us for two halves of 32-key steps,
// and 48.8-50 us for halves of two waves of 32 pairs (two waves per SIMD, half the LDS bytes per flop).
template <int D>
void launch_prefill_d(const AttnArgs& a, int64_t grid, bool beside_decode, hipStream_t s, KernelTiming tm) {
  if (beside_decode)
    hipExtLaunchKernelGGL(prefill_mfma_kernel<D, 1, 4, 1, false>, dim3((unsigned)grid), dim3(256), 0, s, tm.start,
                          tm.stop, 0, a);
  else
    hipExtLaunchKernelGGL(prefill_mfma_kernel<D, 1, 4, 4, false, 32>, dim3((unsigned)grid), dim3(1024), 0, s,
                          tm.start, tm.stop, 0, a);
}

hipError_t launch_prefix_plan(const AttnArgs& a, int32_t* tiles, int32_t* tile_count, int rows_per_tile,
                              hipStream_t s) {
  prefix_plan_kernel<<<dim3(1), dim3(64), 0, s>>>(a, tiles, tile_count, rows_per_tile);
  return hipGetLastError();
}

hipError_t launch_prefix_pass(const AttnArgs& a, int head_dim, hipStream_t s) {
  const int64_t grid = (int64_t)a.tile_capacity * a.chunk_partitions * a.num_kv_heads;
  if (grid <= 0) return hipSuccess;
  if (head_dim == 128)
    prefill_mfma_kernel<128, 1, 4, 1, true><<<dim3((unsigned)grid), dim3(256), 0, s>>>(a);
  else if (head_dim == 64)
    prefill_mfma_kernel<64, 1, 4, 1, true><<<dim3((unsigned)grid), dim3(256), 0, s>>>(a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_prefill(const AttnArgs& a, int head_dim, bool beside_decode, hipStream_t s, KernelTiming tm) {
  if (a.chunk_partitions < 1) return hipErrorInvalidValue;
  const int64_t grid = (int64_t)a.tile_capacity * a.chunk_partitions * a.num_kv_heads;
  if (grid <= 0) return hipSuccess;
  if (head_dim == 128) launch_prefill_d<128>(a, grid, beside_decode, s, tm);
  else if (head_dim == 64) launch_prefill_d<64>(a, grid, beside_decode, s, tm);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
