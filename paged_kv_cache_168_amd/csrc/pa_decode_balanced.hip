// Balanced ("stream-K") paged-attention decode on gfx950.
//
// The attention itself is the one of "Continuous batching: a paradigm shift in inference
// throughput" (guijiagi.com), section 4.1: per query row, walk the request's logical blocks through
// the block table, score the keys, softmax over the visible keys, weighted sum of V. Section 4.1 also
// describes splitting the work per block and merging the per-block softmax results; here the unit
// of work is a 16-token tile and the merge is by log-sum-exp.
//
// Decomposition. Every (request, kv head, head sub-group) pair is a segment of ceil(ctx / 16) tiles.
// All segments, in (request, segment, tile) order, form one global tile sequence that is cut into
// num_waves contiguous slices of equal cost: a tile costs one unit and, on the vector path, each
// segment start two more (the kernel's prologue gives the measured reason). Every wave therefore does
// about the same work whatever the context-length mix, which is what keeps HBM busy to the end of the
// kernel. A slice covers whole segments and at most two pieces of segments shared with the
// neighbouring waves: a whole segment is normalised and written directly; a piece leaves its
// un-normalised partial (reference maximum, weight sum, weighted values) in slot 0 (the wave's
// first piece) or slot 1 (its last). The piece holding a segment's first tile records its slot and
// the piece holding the last tile records its wave, and merge_balanced_kernel combines the pieces of
// each split segment in wave order, so the result does not depend on timing.
// (Combining inside the decode kernel, by the last wave to finish a piece, was measured slower:
// balanced slices finish together, so the arrivals serialize on one counter and the combine lands
// on the kernel's critical path.)
//
// Caller-set context partitions (partition_tokens > 0; the split-K of section 4.1, partitions merged
// by log-sum-exp): the softmax restarts at every multiple of partition_tokens keys, counted from key 0
// of the context, so each partition has its own maximum and sum. A wave folds the partitions it holds
// by log-sum-exp in registers as they end (the part of a partition in its slice counts as one); pieces
// still end only at segment and slice ends, and the merge folds the pieces of a segment as above.
// (Storing a partial per partition and folding them in a merge kernel took the 8 x 32768 batch with
// 512-token partitions from 167 to 195 us of kernel time, plus 10 us more of merge: each partition end
// then waited for its stores before the next tile.)
//
// Per-tile addressing is resolved ahead of time: a window of 64 tile descriptors (physical slot row,
// kv head, first query head, query row, flags) is built with one lane per tile, 64 tiles before it
// is needed, and the hot loop reads them with v_readlane, so no table load sits between a tile and
// the next K/V loads. DEPTH tiles of K and V (16-byte lane loads, HBM straight to VGPRs, shared by
// the GW query heads of the group) are in flight while a tile is computed.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

using namespace dev;

constexpr int kWindowTiles = 64;
constexpr int kFlagFirst = 32;  // first tile of its segment
constexpr int kFlagLast = 64;   // last tile of its segment
constexpr int kValidMask = 31;  // visible tokens in the tile (1..16)
constexpr int kFlagPrefix = 128;  // the request's shared prefix is handled by the prefix pass
constexpr int kFlagPartFirst = 256;  // caller-set partitions: first tile of a context partition
constexpr int kTileShift = 10;

// What the kernels need to know about request `item`. Its inputs are loaded from addresses that are valid
// in every mode (an unused one repeats the request's context length) with no branch between the loads,
// so they take one round trip together.
struct ItemLens {
  bool decode;  // a decode row (one query) of this batch
  int pre;      // shared-prefix tokens (0 without a prefix pass)
  int nvis;     // keys visible to the decode row (0 when the request is not a decode row here)
  int first;    // first tile covered here: with a shared prefix of P tokens (a multiple of the block size)
                // the prefix pass takes keys 0 .. min(P, nvis) - 1, so the row's tiles start at P / 16,
                // or there are none when the prefix covers the whole context
  int nt;       // tiles per segment
  int t;        // query row
};

__device__ __forceinline__ ItemLens item_lens(const AttnArgs& a, int item) {
  const bool mixed = a.mode == kMixedDecodeSeqs;
  const bool has_prefix = a.item_prefix != nullptr;
  // each input through a pointer chosen by the mode (a select, not a branch), loaded unconditionally
  const int32_t* q0p = mixed ? a.query_start_loc + item : a.context_lens + item;
  const int32_t* q1p = mixed ? a.query_start_loc + item + 1 : a.context_lens + item;
  const int32_t* pp = has_prefix ? a.item_prefix + item : a.context_lens + item;
  const int ctx = a.context_lens[item];
  const int q0 = *q0p, q1 = *q1p, pre = *pp;
  ItemLens r;
  r.decode = !mixed || (q1 - q0 == 1 && q0 >= 0 && q0 < a.num_tokens);
  r.pre = has_prefix ? max(pre, 0) : 0;
  r.nvis = r.decode ? min(max(ctx, 0), a.max_blocks * a.block_size) : 0;
  const int tiles = ceil_div(r.nvis, kTileTokens);
  r.first = a.item_prefix == nullptr ? 0 : r.pre >= r.nvis ? tiles : r.pre / kTileTokens;
  r.nt = tiles - r.first;
  r.t = mixed ? q0 : item;
  return r;
}

// Scalar cursor over items in the global tile order.
struct Cursor {
  int item;
  int64_t start;  // global index of the item's first tile
  int nt;         // tiles per segment of the item
  int first;      // the item's first tile in its context (past a shared prefix)
  int nvis, t;
};

__device__ __forceinline__ void cursor_load(const AttnArgs& a, Cursor& c) {
  const ItemLens l = item_lens(a, c.item);
  c.nvis = l.nvis;
  c.first = l.first;
  c.nt = l.nt;
  c.t = l.t;
}

__device__ __forceinline__ void cursor_next(const AttnArgs& a, Cursor& c, int segs) {
  c.start += (int64_t)c.nt * segs;
  do {
    ++c.item;
    if (c.item >= a.num_items) {
      c.nt = 0;
      return;
    }
    cursor_load(a, c);
  } while (c.nt == 0);
}

// One descriptor per lane: lane i describes tile gbase + i of the global sequence.
struct Window {
  int row;    // pool row of the tile's first token: block * block_size + slot (token-major layout), or
              // (block * num_kv_heads + kv head) * block_size + slot (head-major)
  int kvh;    // kv head
  int h0;     // first query head of the segment
  int t;      // query row
  int item;   // decode item (request) of the tile
  int flags;  // visible tokens | kFlagFirst | kFlagLast | kFlagPrefix | kFlagPartFirst |
              // (tile index in its segment << kTileShift)
};

// Fills `w` for global tiles [gbase, gbase + count); `c` is at the item holding gbase on entry and at
// the item holding gbase + count - 1 on return.
template <int GW, bool kParts>
__device__ __forceinline__ void build_window(const AttnArgs& a, Cursor& c, int64_t gbase, int count, int lane, int segs,
                                             Window& w) {
  w.row = 0;
  w.kvh = 0;
  w.h0 = 0;
  w.t = 0;
  w.item = 0;
  w.flags = 0;
  const int64_t g = gbase + lane;
  while (c.nt > 0) {
    const int64_t item_end = c.start + (int64_t)c.nt * segs;
    if (lane < count && g >= c.start && g < item_end) {
      const int off = (int)(g - c.start);
      const int seg = off / c.nt;
      const int tile = off - seg * c.nt;
      const int kvh = seg / a.subgroups;
      const int sub = seg - kvh * a.subgroups;
      const int tok = (c.first + tile) * kTileTokens;
      const int blk = clamp_block(a.block_tables[(int64_t)c.item * a.max_blocks + tok / a.block_size], a.num_blocks);
      w.row = (a.head_major ? blk * a.num_kv_heads + kvh : blk) * a.block_size + tok % a.block_size;
      w.kvh = kvh;
      w.h0 = kvh * a.group + sub * GW;
      w.t = c.t;
      w.item = c.item;
      w.flags = min(kTileTokens, c.nvis - tok) | (tile == 0 ? kFlagFirst : 0) | (tile == c.nt - 1 ? kFlagLast : 0) |
                (c.first > 0 ? kFlagPrefix : 0) | (tile << kTileShift);
      if constexpr (kParts) {  // partitions are fixed by absolute key position (tile c.first + tile of the context)
        w.flags |= (c.first + tile) % a.bal_part_tiles == 0 ? kFlagPartFirst : 0;
      }
    }
    if (item_end >= gbase + count) break;
    cursor_next(a, c, segs);
  }
}

__device__ __forceinline__ int rd(int v, int lane_idx) { return __builtin_amdgcn_readlane(v, lane_idx); }

// Makes the loads of `v` complete here. Used on the rare piece-start path so that the per-tile path
// never carries a pending query load (which would make every tile wait for the K/V prefetch too).
template <int NQ>
__device__ __forceinline__ void settle(uint4 (&v)[NQ]) {
#pragma unroll
  for (int g = 0; g < NQ; ++g) asm volatile("" : "+v"(v[g].x), "+v"(v[g].y), "+v"(v[g].z), "+v"(v[g].w));
}
// The same for loaded floats: keeps the compiler from sinking their loads into the branches that use them
// (which would wait for each load in turn instead of having them all in flight together).
template <int N>
__device__ __forceinline__ void settle(float (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]));
}

// kMfma: the tile arithmetic runs on the matrix cores (MfmaDecodeState, bf16), with K staged in LDS
// like V when streaming (one wave per SIMD leaves LDS to spare; measured 7% faster on the long-context
// 8-head groups) and held in registers when blocks are shared (two waves per SIMD: LDS would limit
// occupancy); otherwise on the vector ALUs (DecodeState).
// kParts: the batch is cut into caller-set context partitions (a.bal_part_tiles > 0); a separate instance, so
// that the bookkeeping of partitions adds no registers to the kernels without them.
template <typename T, int D, int GW, int DEPTH, bool kPrefetchQ, bool kStream, bool kMfma, bool kParts>
__global__ __launch_bounds__(64) void decode_balanced_kernel(AttnArgs a) {
  using State = std::conditional_t<kMfma, MfmaDecodeState<D, GW, DEPTH, kStream>, DecodeState<T, D, GW>>;
  constexpr int NQ = State::kQRegs;
  __shared__ typename State::Shared sh;

  State st;
  st.init(threadIdx.x);
  const int lane = threadIdx.x;
  const int segs = a.num_kv_heads * a.subgroups;

  // The slices are cut in cost units rather than tiles: a segment costs its tiles plus kPieceCost, the
  // tile-equivalent of starting a piece (storing the previous one, whose stores the next loads' waits then
  // also cover, reloading the query, restarting the softmax), so a wave that holds many short segments takes
  // fewer tiles and the waves finish together. A tile at index t of segment k of an item starts at cost
  // k * (nt + kPieceCost) + kPieceCost + t within the item; wave w takes the tiles whose start lies in
  // [w * TC / N, (w + 1) * TC / N). On the vector path a piece start measured 1.7-1.8 tiles (per-tile
  // timestamps on the 64-request batch) and a charge of 2 took the kernel from 93.7 to 90.3 us (3 was
  // slower); on the matrix cores, where segment starts are often cached prefix tiles, a charge made the
  // prefix-shared batch slower, so there the slices are plain equal tile counts.
  constexpr int kPieceCost = kMfma ? 0 : 2;
  const int64_t N = a.num_waves, wid = blockIdx.x;
  const auto seg_cost = [](int nt) { return nt > 0 ? nt + kPieceCost : 0; };
  // lengths of the first 64 items, kept for the searches of the slice bounds below
  const ItemLens none{false, 0, 0, 0, 0, 0};
  const ItemLens lens_first = lane < a.num_items ? item_lens(a, lane) : none;
  const int incl_first = wave_inclusive_scan(lens_first.nt, lane);
  const int inclc_first = wave_inclusive_scan(seg_cost(lens_first.nt), lane);
  int64_t total = (int64_t)rd(inclc_first, 63) * segs;  // total cost
  for (int c0 = 64; c0 < a.num_items; c0 += 64) {
    const int item = c0 + lane;
    total += (int64_t)wave_sum_int(item < a.num_items ? seg_cost(item_lens(a, item).nt) : 0) * segs;
  }
  // the shuffle reduction leaves `total` equal in every lane; make that visible to the compiler so
  // that the slice bounds and the tile loop are scalar (uniform) control flow
  total = ((int64_t)__builtin_amdgcn_readfirstlane((int)(total >> 32)) << 32) |
          (uint32_t)__builtin_amdgcn_readfirstlane((int)(total & 0xffffffff));

  // Global index of the first tile whose cost start is at or after P (the total tile count when none is);
  // with `c` set, also the cursor at the item holding that tile.
  Cursor cur{0, 0, 0, 0, 0, 0};
  auto locate = [&](int64_t P, Cursor* c) -> int64_t {
    int64_t base_cost = 0, base_tiles = 0;
    for (int c0 = 0; c0 < a.num_items; c0 += 64) {
      const int item = c0 + lane;
      const ItemLens lens = c0 == 0 ? lens_first : item < a.num_items ? item_lens(a, item) : none;
      const int incl = c0 == 0 ? incl_first : wave_inclusive_scan(lens.nt, lane);
      const int inclc = c0 == 0 ? inclc_first : wave_inclusive_scan(seg_cost(lens.nt), lane);
      const int64_t chunk_cost = (int64_t)rd(inclc, 63) * segs;
      if (base_cost + chunk_cost > P) {
        const uint64_t m = __builtin_amdgcn_ballot_w64(base_cost + (int64_t)inclc * segs > P);
        const int f = (int)__builtin_ctzll(m);
        const int nt = rd(lens.nt, f);
        const int64_t start = base_tiles + (int64_t)(rd(incl, f) - nt) * segs;
        if (c) {
          c->item = c0 + f;
          c->start = start;
          c->nt = nt;
          c->first = rd(lens.first, f);
          c->nvis = rd(lens.nvis, f);
          c->t = rd(lens.t, f);
        }
        if constexpr (kPieceCost == 0) return P;  // cost and tile positions coincide
        const int64_t off = P - (base_cost + (int64_t)(rd(inclc, f) - (nt + kPieceCost)) * segs);
        const int64_t k = off / (nt + kPieceCost);
        const int64_t r = off - k * (nt + kPieceCost);
        return start + k * nt + (r > kPieceCost ? r - kPieceCost : 0);
      }
      base_cost += chunk_cost;
      base_tiles += (int64_t)rd(incl, 63) * segs;
    }
    return base_tiles;
  };
  const int64_t g1 = kPieceCost == 0 ? (wid + 1) * total / N : locate((wid + 1) * total / N, nullptr);
  const int64_t g0 = locate(wid * total / N, &cur);  // cursor at the item holding tile g0
  if (g0 >= g1) {
    // An empty slice (the batch has fewer tiles than waves) can lie between the first and the last
    // piece of a segment: its slot 0 holds a neutral partial (no weight, zero values) for the merge.
    const int64_t slot = wid * 2;
    if (lane < 2 * GW) a.part_ml[slot * GW * 2 + lane] = (lane & 1) ? 0.0f : kNegInf;
    for (int e = lane; e < GW * D; e += 64) a.part_o[slot * GW * D + e] = 0.0f;
    return;
  }
  const int n = (int)(g1 - g0);

  Window wa, wb;
  build_window<GW, kParts>(a, cur, g0, min(n, kWindowTiles), lane, segs, wa);
  if (n > kWindowTiles) build_window<GW, kParts>(a, cur, g0 + kWindowTiles, min(n - kWindowTiles, kWindowTiles), lane, segs, wb);
  int ja = 0;  // relative index of wa's first tile

  const int64_t slot_stride = a.slot_stride;  // elements between a kv head's rows of consecutive slots
  const T* kc = static_cast<const T*>(a.k_cache);
  const T* vc = static_cast<const T*>(a.v_cache);
  // loads of relative tile j into ring slot d
  auto issue = [&](int j, typename State::Tile& t, int d) {
    const int l = j - ja;
    const int row = l < kWindowTiles ? rd(wa.row, l) : rd(wb.row, l - kWindowTiles);
    const int kvh = l < kWindowTiles ? rd(wa.kvh, l) : rd(wb.kvh, l - kWindowTiles);
    const int64_t base = a.head_major ? (int64_t)row * D : ((int64_t)row * a.num_kv_heads + kvh) * D;
    st.template issue<kStream>(kc, vc, base, slot_stride, t, d, sh);
  };

  const T* qbase = static_cast<const T*>(a.q);
  auto load_q = [&](int t, int h0, uint4 (&qv)[NQ]) {
    st.load_q(qbase + ((int64_t)t * a.num_q_heads + h0) * D, a.scale_log2, qv);
  };
  // Next piece start after relative tile j (n if none): a segment's first tile inside the windows.
  auto next_piece = [&](int j) -> int {
    const int l = j - ja;
    uint64_t m = __builtin_amdgcn_ballot_w64((wa.flags & kFlagFirst) != 0 && lane > l);
    if (m != 0) return ja + (int)__builtin_ctzll(m);
    if (n > ja + kWindowTiles) {
      m = __builtin_amdgcn_ballot_w64((wb.flags & kFlagFirst) != 0 && lane + kWindowTiles > l);
      if (m != 0) return ja + kWindowTiles + (int)__builtin_ctzll(m);
    }
    return n;
  };
  auto prefetch_q = [&](int j, uint4 (&qv)[NQ]) {
    const int ln = j - ja;
    const int t = ln < kWindowTiles ? rd(wa.t, ln) : rd(wb.t, ln - kWindowTiles);
    const int h0 = ln < kWindowTiles ? rd(wa.h0, ln) : rd(wb.h0, ln - kWindowTiles);
    load_q(t, h0, qv);
  };

  // The first query is issued before the first tiles (its address needs no table entry, so it is in
  // flight while the table loads of the windows complete) and settled after them: the start of the
  // slice waits for one round trip of K/V, not for a query round trip followed by a K/V round trip.
  uint4 q_cur[NQ], q_next[kPrefetchQ ? NQ : 1];
  load_q(rd(wa.t, 0), rd(wa.h0, 0), q_cur);

  // Every iteration issues the same loads (past the end of the slice the index is clamped to the
  // last tile, an L2 hit), so the per-tile wait counts never have to cover a path without them.
  typename State::Tile ring[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) issue(min(d, n - 1), ring[d], d);
  settle<NQ>(q_cur);
  int q_next_j = n;
  if constexpr (kPrefetchQ) {
    q_next_j = next_piece(0);
    if (q_next_j < n) prefetch_q(q_next_j, q_next);
  }

  st.reset();
  if constexpr (kParts) st.reset_parts();
  int piece_start_j = 0;
  int piece_first_tile = rd(wa.flags, 0) >> kTileShift;  // tile index (in its segment) where the piece starts
  T* out = static_cast<T*>(a.out);
  const int groups_per_row = a.num_q_heads / GW;

  for (int jb = 0; jb < n; jb += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int j = jb + d;
      if (j < n) {
        if (j == ja + kWindowTiles) {  // slide the descriptor windows
          wa = wb;
          ja += kWindowTiles;
          if (n > ja + kWindowTiles)
            build_window<GW, kParts>(a, cur, g0 + ja + kWindowTiles, min(n - ja - kWindowTiles, kWindowTiles), lane, segs, wb);
        }
        const int l = j - ja;
        const int flags = rd(wa.flags, l);
        if (j > 0 && (flags & kFlagFirst)) {  // a new segment starts: new piece
          if constexpr (kPrefetchQ) {
            if (j == q_next_j) {
#pragma unroll
              for (int g = 0; g < NQ; ++g) q_cur[g] = q_next[g];
            } else {
              load_q(rd(wa.t, l), rd(wa.h0, l), q_cur);
            }
            settle<NQ>(q_cur);
            q_next_j = next_piece(j);
            if (q_next_j < n) prefetch_q(q_next_j, q_next);
          } else {
            load_q(rd(wa.t, l), rd(wa.h0, l), q_cur);
            settle<NQ>(q_cur);
          }
          st.reset();
          if constexpr (kParts) st.reset_parts();
          piece_start_j = j;
          piece_first_tile = 0;
        } else if (kParts && j > 0 && (flags & kFlagPartFirst)) {
          // a context partition starts inside the piece: the one that ended joins the kept partitions, and
          // the softmax restarts for the new one
          st.template fold_parts<false>(sh);
          st.reset();
        }
        st.tile(q_cur, ring[d], d, flags & kValidMask, a.scale_log2, sh);
        issue(min(j + DEPTH, n - 1), ring[d], d);
        const bool piece_end = (flags & kFlagLast) || j == n - 1;
        if (piece_end) {
          if constexpr (kParts) st.template fold_parts<true>(sh);  // the piece's partitions, folded
          st.finish(sh);
          // read the descriptor in uniform control flow: a lane read inside the lane-0 branch below may
          // see a register the compiler considers dead in the other lanes
          const int t = rd(wa.t, l);
          const int h0 = rd(wa.h0, l);
          const int item = rd(wa.item, l);
          T* orow = out + ((int64_t)t * a.num_q_heads + h0) * D;
          const bool seg_end = (flags & kFlagLast) != 0;
          const int64_t rec_index = (int64_t)item * groups_per_row + h0 / GW;
          // the piece record read by the merge: the first piece's partial slot and the last piece's wave
          if (lane == 0) {
            int32_t* rec = a.seg_piece + 2 * rec_index;
            if (piece_first_tile == 0) rec[0] = (int)(wid * 2 + (piece_start_j == 0 ? 0 : 1));
            if (seg_end) rec[1] = (int)wid;
          }
          if (piece_first_tile == 0 && seg_end && (flags & kFlagPrefix)) {
            // a whole segment of a request with a shared prefix: its partial meets the prefix's in the merge
            const int64_t slot = (int64_t)t * a.num_q_heads + h0;
            st.store_partial(a.seg_o + slot * D, D, a.seg_ml + slot * 2, 2, sh);
          } else if (piece_first_tile == 0 && seg_end) {
            st.store_output(orow, sh);
          } else {
            const int64_t slot = wid * 2 + (piece_start_j == 0 ? 0 : 1);
            st.store_partial(a.part_o + slot * GW * D, D, a.part_ml + slot * GW * 2, 2, sh);
          }
        }
      }
    }
  }
  st.drain();
}


// What a merge wave needs to know about its request: item_lens (as the decode kernel saw them) and the
// segment's piece record, loaded together and waited for at once, since a load behind an early return
// cannot be moved ahead of it.
struct MergeItem {
  bool decode;  // a decode row of this batch
  bool prefix;  // shared-prefix partials come first
  int npre;     // the row's prefix partitions (those it sees keys of)
  int t;        // query row
  int nvis, nt;
  int wf_slot;  // partial slot of the segment's first piece
  int wf, wl;   // waves holding the first and the last piece
};

__device__ __forceinline__ MergeItem merge_item(const AttnArgs& a, int item, int group_index) {
  const int32_t* rec = a.seg_piece + 2 * (int64_t)group_index;
  const int rec_first = rec[0], rec_last = rec[1];
  const ItemLens l = item_lens(a, item);
  // (the kernel arguments read after the early returns are loaded here too, not one by one behind them)
  asm volatile("" ::"s"(l.nvis), "s"(l.nt), "s"(l.t), "s"(l.pre), "s"(rec_first), "s"(rec_last), "s"(a.out),
               "s"(a.num_waves), "s"(a.part_o), "s"(a.part_ml));
  MergeItem m;
  m.t = l.t;
  m.decode = l.decode && l.t >= 0 && l.t < a.num_tokens;
  m.nvis = l.nvis;
  m.nt = l.nt;
  m.prefix = l.pre > 0;
  m.npre = m.prefix ? ceil_div(min(l.pre, l.nvis), a.prefix_part_tokens) : 0;
  // the record is only read when the decode kernel wrote it (the request has tiles); kept inside the partials
  m.wf_slot = m.nt > 0 ? min(max(rec_first, 0), 2 * a.num_waves - 1) : 0;
  m.wf = m.wf_slot >> 1;
  m.wl = m.nt > 0 ? min(max(rec_last, m.wf), a.num_waves - 1) : 0;
  return m;
}

// One wave per (decode row, head group of GW query heads): combines the pieces of a segment that
// several waves shared, in wave order, and writes zeros for rows without visible keys. Segments held
// by one wave were written by it, unless the request has a shared prefix: then the prefix pass's partials
// (one per prefix partition the row sees keys of) come first, followed by the segment's partial or its pieces. The pieces after the first are their
// waves' first pieces (slot 0); an empty slice between them left a neutral partial there.
template <typename T, int D, int GW>
__global__ __launch_bounds__(64) void merge_balanced_kernel(AttnArgs a) {
  constexpr int KPL = GW * D / 64;  // output elements per lane: element e = lane*KPL + k, head e / D
  constexpr int CH = GW >= 8 ? 4 : 8;  // pieces whose loads are in flight together
  const int lane = threadIdx.x;
  const int groups_per_row = a.num_q_heads / GW;
  const int grp = blockIdx.x % groups_per_row;
  const int item = blockIdx.x / groups_per_row;
  const MergeItem it = merge_item(a, item, blockIdx.x);
  if (!it.decode) return;
  T* orow = static_cast<T*>(a.out) + ((int64_t)it.t * a.num_q_heads + grp * GW) * D;
  if (it.nvis <= 0) {
#pragma unroll
    for (int k = 0; k < KPL; ++k) orow[lane * KPL + k] = T(0);
    return;
  }
  const int wf = it.wf, wl = it.wl;
  const bool split = it.nt > 0 && wf != wl;
  if (!it.prefix && !split) return;  // one wave held the whole segment
  const int head = (lane * KPL) / D;

  float M[GW], Ls[GW], acc[KPL];
#pragma unroll
  for (int g = 0; g < GW; ++g) {
    M[g] = kNegInf;
    Ls[g] = 0.0f;
  }
#pragma unroll
  for (int k = 0; k < KPL; ++k) acc[k] = 0.0f;
  // Takes one partial's (max, sum) pairs (lane 2g and 2g + 1 of ml_lane hold head g's) into M and Ls;
  // keep / take are the factors of this lane's head for the old accumulators and the partial's outputs.
  auto weigh = [&](float ml_lane, float& keep_lane, float& take_lane) {
    keep_lane = 1.0f;
    take_lane = 0.0f;
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      const float m = __shfl(ml_lane, 2 * g), l = __shfl(ml_lane, 2 * g + 1);
      const float mn = fmaxf(M[g], m);
      const float keep = M[g] == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(M[g] - mn);
      const float take = m == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
      Ls[g] = Ls[g] * keep + l * take;
      M[g] = mn;
      if (g == head) {
        keep_lane = keep;
        take_lane = take;
      }
    }
  };
  // a partial of GW heads stored contiguously from (slot * 2, slot * D)
  auto fold_slot = [&](const float* ml, const float* o) {
    const float ml_lane = ml[lane < 2 * GW ? lane : 0];
    float po[KPL];
#pragma unroll
    for (int k = 0; k < KPL; ++k) po[k] = o[lane * KPL + k];
    float kl, tl;
    weigh(ml_lane, kl, tl);
#pragma unroll
    for (int k = 0; k < KPL; ++k) acc[k] = acc[k] * kl + po[k] * tl;
  };
  if (it.prefix) {
    const int64_t slot = (int64_t)it.t * a.num_q_heads + grp * GW;
    // the prefix partitions: head g's partial of partition p at ((slot + g) * parts + p)
    const int P = a.prefix_parts;
    const int g_ml = lane < 2 * GW ? lane >> 1 : 0;
    const int64_t head_o = (slot + (lane * KPL) / D) * P;
    const int d0 = (lane * KPL) % D;
    for (int p = 0; p < it.npre; ++p) {
      const float ml_lane = a.prefix_ml[((slot + g_ml) * P + p) * 2 + (lane & 1)];
      float po[KPL];
#pragma unroll
      for (int k = 0; k < KPL; ++k) po[k] = a.prefix_o[(head_o + p) * D + d0 + k];
      float kl, tl;
      weigh(ml_lane, kl, tl);
#pragma unroll
      for (int k = 0; k < KPL; ++k) acc[k] = acc[k] * kl + po[k] * tl;
    }
    if (it.nt > 0 && !split) fold_slot(a.seg_ml + slot * 2, a.seg_o + slot * D);
  }
  if (split) {
    for (int w0 = wf; w0 <= wl; w0 += CH) {
      float ml[CH];
      float po[CH][KPL];
      // loads of all CH pieces first; an entry past the last piece reloads the last one and is not folded
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int w = min(w0 + c, wl);
        const int64_t slot = w == wf ? it.wf_slot : (int64_t)w * 2;
        ml[c] = a.part_ml[slot * GW * 2 + (lane < 2 * GW ? lane : 0)];
        const float* src = a.part_o + slot * GW * D + lane * KPL;
#pragma unroll
        for (int k = 0; k < KPL; ++k) po[c][k] = src[k];
      }
      settle<CH>(ml);
#pragma unroll
      for (int c = 0; c < CH; ++c) settle<KPL>(po[c]);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        if (w0 + c <= wl) {
          float kl, tl;
          weigh(ml[c], kl, tl);
#pragma unroll
          for (int k = 0; k < KPL; ++k) acc[k] = acc[k] * kl + po[c][k] * tl;
        }
      }
    }
  }
  float ls_lane = Ls[0];
#pragma unroll
  for (int g = 1; g < GW; ++g)
    if (g == head) ls_lane = Ls[g];
  const float inv = 1.0f / ls_lane;
#pragma unroll
  for (int k = 0; k < KPL; ++k) {
    const float o = acc[k] * inv;
    if constexpr (sizeof(T) == 2) orow[lane * KPL + k] = __builtin_bit_cast(uint16_t, (__bf16)o);
    else orow[lane * KPL + k] = o;
  }
}

// One wave per (decode row, query head): the same combination as merge_balanced_kernel for one head, with
// the (max, sum) pairs wave-uniform and every piece's loads in flight together (up to kPieces at a time),
// so a segment split over many waves merges in one or two round trips.
template <typename T, int D, int GW>
__global__ __launch_bounds__(64) void merge_head_kernel(AttnArgs a) {
  constexpr int KPL = D / 64;      // output elements per lane
  // pieces whose loads are in flight together: the long-context segments are split over 24 waves at 1536
  // waves (24 measured 0.5 us per step faster than 16 there, 32 no faster)
  constexpr int kPieces = 24;
  const int lane = threadIdx.x;
  const int h = blockIdx.x % a.num_q_heads;
  const int item = blockIdx.x / a.num_q_heads;
  const int groups_per_row = a.num_q_heads / GW;
  const int grp = h / GW, g = h - grp * GW;
  const MergeItem it = merge_item(a, item, item * groups_per_row + grp);
  if (!it.decode) return;
  T* orow = static_cast<T*>(a.out) + ((int64_t)it.t * a.num_q_heads + h) * D + lane * KPL;
  if (it.nvis <= 0) {
#pragma unroll
    for (int k = 0; k < KPL; ++k) orow[k] = T(0);
    return;
  }
  const int wf = it.wf, wl = it.wl;
  const bool split = it.nt > 0 && wf != wl;
  if (!it.prefix && !split) return;  // one wave held the whole segment

  float M = kNegInf, L = 0.0f, acc[KPL];
#pragma unroll
  for (int k = 0; k < KPL; ++k) acc[k] = 0.0f;
  auto fold = [&](float m, float l, const float* o) {
    float po[KPL];
#pragma unroll
    for (int k = 0; k < KPL; ++k) po[k] = o[k];
    const float mn = fmaxf(M, m);
    const float keep = M == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(M - mn);
    const float take = m == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
    L = L * keep + l * take;
    M = mn;
#pragma unroll
    for (int k = 0; k < KPL; ++k) acc[k] = acc[k] * keep + po[k] * take;
  };
  if (it.prefix) {
    const int64_t slot = (int64_t)it.t * a.num_q_heads + h;
    for (int p = 0; p < it.npre; ++p) {  // the prefix partitions
      const int64_t ps = slot * a.prefix_parts + p;
      fold(a.prefix_ml[ps * 2], a.prefix_ml[ps * 2 + 1], a.prefix_o + ps * D + lane * KPL);
    }
    if (it.nt > 0 && !split) fold(a.seg_ml[slot * 2], a.seg_ml[slot * 2 + 1], a.seg_o + slot * D + lane * KPL);
  }
  if (split) {
    for (int w0 = wf; w0 <= wl; w0 += kPieces) {
      float m[kPieces], l[kPieces], po[kPieces][KPL];
      // loads of all pieces first; an entry past the last piece reloads the last one and is not folded
#pragma unroll
      for (int c = 0; c < kPieces; ++c) {
        const int w = min(w0 + c, wl);
        const int64_t slot = w == wf ? it.wf_slot : (int64_t)w * 2;
        m[c] = a.part_ml[(slot * GW + g) * 2];
        l[c] = a.part_ml[(slot * GW + g) * 2 + 1];
        const float* src = a.part_o + (slot * GW + g) * D + lane * KPL;
#pragma unroll
        for (int k = 0; k < KPL; ++k) po[c][k] = src[k];
      }
      settle<kPieces>(m);
      settle<kPieces>(l);
#pragma unroll
      for (int c = 0; c < kPieces; ++c) settle<KPL>(po[c]);
#pragma unroll
      for (int c = 0; c < kPieces; ++c) {
        // past the last piece, or an empty slice's neutral partial: nothing to fold
        if (w0 + c <= wl && m[c] != kNegInf) {
          const float mn = fmaxf(M, m[c]);
          const float keep = M == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(M - mn);
          const float take = __builtin_amdgcn_exp2f(m[c] - mn);
          L = L * keep + l[c] * take;
          M = mn;
#pragma unroll
          for (int k = 0; k < KPL; ++k) acc[k] = acc[k] * keep + po[c][k] * take;
        }
      }
    }
  }
  const float inv = 1.0f / L;
#pragma unroll
  for (int k = 0; k < KPL; ++k) {
    const float o = acc[k] * inv;
    if constexpr (sizeof(T) == 2) orow[k] = __builtin_bit_cast(uint16_t, (__bf16)o);
    else orow[k] = o;
  }
}

template <typename T, int D, int GW>
hipError_t launch_balanced_t(const AttnArgs& a, bool merge, hipStream_t s, KernelTiming tm) {
  if (a.num_waves <= 0) return hipSuccess;
  // ring slots: DEPTH - 1 tiles stay in flight while one is computed. Streaming (private blocks) runs
  // one wave per SIMD and affords a deeper ring; cached loads run two waves per SIMD.
  // Matrix cores for bf16 groups of eight heads (the vector ALUs would bound them), and for groups of four
  // when blocks are shared (cached loads); streaming groups of four are faster on the vector ALUs.
  constexpr bool kMfmaStream = sizeof(T) == 2 && GW == 8;  // as balanced_uses_mfma(1, GW, false)
  constexpr bool kMfmaCached = sizeof(T) == 2 && GW >= 4;  // as balanced_uses_mfma(1, GW, true)
  constexpr int kDepthStream = kMfmaStream ? 3 : GW >= 8 ? 2 : 3;
  constexpr int kDepthCached = kMfmaCached ? 3 : GW >= 4 ? 2 : 3;
  if (!merge) {
    const dim3 grid((unsigned)a.num_waves), block(64);
    const bool parts = a.bal_part_tiles > 0;
    if (a.cache_kv) {
      if (parts)
        hipExtLaunchKernelGGL(
            decode_balanced_kernel<T, D, GW, kDepthCached, kMfmaCached || GW <= 4, false, kMfmaCached, true>, grid,
            block, 0, s, tm.start, tm.stop, 0, a);
      else
        hipExtLaunchKernelGGL(
            decode_balanced_kernel<T, D, GW, kDepthCached, kMfmaCached || GW <= 4, false, kMfmaCached, false>, grid,
            block, 0, s, tm.start, tm.stop, 0, a);
    } else {
      if (parts)
        hipExtLaunchKernelGGL(
            decode_balanced_kernel<T, D, GW, kDepthStream, kMfmaStream || GW <= 4, true, kMfmaStream, true>, grid,
            block, 0, s, tm.start, tm.stop, 0, a);
      else
        hipExtLaunchKernelGGL(
            decode_balanced_kernel<T, D, GW, kDepthStream, kMfmaStream || GW <= 4, true, kMfmaStream, false>, grid,
            block, 0, s, tm.start, tm.stop, 0, a);
    }
  } else {
    // Eight-head groups merge one head per wave: their long segments are split over many waves (24 pieces
    // each on the 8 x 32768 batch), and per-head waves take all of a segment's pieces in one round trip
    // (measured: 182 vs 193 us per step there; for four-head groups the per-group merge is as fast or faster).
    if constexpr (GW >= 8) {
      const int64_t grid = (int64_t)a.num_items * a.num_q_heads;
      if (grid > 0) merge_head_kernel<T, D, GW><<<dim3((unsigned)grid), dim3(64), 0, s>>>(a);
    } else {
      const int64_t grid = (int64_t)a.num_items * (a.num_q_heads / GW);
      if (grid > 0) merge_balanced_kernel<T, D, GW><<<dim3((unsigned)grid), dim3(64), 0, s>>>(a);
    }
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_balanced_d(const AttnArgs& a, bool merge, hipStream_t s, KernelTiming tm) {
  switch (a.heads_per_wave) {
    case 1: return launch_balanced_t<T, D, 1>(a, merge, s, tm);
    case 2: return launch_balanced_t<T, D, 2>(a, merge, s, tm);
    case 4: return launch_balanced_t<T, D, 4>(a, merge, s, tm);
    case 8: return launch_balanced_t<T, D, 8>(a, merge, s, tm);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_balanced(const AttnArgs& a, int dtype, int head_dim, bool merge, hipStream_t s, KernelTiming tm) {
  if (dtype == 1) {
    if (head_dim == 128) return launch_balanced_d<uint16_t, 128>(a, merge, s, tm);
    if (head_dim == 64) return launch_balanced_d<uint16_t, 64>(a, merge, s, tm);
  } else {
    if (head_dim == 128) return launch_balanced_d<float, 128>(a, merge, s, tm);
    if (head_dim == 64) return launch_balanced_d<float, 64>(a, merge, s, tm);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t balanced_partial_bytes(int num_waves, int heads_per_wave, int head_dim, size_t* ml_bytes) {
  const size_t slots = (size_t)num_waves * 2 * heads_per_wave;
  *ml_bytes = (slots * 2 * sizeof(float) + 255) / 256 * 256;
  return *ml_bytes + (slots * head_dim * sizeof(float) + 255) / 256 * 256;
}

hipError_t launch_decode_balanced(const AttnArgs& a, int dtype, int head_dim, hipStream_t s, KernelTiming tm) {
  return launch_balanced(a, dtype, head_dim, false, s, tm);
}

hipError_t launch_merge_balanced(const AttnArgs& a, int dtype, int head_dim, hipStream_t s) {
  return launch_balanced(a, dtype, head_dim, true, s, KernelTiming{});
}

}  // namespace pa
