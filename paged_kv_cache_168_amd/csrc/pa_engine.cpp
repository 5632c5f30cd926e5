// Host block manager and continuous-batching scheduler (C ABI in pa_engine.h).
//
// Blocks: a LIFO free list with a reference count and a fill count (filled slots) per block, as in the
// physical block manager of "PagedAttention memory paging and continuous batching in practice": an
// allocated block starts with one reference; a block returns to the free list when its last reference
// goes. Requests grow one block at a time, when a token starts a new block.
//
// Scheduling: release finished requests; resume swapped requests (they come first); admit waiting
// requests while the prompt's blocks plus a reserve are free ("Continuous batching" page, section 3.2;
// the in-practice page's engine keeps two blocks in reserve); then form the step's batch under the
// token budget, decodes first and prompt slices after (chunked prefill), growing tables on demand and
// copying a shared block before a request writes into it. When no block is free the newest running
// request that is not yet in the batch is preempted (the vLLM-mechanism page: lowest priority, usually
// the newest): with room in the host pool its exclusive blocks are swapped out (shared blocks stay on
// the GPU), otherwise it drops all its blocks and recomputes its tokens when admitted again
// ("Continuous batching" page, section 3.3).
//
// Block moves of one step must run in the order swap_in, swap_out, copies (then the cache write): a
// host block freed by a resume may receive a swap-out of the same step, and a GPU block freed by a
// preemption may be reused by a copy or a new token of the same step. A block that is the source of a
// copy in a step is never the destination of another copy of that step.
#include <algorithm>
#include <cstdint>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_engine.h"

namespace {

enum class Phase { kWaiting, kRunning, kSwapped };

struct Request {
  int64_t id = 0;
  int32_t max_new = 0;      // tokens to generate in total
  int32_t known = 0;        // tokens whose K/V the request needs: prompt + generated
  int32_t cached = 0;       // tokens whose K/V are in the cache
  int32_t generated = 0;
  int32_t prefill_end = 0;  // the request is in its prompt while cached < prefill_end
  std::vector<int32_t> table;  // GPU block of each logical block
  std::vector<int32_t> host;   // while swapped: host block of each logical block, -1 if it stayed on the GPU
  Phase phase = Phase::kWaiting;
  bool finish = false;
  bool in_batch = false;    // scheduled in the current step
  uint64_t admitted = 0;    // admission order (larger = newer)
};

struct BlockPool {
  std::vector<int32_t> free_list;  // LIFO: the last freed block is the next allocated
  std::vector<int32_t> ref, fill;

  void init(int32_t n) {
    free_list.clear();
    for (int32_t i = 0; i < n; ++i) free_list.push_back(i);
    ref.assign(n, 0);
    fill.assign(n, 0);
  }
  int32_t free_count() const { return (int32_t)free_list.size(); }
  bool alloc(int32_t* id) {
    if (free_list.empty()) return false;
    *id = free_list.back();
    free_list.pop_back();
    ref[*id] = 1;
    fill[*id] = 0;
    return true;
  }
  void release(int32_t id) {
    if (--ref[id] <= 0) {
      ref[id] = 0;
      fill[id] = 0;
      free_list.push_back(id);
    }
  }
};

int32_t blocks_for(int64_t tokens, int32_t bs) { return (int32_t)((tokens + bs - 1) / bs); }

}  // namespace

struct pa_engine {
  pa_engine_config cfg{};
  BlockPool gpu, host;
  std::unordered_map<int64_t, Request> reqs;
  std::deque<int64_t> waiting, swapped;
  std::vector<int64_t> running;  // admission order
  uint64_t next_admit = 1;
  std::vector<uint8_t> copy_src;  // GPU blocks read by a copy of the current step
  std::vector<int32_t> copy_marked;  // the blocks marked in copy_src (cleared at the next step)
  pa_engine_stats st{};
  // outputs of the last step
  std::vector<int64_t> ids, finished, preempted;
  std::vector<int32_t> qlen, ctx, qsl, tables, copies, swap_out, swap_in;

  void release(Request& r) {
    for (size_t i = 0; i < r.table.size(); ++i) {
      if (r.phase == Phase::kSwapped && r.host[i] >= 0) host.release(r.host[i]);
      else gpu.release(r.table[i]);
    }
    r.table.clear();
    r.host.clear();
  }

  // Newest running request not yet in this step's batch, other than `self` (0 if none).
  Request* victim(const Request* self) {
    Request* v = nullptr;
    for (int64_t id : running) {
      Request& c = reqs[id];
      if (&c == self || c.in_batch) continue;
      if (v == nullptr || c.admitted > v->admitted) v = &c;
    }
    return v;
  }

  void preempt(Request& v) {
    int32_t exclusive = 0;
    for (int32_t b : v.table) exclusive += gpu.ref[b] == 1;
    running.erase(std::find(running.begin(), running.end(), v.id));
    preempted.push_back(v.id);
    ++st.preemptions;
    if (cfg.num_host_blocks > 0 && host.free_count() >= exclusive) {
      v.host.assign(v.table.size(), -1);
      for (size_t i = 0; i < v.table.size(); ++i) {
        const int32_t b = v.table[i];
        if (gpu.ref[b] != 1) continue;  // shared: stays on the GPU, still referenced
        int32_t h = -1;
        host.alloc(&h);
        host.fill[h] = gpu.fill[b];
        swap_out.push_back(b);
        swap_out.push_back(h);
        gpu.release(b);
        v.host[i] = h;
      }
      v.phase = Phase::kSwapped;
      swapped.push_back(v.id);
      ++st.swaps;
    } else {
      release(v);
      v.cached = 0;
      v.prefill_end = v.known;
      v.phase = Phase::kWaiting;
      waiting.push_front(v.id);
      ++st.recomputes;
    }
  }

  // One GPU block for `r`, preempting other requests while none is free. Blocks read by a copy of this
  // step are skipped when `for_copy` (they must not be overwritten by another copy of the same step).
  // Returns false when `r` itself had to be preempted.
  bool alloc_for(Request& r, int32_t* id, bool for_copy) {
    for (;;) {
      std::vector<int32_t> held;
      bool ok = false;
      while (gpu.alloc(id)) {
        if (!(for_copy && copy_src[*id])) {
          ok = true;
          break;
        }
        held.push_back(*id);
      }
      for (auto it = held.rbegin(); it != held.rend(); ++it) {
        gpu.ref[*it] = 0;
        gpu.free_list.push_back(*it);
      }
      if (ok) return true;
      Request* v = victim(&r);
      if (v == nullptr) {
        preempt(r);
        return false;
      }
      preempt(*v);
    }
  }

  pa_status step(pa_engine_batch* out) {
    ids.clear(), finished.clear(), preempted.clear();
    qlen.clear(), ctx.clear(), qsl.assign(1, 0), tables.clear(), copies.clear(), swap_out.clear(), swap_in.clear();
    for (int32_t b : copy_marked) copy_src[b] = 0;
    copy_marked.clear();
    const int32_t BS = cfg.block_size, W = cfg.max_blocks_per_seq;

    // 1. release finished requests
    {
      std::vector<int64_t> keep;
      for (int64_t id : running) {
        Request& r = reqs[id];
        if (r.finish || r.generated >= r.max_new) {
          release(r);
          finished.push_back(id);
          reqs.erase(id);
        } else {
          keep.push_back(id);
        }
      }
      running = keep;
    }
    for (auto* q : {&waiting, &swapped}) {
      std::deque<int64_t> keep;
      for (int64_t id : *q) {
        Request& r = reqs[id];
        if (r.finish) {
          release(r);
          finished.push_back(id);
          reqs.erase(id);
        } else {
          keep.push_back(id);
        }
      }
      *q = keep;
    }

    // 2. resume swapped requests, oldest first
    while (!swapped.empty() && (int32_t)running.size() < cfg.max_num_seqs) {
      Request& r = reqs[swapped.front()];
      int32_t need = 0;
      for (int32_t h : r.host) need += h >= 0;
      if (gpu.free_count() < need + cfg.reserve_blocks) break;
      for (size_t i = 0; i < r.table.size(); ++i) {
        if (r.host[i] < 0) continue;
        int32_t b = -1;
        gpu.alloc(&b);
        gpu.fill[b] = host.fill[r.host[i]];
        swap_in.push_back(r.host[i]);
        swap_in.push_back(b);
        host.release(r.host[i]);
        r.table[i] = b;
      }
      r.host.clear();
      r.phase = Phase::kRunning;
      r.admitted = next_admit++;
      running.push_back(r.id);
      swapped.pop_front();
    }

    // 3. admit waiting requests, first come first served, once no swapped request waits
    while (swapped.empty() && !waiting.empty() && (int32_t)running.size() < cfg.max_num_seqs) {
      Request& r = reqs[waiting.front()];
      const int32_t need = blocks_for(r.known, BS);
      if (gpu.free_count() < need + cfg.reserve_blocks) break;
      for (int32_t i = 0; i < need; ++i) {
        int32_t b = -1;
        gpu.alloc(&b);
        r.table.push_back(b);
      }
      r.phase = Phase::kRunning;
      r.admitted = next_admit++;
      running.push_back(r.id);
      waiting.pop_front();
    }

    // 4. the batch: decodes first, then prompt slices, within the token budget
    for (int64_t id : running) reqs[id].in_batch = false;
    std::vector<int64_t> order;
    for (int64_t id : running)
      if (reqs[id].cached >= reqs[id].prefill_end) order.push_back(id);
    for (int64_t id : running)
      if (reqs[id].cached < reqs[id].prefill_end) order.push_back(id);
    int32_t budget = cfg.max_num_batched_tokens;
    std::vector<int64_t> batch;
    for (int64_t id : order) {
      if (budget <= 0) break;
      auto it = reqs.find(id);
      Request& r = it->second;
      if (r.phase != Phase::kRunning) continue;  // preempted earlier in this step
      const int32_t limit = r.cached < r.prefill_end ? cfg.chunk_tokens : 1;
      const int32_t q = std::min(std::min(r.known - r.cached, limit), budget);
      if (q <= 0) continue;
      bool ok = true;
      // blocks for the new positions, grown on demand
      while (ok && (int32_t)r.table.size() < blocks_for(r.cached + q, BS)) {
        int32_t b = -1;
        ok = alloc_for(r, &b, false);
        if (ok) r.table.push_back(b);
      }
      // copy-on-write: a written block that other requests share is copied first
      for (int32_t lb = r.cached / BS; ok && lb <= (r.cached + q - 1) / BS; ++lb) {
        const int32_t src = r.table[lb];
        if (gpu.ref[src] <= 1) continue;
        int32_t dst = -1;
        copy_src[src] = 1;
        copy_marked.push_back(src);
        ok = alloc_for(r, &dst, true);
        if (!ok) break;
        // the source may have been released by a preemption above; then the request holds it alone
        if (gpu.ref[src] <= 1) {
          gpu.release(dst);
          continue;
        }
        copies.push_back(src);
        copies.push_back(dst);
        gpu.fill[dst] = gpu.fill[src];
        gpu.release(src);
        r.table[lb] = dst;
        ++st.copies;
      }
      if (!ok) continue;  // r was preempted
      for (int32_t lb = r.cached / BS; lb <= (r.cached + q - 1) / BS; ++lb)
        gpu.fill[r.table[lb]] = std::max(gpu.fill[r.table[lb]], std::min(BS, r.cached + q - lb * BS));
      r.in_batch = true;
      r.cached += q;
      budget -= q;
      batch.push_back(id);
      qlen.push_back(q);
    }

    // outputs (a request preempted after it was scheduled is impossible: victims are never in the batch)
    int32_t max_q = 0;
    tables.assign(batch.size() * (size_t)W, -1);
    for (size_t i = 0; i < batch.size(); ++i) {
      Request& r = reqs[batch[i]];
      ids.push_back(r.id);
      ctx.push_back(r.cached);
      qsl.push_back(qsl.back() + qlen[i]);
      max_q = std::max(max_q, qlen[i]);
      const size_t n = std::min(r.table.size(), (size_t)W);
      std::copy(r.table.begin(), r.table.begin() + n, tables.begin() + i * (size_t)W);
    }

    // 5. a request whose cached tokens reach its known tokens produces its next token
    for (int64_t id : batch) {
      Request& r = reqs[id];
      if (r.cached == r.known) {
        ++r.known;
        ++r.generated;
      }
    }

    *out = pa_engine_batch{};
    out->num_seqs = (int32_t)batch.size();
    out->num_tokens = qsl.back();
    out->max_query_len = max_q;
    out->request_ids = ids.data();
    out->query_lens = qlen.data();
    out->context_lens = ctx.data();
    out->query_start_loc = qsl.data();
    out->block_tables = tables.data();
    out->num_copies = (int32_t)copies.size() / 2;
    out->copies = copies.data();
    out->num_swap_out = (int32_t)swap_out.size() / 2;
    out->swap_out = swap_out.data();
    out->num_swap_in = (int32_t)swap_in.size() / 2;
    out->swap_in = swap_in.data();
    out->num_finished = (int32_t)finished.size();
    out->finished = finished.data();
    out->num_preempted = (int32_t)preempted.size();
    out->preempted = preempted.data();
    return PA_OK;
  }
};

extern "C" {

pa_status pa_engine_create(const pa_engine_config* config, pa_engine** engine) {
  if (config == nullptr || engine == nullptr) return PA_ERR_NULL_POINTER;
  const pa_engine_config& c = *config;
  if (c.num_blocks < 1 || c.block_size < 1 || c.max_blocks_per_seq < 1 || c.max_num_seqs < 1 ||
      c.max_num_batched_tokens < 1 || c.chunk_tokens < 1 || c.reserve_blocks < 0 || c.num_host_blocks < 0 ||
      (int64_t)c.max_blocks_per_seq * c.block_size > INT32_MAX)
    return PA_ERR_INVALID_ARGUMENT;
  pa_engine* e = new (std::nothrow) pa_engine();
  if (e == nullptr) return PA_ERR_INVALID_ARGUMENT;
  e->cfg = c;
  e->gpu.init(c.num_blocks);
  e->host.init(c.num_host_blocks);
  e->copy_src.assign(c.num_blocks, 0);
  *engine = e;
  return PA_OK;
}

void pa_engine_destroy(pa_engine* engine) { delete engine; }

pa_status pa_engine_submit(pa_engine* e, int64_t request_id, int32_t prompt_tokens, int32_t max_new_tokens) {
  if (e == nullptr) return PA_ERR_NULL_POINTER;
  if (prompt_tokens < 1 || max_new_tokens < 1 || e->reqs.count(request_id) ||
      (int64_t)prompt_tokens + max_new_tokens > (int64_t)e->cfg.max_blocks_per_seq * e->cfg.block_size)
    return PA_ERR_INVALID_ARGUMENT;
  Request r;
  r.id = request_id;
  r.max_new = max_new_tokens;
  r.known = prompt_tokens;
  r.prefill_end = prompt_tokens;
  e->reqs.emplace(request_id, std::move(r));
  e->waiting.push_back(request_id);
  return PA_OK;
}

pa_status pa_engine_fork(pa_engine* e, int64_t parent_id, int64_t child_id, int32_t max_new_tokens) {
  if (e == nullptr) return PA_ERR_NULL_POINTER;
  auto it = e->reqs.find(parent_id);
  if (it == e->reqs.end() || e->reqs.count(child_id) || max_new_tokens < 1) return PA_ERR_INVALID_ARGUMENT;
  const Request& p = it->second;
  if (p.phase != Phase::kRunning || p.cached < p.prefill_end || p.finish ||
      (int32_t)e->running.size() >= e->cfg.max_num_seqs ||
      (int64_t)p.known + max_new_tokens > (int64_t)e->cfg.max_blocks_per_seq * e->cfg.block_size)
    return PA_ERR_INVALID_ARGUMENT;
  Request c = p;
  c.id = child_id;
  c.max_new = p.generated + max_new_tokens;
  c.admitted = e->next_admit++;
  c.in_batch = false;
  for (int32_t b : c.table) ++e->gpu.ref[b];
  e->running.push_back(child_id);
  e->reqs.emplace(child_id, std::move(c));
  return PA_OK;
}

pa_status pa_engine_finish(pa_engine* e, int64_t request_id) {
  if (e == nullptr) return PA_ERR_NULL_POINTER;
  auto it = e->reqs.find(request_id);
  if (it == e->reqs.end()) return PA_ERR_INVALID_ARGUMENT;
  it->second.finish = true;
  return PA_OK;
}

pa_status pa_engine_step(pa_engine* e, pa_engine_batch* batch) {
  if (e == nullptr || batch == nullptr) return PA_ERR_NULL_POINTER;
  return e->step(batch);
}

pa_status pa_engine_get_stats(const pa_engine* e, pa_engine_stats* s) {
  if (e == nullptr || s == nullptr) return PA_ERR_NULL_POINTER;
  *s = e->st;
  s->free_blocks = e->gpu.free_count();
  s->used_blocks = e->cfg.num_blocks - s->free_blocks;
  s->free_host_blocks = e->host.free_count();
  s->waiting = (int32_t)e->waiting.size();
  s->running = (int32_t)e->running.size();
  s->swapped = (int32_t)e->swapped.size();
  int64_t stored = 0;
  int32_t empty = 0;
  for (int32_t b = 0; b < e->cfg.num_blocks; ++b) {
    if (e->gpu.ref[b] <= 0) continue;
    stored += e->gpu.fill[b];
    empty += e->gpu.fill[b] == 0;
  }
  s->stored_tokens = stored;
  s->empty_blocks = empty;
  return PA_OK;
}

}  // extern "C"
