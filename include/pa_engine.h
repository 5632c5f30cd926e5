/*
 * pa_engine.h - host-side block manager and continuous-batching scheduler that
 * produce the batches the paged-attention kernels consume (C ABI).
 *
 * What it does, step by step (one call to pa_engine_step = one iteration of the
 * serving loop):
 *   1. Release: requests that finished (reached max_new_tokens, or were marked
 *      with pa_engine_finish) give back their blocks. A block returns to the free
 *      list when its reference count drops to zero.
 *   2. Resume: swapped-out requests come back first, oldest first, when their
 *      blocks fit; their host blocks are copied back into fresh GPU blocks.
 *   3. Admit: waiting requests, first come first served, while fewer than
 *      max_num_seqs requests run and the free list holds the prompt's blocks plus
 *      reserve_blocks; all prompt blocks are allocated at admission.
 *   4. Batch: every running request in its decode phase contributes its one new
 *      token; requests still in their prompt contribute a slice of at most
 *      chunk_tokens; the total stays within max_num_batched_tokens. A new token
 *      that starts a block allocates it on demand; a token written into a block
 *      that other requests share copies that block first (copy-on-write). When no
 *      block is free, the most recently admitted running request is preempted:
 *      its exclusive blocks are swapped to the host pool when it has room, else
 *      all its blocks are freed and the request recomputes its tokens later.
 *   5. Generate: a request whose cached tokens reach its known tokens produces
 *      one new token after the step.
 *   Sources: "PagedAttention memory paging and continuous batching in practice"
 *   page (bxagent.cn): the physical block manager (LIFO free list, reference
 *   counts, on-demand growth, release on completion), the continuous-batching
 *   engine (admission with a two-block reserve, per-step token append, immediate
 *   release), chunked prefill (512-token slices under a per-step token budget)
 *   and the configuration table (block size, max-num-seqs); "Continuous batching"
 *   page (guijiagi.com), section 3.2 (release, resume swapped, admit waiting,
 *   preempt) and section 3.3 (swap or recompute); "The PagedAttention mechanism
 *   in vLLM and memory optimisation practice" page (intelliparadigm.com), the
 *   preemption flow (newest request first, only exclusive blocks swapped) and
 *   the block-utilisation metric.
 *
 * The engine is host code: it touches no GPU memory. The caller executes each
 * step's block moves with pa_copy_blocks in the order swap_in, swap_out, copies
 * (a host block freed by a resume may take a swap-out of the same step; a GPU
 * block freed by a preemption may take a copy or a new token of the same step;
 * no block is both the source and the destination of the step's copies), then
 * stores the step's new K/V rows (pa_cache_write) and runs the attention
 * (pa_varlen_mixed) with the step's tables. An engine is not thread-safe; use
 * one per thread.
 */
#ifndef PA_ENGINE_H_
#define PA_ENGINE_H_

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_engine pa_engine;

typedef struct {
  int32_t num_blocks;             /* GPU pool blocks, >= 1 */
  int32_t block_size;             /* tokens per block, >= 1 */
  int32_t max_blocks_per_seq;     /* table width W: a request holds at most W blocks */
  int32_t max_num_seqs;           /* running requests, >= 1 */
  int32_t max_num_batched_tokens; /* query tokens per step, >= max_num_seqs would keep every decode running */
  int32_t chunk_tokens;           /* longest prompt slice per step, >= 1 */
  int32_t reserve_blocks;         /* free blocks admission leaves in hand, >= 0 */
  int32_t num_host_blocks;        /* host pool for swapped blocks; 0: preemption recomputes */
} pa_engine_config;

/* One step's batch. Every pointer is owned by the engine and stays valid until
 * the next pa_engine_step or pa_engine_destroy on the same engine. */
typedef struct {
  int32_t num_seqs;               /* requests in the batch */
  int32_t num_tokens;             /* query tokens = query_start_loc[num_seqs] */
  int32_t max_query_len;
  const int64_t* request_ids;     /* [num_seqs] */
  const int32_t* query_lens;      /* [num_seqs] */
  const int32_t* context_lens;    /* [num_seqs]: cached tokens once this step's are written */
  const int32_t* query_start_loc; /* [num_seqs + 1] */
  const int32_t* block_tables;    /* [num_seqs][max_blocks_per_seq], -1 past the used blocks */
  int32_t num_copies;             /* copy-on-write pairs within the GPU pool */
  const int32_t* copies;          /* [num_copies][2] (source, destination) */
  int32_t num_swap_out;           /* GPU block -> host block pairs */
  const int32_t* swap_out;        /* [num_swap_out][2] */
  int32_t num_swap_in;            /* host block -> GPU block pairs */
  const int32_t* swap_in;         /* [num_swap_in][2] */
  int32_t num_finished;           /* requests released at the start of this step */
  const int64_t* finished;        /* [num_finished] */
  int32_t num_preempted;          /* requests preempted during this step */
  const int64_t* preempted;       /* [num_preempted] */
} pa_engine_batch;

typedef struct {
  int32_t free_blocks, used_blocks, free_host_blocks;
  int32_t empty_blocks;           /* used blocks that hold no token yet (prompt blocks allocated ahead) */
  int32_t waiting, running, swapped;
  int64_t stored_tokens;          /* filled slots of the used blocks (a shared slot counts once) */
  int64_t preemptions, swaps, recomputes, copies;
} pa_engine_stats;

/* Creates an engine. Returns PA_ERR_INVALID_ARGUMENT for a field out of range. */
pa_status pa_engine_create(const pa_engine_config* config, pa_engine** engine);
void pa_engine_destroy(pa_engine* engine);

/* Queues a request with a prompt of prompt_tokens tokens that will generate
 * max_new_tokens tokens. Rejected (PA_ERR_INVALID_ARGUMENT) when the id is in
 * use, prompt_tokens < 1, max_new_tokens < 1, or the request could outgrow its
 * table (prompt_tokens + max_new_tokens > max_blocks_per_seq * block_size). */
pa_status pa_engine_submit(pa_engine* engine, int64_t request_id, int32_t prompt_tokens, int32_t max_new_tokens);

/* Starts request child_id as a branch of running request parent_id (parallel
 * sampling, beam search): the child shares every block of the parent (reference
 * counts rise) and continues from the same tokens with its own max_new_tokens.
 * The parent must be running with its prompt done, and a running slot must be
 * free. */
pa_status pa_engine_fork(pa_engine* engine, int64_t parent_id, int64_t child_id, int32_t max_new_tokens);

/* Marks a request finished (end of sequence); it is released at the next step. */
pa_status pa_engine_finish(pa_engine* engine, int64_t request_id);

/* Schedules one step and describes it in *batch. */
pa_status pa_engine_step(pa_engine* engine, pa_engine_batch* batch);

pa_status pa_engine_get_stats(const pa_engine* engine, pa_engine_stats* stats);

#ifdef __cplusplus
}
#endif

#endif /* PA_ENGINE_H_ */
