/*
 * pa.h - paged attention on AMD Instinct MI355X (gfx950): the C ABI.
 *
 * Operation (all entry points). Keys and values of every request live in a
 * pool of fixed-size physical blocks; a request's block table maps its logical
 * block b (tokens b*block_size .. b*block_size + block_size - 1) to a physical
 * block anywhere in the pool. For each query token and query head the library
 * reads K through the table, forms scaled scores q.k * scale, takes a
 * numerically stable softmax over the keys the token may see, and writes the
 * softmax-weighted sum of V. Nothing is copied into contiguous memory.
 *   Sources: "Continuous batching: a paradigm shift in inference throughput"
 *   (guijiagi.com), section 2.2 (block table, 16-token blocks) and section 4.1
 *   (the PagedAttention kernel: per-block addressing through the table,
 *   scaled dot product, softmax, weighted sum of V, normalisation);
 *   "PagedAttention memory paging and continuous batching in practice"
 *   (bxagent.cn), the PagedAttention mechanism section (logical vs physical
 *   blocks, on-demand allocation, custom kernel with on-chip tiling, zero copy)
 *   and the chunked-prefill section (prefill slices mixed with decodes).
 *
 * Layouts (row-major, element type = params.dtype unless stated):
 *   q, out          [num_tokens][num_q_heads][head_dim]
 *   k_cache,v_cache [num_blocks][block_size][num_kv_heads][head_dim] (PA_LAYOUT_TOKEN_MAJOR), or
 *                   [num_blocks][num_kv_heads][block_size][head_dim] (PA_LAYOUT_HEAD_MAJOR)
 *   block_tables    int32 [num_seqs][max_blocks_per_seq]
 *   context_lens    int32 [num_seqs]   cached tokens of the request, counting
 *                                      this step's own tokens (already written)
 *   query_start_loc int32 [num_seqs+1] query rows of request s are
 *                                      query_start_loc[s] .. query_start_loc[s+1]-1
 * Query head h reads kv head h / (num_q_heads / num_kv_heads).
 * Row j of a request with q_len query rows sees keys 0 .. ctx - q_len + j
 * (causal, aligned to the end of the context); decode is q_len = 1.
 *
 * Ownership and execution: every pointer is caller-owned device memory except
 * `params` and the host-side checker's arguments (host memory). The library
 * allocates no device memory at run time (the static scratch of
 * pa_decode_noalloc is part of its code, loaded with it) and keeps no per-call
 * state. Calls enqueue kernels on
 * `stream` (a hipStream_t; NULL = the default stream) and return without
 * synchronising; buffers must stay alive until the stream passes the call.
 * `out` is fully overwritten. Calls are thread-safe; two calls that share a
 * workspace must not overlap on the device.
 *
 * Workspace: device memory of at least the *_workspace_size bytes, owned by
 * the caller, with no required contents; the library overwrites what it uses.
 *
 * Errors: a status code is returned and nothing throws. Only host scalars and
 * pointers are validated (before any HIP call). Device-data preconditions
 * (0 <= block ids < num_blocks for every block a request uses,
 * 1 <= context_lens[s] <= max_blocks_per_seq * block_size, query_start_loc
 * non-decreasing from 0 to num_tokens, q_len <= context_len) are the caller's;
 * pa_check_inputs_host verifies them on host copies; for pa_varlen_mixed also
 * q_len <= max_query_len for every request (rows of a longer slice are not
 * computed and their rows of `out` keep what they held). Kernels clamp block ids
 * and lengths into range so that bad device data never reads outside the
 * buffers; the output for such rows is then unspecified.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pa_status;
enum {
  PA_OK = 0,
  PA_ERR_NULL_POINTER = 1,       /* a required pointer is NULL */
  PA_ERR_INVALID_ARGUMENT = 2,   /* a scalar is out of its documented range */
  PA_ERR_UNSUPPORTED = 3,        /* a valid shape this build has no kernel for */
  PA_ERR_WORKSPACE_TOO_SMALL = 4,/* workspace_bytes < the *_workspace_size value */
  PA_ERR_HIP = 5                 /* a HIP launch failed; see pa_last_error_detail */
};

enum { PA_DTYPE_FP32 = 0, PA_DTYPE_BF16 = 1 };

/* pa_params.layout: how a physical block of the caches holds its tokens' rows. */
enum {
  /* [block][slot][kv head][head_dim]: a token's rows of every KV head together, the indexing of the kernel in
     section 4.1 of the "Continuous batching" page (block base + slot * row + head offset). */
  PA_LAYOUT_TOKEN_MAJOR = 0,
  /* [block][kv head][slot][head_dim]: each KV head's part of a block contiguous, as a block is described in
     section 1.1 of "The PagedAttention mechanism in vLLM and memory optimisation practice" (a contiguous
     region within one attention head). A 16-token tile of one KV head is then one contiguous run of bytes. */
  PA_LAYOUT_HEAD_MAJOR = 1
};

/* Bits of pa_params.flags. */
enum {
  /* Requests of the batch share physical blocks (a common prefix, copy-on-write beam branches, as
     in the prefix-sharing section of the "Continuous batching" page). K and V are then read with
     ordinary cached loads, and the decode work is spread over more waves, so a block that several
     requests use is served from the GPU caches after its first read. Without the flag K and V are
     read with streaming (non-temporal) loads, which move a batch of private blocks faster but give
     the caches no reuse. Both give the attention within the same error bounds; the work split, and
     so the rounding of the log-sum-exp merge, may differ between the two. */
  PA_FLAG_SHARED_BLOCKS = 1
};

typedef struct {
  int32_t num_q_heads;        /* Hq >= 1, a multiple of num_kv_heads */
  int32_t num_kv_heads;       /* Hkv >= 1 */
  int32_t head_dim;           /* D: 64 or 128 */
  int32_t block_size;         /* tokens per physical block, >= 1 (16 and 32 take the fast path) */
  int32_t num_blocks;         /* blocks in the pool (rows of k_cache / v_cache), >= 1 */
  int32_t max_blocks_per_seq; /* W: row stride of block_tables, >= 1 */
  int32_t dtype;              /* PA_DTYPE_FP32 or PA_DTYPE_BF16; q, caches and out share it */
  float scale;                /* score scale, used as given (typically 1/sqrt(head_dim)); finite */
  int32_t partition_tokens;   /* keys per context partition: 0 = automatic, else a multiple of 16
                                 in [16, 1024]. Decode rows with block_size a multiple of 16 take
                                 the balanced split (16-token tiles spread evenly over a fixed wave
                                 count): with 0 a row's keys are cut only where the waves' slices
                                 meet; with a set value the softmax also restarts at each
                                 multiple of partition_tokens (absolute key position), so each
                                 partition has its own (max, sum, weighted values), and a row's
                                 partitions are merged by log-sum-exp (in registers for those one
                                 wave holds, by the merge kernel across waves). bf16 chunk rows on the
                                 matrix cores: 0 = one row tile covers all its keys, else partitions
                                 merged the same way. Rows on the partition kernel (other block
                                 sizes and shapes): 0 = 512. Any value gives the same result in exact
                                 arithmetic; only the rounding differs. */
  int32_t flags;              /* 0 or PA_FLAG_SHARED_BLOCKS; other bits are invalid */
  int32_t layout;             /* PA_LAYOUT_TOKEN_MAJOR (0) or PA_LAYOUT_HEAD_MAJOR; every entry point that
                                 takes the caches honours it (the block copy moves whole blocks in either) */
} pa_params;

/*
 * An auxiliary stream and two events (hipStream_t, hipEvent_t, created by the
 * caller on the device of the call's stream; the events only order the two
 * streams, so they may have timing and the system-scope fence disabled, as the
 * library's own have: hipEventDisableTiming | hipEventDisableSystemFence) for
 * the *_ex entry points. The call records `fork_event` on its
 * stream, makes `stream` wait for it, runs its second branch there, records
 * `join_event` on `stream` and makes its own stream wait for that; with these
 * the library keeps no state of its own for the call. Calls that share one
 * pa_aux must be ordered (one stream, or synchronised), like calls that share
 * a workspace.
 */
typedef struct {
  void* stream;
  void* fork_event;
  void* join_event;
} pa_aux;

/*
 * Bytes of device workspace pa_decode needs for num_seqs requests. It is 0 only
 * when no request can span more than one context partition (max_blocks_per_seq
 * * block_size <= partition_tokens, 0 meaning 512) and the batch runs one wave
 * per context: block_size not a multiple of 16, or contexts of at most 64
 * tokens, or num_seqs * num_kv_heads * (heads per KV head / heads per wave) of
 * at least 4096 waves; the workspace pointer may then be NULL. Returns 0 for
 * invalid parameters as well; pa_decode reports them.
 */
size_t pa_decode_workspace_size(const pa_params* params, int32_t num_seqs);

/*
 * Decode step: one query token per request (num_tokens = num_seqs, query row s
 * belongs to request s); row s sees context_lens[s] keys. The batch's work
 * (request, kv head, 16-token tile) is cut into contiguous slices of equal
 * cost (tiles, plus a fixed charge per segment start on the vector path), one
 * per wave;
 * a request split between waves is merged by the log-sum-exp of its pieces,
 * which equals the single-pass softmax in exact arithmetic. For bf16 with
 * eight query heads per KV head (and with four under PA_FLAG_SHARED_BLOCKS)
 * each tile's scores and weighted values are computed on the matrix cores;
 * otherwise on the vector ALUs. A set partition_tokens also restarts the softmax at
 * each multiple of partition_tokens keys and merges the partitions by log-sum-exp;
 * block sizes that are not a multiple of 16 always use context partitions (of
 * partition_tokens keys, 0 meaning 512) merged the same way. A batch whose
 * contexts fit one partition runs one wave per (request, kv head, head group)
 * with no merge when the contexts are at most 64 tokens or those waves number
 * at least 4096 (the cases where that beats the equal-cost cut).
 *   Source: "Continuous batching" page, section 4.1 (kernel over a request's
 *   blocks; per-block partial products whose softmax results are merged).
 * num_seqs == 0 is a successful no-op.
 */
pa_status pa_decode(const pa_params* params, int32_t num_seqs, void* out, const void* q,
                    const void* k_cache, const void* v_cache, const int32_t* block_tables,
                    const int32_t* context_lens, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * pa_decode without a workspace argument, for callers that cannot allocate device memory around the call:
 * code under HIP graph capture, tight serving loops, harnesses that forbid allocation. The same kernels as
 * pa_decode, on the same arguments, give the same bits; their scratch memory (partials and piece records)
 * is a static array of the library, 32 MiB (33554432 bytes) per GPU, created when the library's code is
 * loaded on that GPU and held until the process ends. The call allocates nothing: no hipMalloc, hipFree or
 * allocating library routine.
 * Every call on one GPU shares that GPU's array, which keeps the last call's contents (the kernels need none
 * and overwrite what they use): calls that overlap on one GPU (two streams, two threads, two processes'
 * contexts aside) race and give unspecified output; order them on one stream. The stream (NULL = the default
 * stream) must belong to the current device, else PA_ERR_INVALID_ARGUMENT. A batch whose
 * pa_decode_workspace_size exceeds 32 MiB is rejected with PA_ERR_WORKSPACE_TOO_SMALL before any device
 * work (pa_decode with a caller workspace serves it). Other errors as pa_decode.
 */
pa_status pa_decode_noalloc(const pa_params* params, int32_t num_seqs, void* out, const void* q,
                            const void* k_cache, const void* v_cache, const int32_t* block_tables,
                            const int32_t* context_lens, void* stream);

/*
 * Bytes of device workspace pa_varlen_mixed needs (always > 0 for
 * num_tokens > 0: it also holds the device work list).
 */
size_t pa_varlen_mixed_workspace_size(const pa_params* params, int32_t num_seqs,
                                      int32_t num_tokens, int32_t max_query_len);

/*
 * One continuous-batching step over variable-length requests: decodes
 * (q_len = 1) and chunked-prefill slices (q_len > 1, causal inside the slice)
 * in any order. num_tokens = query_start_loc[num_seqs]; max_query_len is an
 * upper bound on every q_len (1 means pure decode). The device routes each
 * request to the decode kernels or, for bf16 slices, to the MFMA tile kernel,
 * from query_start_loc alone: there is no host synchronisation. The chunk
 * tiles and their device work list run on an auxiliary stream forked from
 * `stream` with an event and
 * joined back into it before the call's work on `stream` completes; the
 * library creates that stream and two events once per (calling thread,
 * device) and keeps them until the process ends.
 *   Source: "PagedAttention memory paging and continuous batching in
 *   practice" page, chunked-prefill section (512-token prefill slices batched
 *   with every running decode under a per-step token budget); causal
 *   alignment as stated at the top of this header.
 */
pa_status pa_varlen_mixed(const pa_params* params, int32_t num_seqs, int32_t num_tokens,
                          int32_t max_query_len, void* out, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* block_tables,
                          const int32_t* context_lens, const int32_t* query_start_loc,
                          void* workspace, size_t workspace_bytes, void* stream);
/* pa_varlen_mixed with the caller's auxiliary stream and events (aux NULL: as pa_varlen_mixed, which
   uses the library's own); a pa_aux with a NULL member is PA_ERR_NULL_POINTER. */
pa_status pa_varlen_mixed_ex(const pa_params* params, int32_t num_seqs, int32_t num_tokens,
                             int32_t max_query_len, void* out, const void* q, const void* k_cache,
                             const void* v_cache, const int32_t* block_tables,
                             const int32_t* context_lens, const int32_t* query_start_loc,
                             void* workspace, size_t workspace_bytes, void* stream, const pa_aux* aux);

/*
 * Decode with shared prefixes: the result of pa_decode, for a batch whose
 * requests come in groups that share the blocks of a common prefix (a system
 * prompt, the branches of a beam), as in the prefix-sharing section of the
 * "Continuous batching" page (section 4.2) and the copy-on-write sharing of the
 * "PagedAttention memory paging and continuous batching in practice" page.
 * Group g is the requests group_start[g] .. group_start[g+1]-1 (group_start[0]
 * = 0, non-decreasing, group_start[num_groups] = num_seqs); its requests share
 * the blocks of their first group_prefix[g] tokens (a multiple of block_size):
 * block_tables[s][b] is the same for every request s of the group and every
 * b < group_prefix[g] / block_size. group_prefix[g] = 0 marks a group without
 * sharing. The prefix keys are then read once per group: all of the group's
 * queries meet them in one pass on the matrix cores, beside the decode of each
 * request's own suffix, and the log-sum-exp merge joins the two. The prefix is
 * read through the table of the group's first request, so it is cut to that
 * request's context (in whole blocks); a later request shorter than the prefix
 * sees only its own tokens of it.
 * group_start and group_prefix are int32 device arrays. The prefix pass runs on
 * the auxiliary stream described under pa_varlen_mixed. Shapes without a
 * prefix pass (fp32, block sizes that are not a multiple of 16, GQA groups that
 * do not divide 64) run as pa_decode. A table that does not share what its group
 * declares gives unspecified output (group bounds are clamped on the device, so
 * no access leaves the arrays; pa_check_groups_host checks a description on host
 * copies). Workspace: pa_decode_shared_workspace_size bytes.
 */
size_t pa_decode_shared_workspace_size(const pa_params* params, int32_t num_seqs, int32_t num_groups);
pa_status pa_decode_shared(const pa_params* params, int32_t num_seqs, int32_t num_groups, void* out,
                           const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* context_lens,
                           const int32_t* group_start, const int32_t* group_prefix, void* workspace,
                           size_t workspace_bytes, void* stream);
/* pa_decode_shared with the caller's auxiliary stream and events (aux NULL: as pa_decode_shared, which
   uses the library's own); a pa_aux with a NULL member is PA_ERR_NULL_POINTER. */
pa_status pa_decode_shared_ex(const pa_params* params, int32_t num_seqs, int32_t num_groups, void* out,
                              const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens,
                              const int32_t* group_start, const int32_t* group_prefix, void* workspace,
                              size_t workspace_bytes, void* stream, const pa_aux* aux);

/*
 * KV-cache write: stores this step's new key and value rows in the paged cache,
 * where pa_decode / pa_varlen_mixed read them (call it first, on the same
 * stream). Token t is row j of request s (query_start_loc as for
 * pa_varlen_mixed; NULL means a decode batch, token t of request t, and then
 * num_tokens == num_seqs); its absolute position is
 * pos = context_lens[s] - q_len + j, so context_lens already counts the new
 * tokens, exactly as for the attention. Logical block pos / block_size of the
 * request is physical block block_tables[s][pos / block_size], slot
 * pos % block_size.
 *   Sources: "Continuous batching" page, section 2.2 (the block table maps a
 *   request's logical blocks to physical blocks); "PagedAttention memory
 *   paging and continuous batching in practice" page, logical and physical
 *   blocks (a new token fills the next slot of a block allocated on demand).
 * Layouts: k_new, v_new [num_tokens][num_kv_heads][head_dim] of params.dtype;
 * k_cache, v_cache as above (written). params.num_q_heads, scale,
 * partition_tokens and flags are validated but not used.
 * Only the slot rows of the new tokens are written; every other byte of the
 * caches is left as it was. A token whose position is negative or beyond
 * max_blocks_per_seq * block_size, or whose table entry is not a block of the
 * pool, is skipped. num_seqs == 0 or num_tokens == 0 is a successful no-op.
 */
pa_status pa_cache_write(const pa_params* params, int32_t num_seqs, int32_t num_tokens, void* k_cache,
                         void* v_cache, const void* k_new, const void* v_new, const int32_t* block_tables,
                         const int32_t* context_lens, const int32_t* query_start_loc, void* stream);

/*
 * Block copy: for each pair i, copies physical block mapping[2i] of the
 * source pools (keys and values) to block mapping[2i+1] of the destination
 * pools. One operation covers the two block moves of the pages:
 *   - copy-on-write: source and destination are the same pool (dst_k == src_k,
 *     dst_v == src_v); a block that several requests share is copied to a free
 *     block before one of them writes into it ("PagedAttention memory paging
 *     and continuous batching in practice" page, comparison table:
 *     copy-on-write and shared blocks for multi-branch decoding; "Continuous
 *     batching" page, section 4.2, prefix sharing);
 *   - swap: one pool is GPU memory and the other pinned host memory;
 *     preemption moves a request's blocks to the host and resumption brings
 *     them back, block by block, on a stream of the caller's choice (a copy
 *     stream beside the compute stream) ("Continuous batching" page, section
 *     3.3, preemption by swapping; "The PagedAttention mechanism in vLLM and
 *     memory optimisation practice" page, section 2.1, block-granular swap on
 *     dedicated copy streams).
 * The copy is one kernel; it reads and writes pinned host memory directly
 * across the host link, so a scattered block list costs one launch.
 * Layouts: every pool is n blocks of block_size x num_kv_heads x head_dim
 * elements of params.dtype (either params.layout: a block moves whole),
 * n = src_num_blocks or dst_num_blocks; mapping is int32
 * [num_pairs][2] (source id, destination id). params.num_q_heads, num_blocks,
 * max_blocks_per_seq, scale, partition_tokens and flags are validated but not
 * used.
 * Memory: each pool and mapping is device memory of the current device or
 * pinned host memory (hipHostMalloc; a torch tensor made with
 * pin_memory=True), lies inside one allocation together with its whole
 * extent, and is 16-byte aligned (mapping 8-byte). Anything else (pageable
 * host memory, another device's memory, a pool that runs past its allocation)
 * is rejected with PA_ERR_INVALID_ARGUMENT before any launch.
 * Preconditions (the caller's; pa_check_copy_host checks them on a host copy
 * of mapping): destination ids are distinct, and within one pool no block is
 * both a source and a destination, so the pairs are independent and are
 * copied in parallel. A pair with an id outside its pool is skipped. Nothing
 * but the destination blocks is written. num_pairs == 0 is a successful no-op.
 */
pa_status pa_copy_blocks(const pa_params* params, int32_t num_pairs, void* dst_k, void* dst_v,
                         int32_t dst_num_blocks, const void* src_k, const void* src_v, int32_t src_num_blocks,
                         const int32_t* mapping, void* stream);

/*
 * Host-side check of pa_copy_blocks' preconditions on a HOST copy of mapping
 * (same_pool != 0 for a copy within one pool, which then has one block
 * count). Returns PA_OK, or PA_ERR_INVALID_ARGUMENT with *first_bad set to
 * the first pair whose ids leave their pool, whose destination repeats an
 * earlier destination, or whose destination is a source of the call (-1 for
 * a scalar problem). first_bad may be NULL.
 */
pa_status pa_check_copy_host(int32_t num_pairs, const int32_t* mapping, int32_t src_num_blocks,
                             int32_t dst_num_blocks, int32_t same_pool, int64_t* first_bad);

/*
 * Host-side check of the device-data preconditions on HOST copies of the
 * tables (query_start_loc may be NULL for a decode batch, num_tokens is then
 * num_seqs). max_query_len > 0 also checks q_len <= max_query_len for every
 * request (the pa_varlen_mixed argument); 0 skips that check. Returns PA_OK,
 * or PA_ERR_INVALID_ARGUMENT with *first_bad set to the index of the first
 * offending request (or -1 for a scalar problem). first_bad may be NULL.
 */
pa_status pa_check_inputs_host(const pa_params* params, int32_t num_seqs, int32_t num_tokens,
                               int32_t max_query_len, const int32_t* block_tables,
                               const int32_t* context_lens, const int32_t* query_start_loc,
                               int64_t* first_bad);

/*
 * Host-side check of pa_decode_shared's group description on HOST copies:
 * group_start runs from 0 to num_seqs without decreasing; every group_prefix
 * is a non-negative multiple of block_size; and every request of a group lists
 * the group's first request's blocks for the prefix tokens it sees (its first
 * ceil(min(prefix, ctx) / block_size) table entries). The prefix cut to the
 * first request's context (see pa_decode_shared) is what is checked. Returns
 * PA_OK, or PA_ERR_INVALID_ARGUMENT with *first_bad set to the first offending
 * group (-1 for a scalar problem). first_bad may be NULL.
 */
pa_status pa_check_groups_host(const pa_params* params, int32_t num_seqs, int32_t num_groups,
                               const int32_t* group_start, const int32_t* group_prefix,
                               const int32_t* block_tables, const int32_t* context_lens, int64_t* first_bad);

/* Static text for a status code. */
const char* pa_status_string(pa_status status);

/* Text of the last PA_ERR_HIP / argument error on the calling thread ("" if none). */
const char* pa_last_error_detail(void);

/*
 * Profiling hook: the next pa_decode, pa_decode_shared, pa_varlen_mixed,
 * pa_cache_write, pa_copy_blocks or pa_probe_stream_read (pa_probe.h) call on
 * the calling thread that launches a kernel launches
 * its dominant kernel (the decode kernel of the attention calls, the chunk
 * kernel of a pa_varlen_mixed call whose one request is a chunked-prefill
 * slice; the one kernel of the others) with `start_event` and `stop_event` attached
 * (hipExtLaunchKernel), so that they record the kernel's own start and end on
 * the call's stream (hipEvent_t handles created by the caller, with timing
 * enabled). One-shot; NULL, NULL clears it.
 */
pa_status pa_set_kernel_timing_events(void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
