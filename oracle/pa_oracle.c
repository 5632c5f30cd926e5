/*
 * Paged-attention oracle: plain, slow, fp64 CPU reference.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path links, loads or calls
 * this file; only the test suite, the smoke check and the benchmark's CPU
 * baseline do. It shares no code, header or table with the HIP kernels.
 *
 * What it computes (one output row per query token t and query head h):
 *
 *   - The request of token t, its position and the number of visible keys:
 *     a query slice of q_len tokens sits at the END of the request's context
 *     of ctx cached tokens, so row j of the slice has absolute position
 *     ctx - q_len + j and sees keys 0 .. ctx - q_len + j (n = ctx - q_len + j + 1).
 *     Decode is the case q_len = 1 (n = ctx). The pages' kernel loops over
 *     kv_pos < seq_len with seq_len counting every cached token ("Continuous
 *     batching" page, section 4.1, the PagedAttention CUDA kernel); the causal
 *     alignment for a chunk follows from the chunked-prefill description
 *     ("PagedAttention + continuous batching in practice" page, section on
 *     chunked prefill): the slice's own keys are already in the cache.
 *   - The block-table dereference: logical token i lives in logical block
 *     i / block_size at slot i % block_size, and logical block b of request s
 *     is physical block block_tables[s][b] ("Continuous batching" page, section
 *     2.2 and its worked table 0->7, 1->12, 2->3, 3->19; "in practice" page,
 *     logical/physical blocks with the 48-token example). The cache layout is
 *     [num_blocks][block_size][num_kv_heads][head_dim], the indexing the
 *     section 4.1 kernel uses (block * block_size * d + slot * d + head offset).
 *   - Query head h reads kv head h / (num_q_heads / num_kv_heads).
 *   - Scores x_i = scale * (q . k_i); the output is the softmax-weighted sum of
 *     the v_i, normalised by the sum of the weights (section 4.1: scaled dot
 *     product, softmax, weighted sum of V, final normalisation). The printed
 *     kernel's running sum is not rescaled when the maximum grows, so this
 *     oracle does not follow its recurrence: it evaluates the textbook
 *     definition in two passes (maximum, then exponentials), which any correct
 *     online or split evaluation equals in exact arithmetic.
 *   - A row with n <= 0 visible keys is written as zeros.
 *
 * Inputs are read element by element and widened exactly to double
 * (fp32 -> double, bf16 -> fp32 -> double). All arithmetic is in double with
 * libm exp; each row is evaluated serially in a fixed order, so the result
 * does not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARGUMENT -1
#define ORACLE_BAD_QUERY_START_LOC -2
#define ORACLE_BAD_CONTEXT_LEN -3
#define ORACLE_BAD_BLOCK_ID -4
#define ORACLE_OUT_OF_MEMORY -5

typedef struct {
  int dtype; /* 0 = fp32, 1 = bf16 stored as raw 16-bit patterns */
  int num_seqs, num_tokens;
  int num_q_heads, num_kv_heads, head_dim;
  int block_size, num_blocks, max_blocks_per_seq;
  double scale;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start_loc; /* NULL: token s is the single query of request s */
} oracle_problem;

/* Element e of a tensor stored as fp32 or bf16, widened exactly. */
static double element(const oracle_problem* p, const void* base, int64_t e) {
  if (p->dtype == 0) return (double)((const float*)base)[e];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[e] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Request that owns query token t. */
static int request_of_token(const oracle_problem* p, int t) {
  if (p->query_start_loc == NULL) return t;
  for (int s = 0; s < p->num_seqs; ++s)
    if (p->query_start_loc[s] <= t && t < p->query_start_loc[s + 1]) return s;
  return -1;
}

/* Number of keys query token t sees (its causal horizon). */
static int visible_keys(const oracle_problem* p, int t, int s) {
  int ctx = p->context_lens[s];
  if (p->query_start_loc == NULL) return ctx;
  int q_len = p->query_start_loc[s + 1] - p->query_start_loc[s];
  int j = t - p->query_start_loc[s];
  return ctx - q_len + j + 1;
}

/* Element offset of (logical token i, kv head g) of request s in a cache. */
static int64_t kv_row_offset(const oracle_problem* p, int s, int i, int g) {
  int32_t block = p->block_tables[(int64_t)s * p->max_blocks_per_seq + i / p->block_size];
  int slot = i % p->block_size;
  return (((int64_t)block * p->block_size + slot) * p->num_kv_heads + g) * p->head_dim;
}

static int check_problem(const oracle_problem* p) {
  if (p->num_seqs < 0 || p->num_tokens < 0 || p->num_q_heads <= 0 || p->num_kv_heads <= 0 ||
      p->head_dim <= 0 || p->block_size <= 0 || p->num_blocks < 0 || p->max_blocks_per_seq < 0 ||
      p->num_q_heads % p->num_kv_heads != 0 || (p->dtype != 0 && p->dtype != 1))
    return ORACLE_BAD_ARGUMENT;
  if (p->query_start_loc == NULL) {
    if (p->num_tokens != p->num_seqs) return ORACLE_BAD_ARGUMENT;
  } else {
    if (p->query_start_loc[0] != 0 || p->query_start_loc[p->num_seqs] != p->num_tokens)
      return ORACLE_BAD_QUERY_START_LOC;
    for (int s = 0; s < p->num_seqs; ++s)
      if (p->query_start_loc[s + 1] < p->query_start_loc[s]) return ORACLE_BAD_QUERY_START_LOC;
  }
  for (int s = 0; s < p->num_seqs; ++s) {
    int ctx = p->context_lens[s];
    if (ctx < 0 || (int64_t)ctx > (int64_t)p->max_blocks_per_seq * p->block_size)
      return ORACLE_BAD_CONTEXT_LEN;
    int used_blocks = (ctx + p->block_size - 1) / p->block_size;
    for (int b = 0; b < used_blocks; ++b) {
      int32_t id = p->block_tables[(int64_t)s * p->max_blocks_per_seq + b];
      if (id < 0 || id >= p->num_blocks) return ORACLE_BAD_BLOCK_ID;
    }
  }
  return ORACLE_OK;
}

/* One output row: query token t, query head h -> out[0 .. head_dim). */
static int attention_row(const oracle_problem* p, int t, int h, double* x, double* out) {
  const int D = p->head_dim;
  const int group = p->num_q_heads / p->num_kv_heads;
  const int s = request_of_token(p, t);
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  if (s < 0) return ORACLE_BAD_QUERY_START_LOC;
  const int n = visible_keys(p, t, s);
  if (n <= 0) return ORACLE_OK;
  const int g = h / group;
  const int64_t q_off = ((int64_t)t * p->num_q_heads + h) * D;

  for (int i = 0; i < n; ++i) {
    int64_t k_off = kv_row_offset(p, s, i, g);
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += element(p, p->q, q_off + d) * element(p, p->k_cache, k_off + d);
    x[i] = p->scale * dot;
  }
  double m = x[0];
  for (int i = 1; i < n; ++i)
    if (x[i] > m) m = x[i];
  double z = 0.0;
  for (int i = 0; i < n; ++i) {
    x[i] = exp(x[i] - m);
    z += x[i];
  }
  for (int i = 0; i < n; ++i) {
    int64_t v_off = kv_row_offset(p, s, i, g);
    for (int d = 0; d < D; ++d) out[d] += x[i] * element(p, p->v_cache, v_off + d);
  }
  for (int d = 0; d < D; ++d) out[d] /= z;
  return ORACLE_OK;
}

/*
 * Computes rows[r] = t * num_q_heads + h for r < num_rows into
 * out[r * head_dim ...]; rows == NULL means every (t, h) in order
 * (out then has num_tokens * num_q_heads * head_dim doubles).
 */
int pa_oracle_attention(int dtype, int num_seqs, int num_tokens, int num_q_heads, int num_kv_heads,
                        int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                        float scale, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, const int32_t* context_lens,
                        const int32_t* query_start_loc, const int64_t* rows, int64_t num_rows,
                        double* out, int num_threads) {
  oracle_problem p = {dtype, num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, block_size,
                      num_blocks, max_blocks_per_seq, (double)scale, q, k_cache, v_cache,
                      block_tables, context_lens, query_start_loc};
  int status = check_problem(&p);
  if (status != ORACLE_OK) return status;
  const int64_t total = rows ? num_rows : (int64_t)num_tokens * num_q_heads;
  if (rows)
    for (int64_t r = 0; r < num_rows; ++r)
      if (rows[r] < 0 || rows[r] >= (int64_t)num_tokens * num_q_heads) return ORACLE_BAD_ARGUMENT;
  int max_n = 1;
  for (int s = 0; s < num_seqs; ++s)
    if (context_lens[s] > max_n) max_n = context_lens[s];
  if (num_threads < 1) num_threads = 1;
  int failed = 0;
#pragma omp parallel num_threads(num_threads)
  {
    double* x = (double*)malloc(sizeof(double) * (size_t)max_n);
    if (x == NULL) {
#pragma omp atomic write
      failed = ORACLE_OUT_OF_MEMORY;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int64_t r = 0; r < total; ++r) {
        int64_t row = rows ? rows[r] : r;
        int rs = attention_row(&p, (int)(row / num_q_heads), (int)(row % num_q_heads), x,
                               out + r * head_dim);
        if (rs != ORACLE_OK) {
#pragma omp atomic write
          failed = rs;
        }
      }
      free(x);
    }
  }
  return failed;
}

/*
 * Read map: counts[block * block_size + slot] += 1 for every (query token,
 * query head) row that reads key/value slot (block, slot), through the same
 * dereference the attention rows use.
 */
int pa_oracle_read_counts(int num_seqs, int num_tokens, int num_q_heads, int num_kv_heads,
                          int block_size, int num_blocks, int max_blocks_per_seq,
                          const int32_t* block_tables, const int32_t* context_lens,
                          const int32_t* query_start_loc, int64_t* counts) {
  oracle_problem p = {0, num_seqs, num_tokens, num_q_heads, num_kv_heads, 1, block_size,
                      num_blocks, max_blocks_per_seq, 1.0, NULL, NULL, NULL,
                      block_tables, context_lens, query_start_loc};
  int status = check_problem(&p);
  if (status != ORACLE_OK) return status;
  memset(counts, 0, sizeof(int64_t) * (size_t)num_blocks * block_size);
  for (int t = 0; t < num_tokens; ++t) {
    int s = request_of_token(&p, t);
    if (s < 0) return ORACLE_BAD_QUERY_START_LOC;
    int n = visible_keys(&p, t, s);
    for (int h = 0; h < num_q_heads; ++h)
      for (int i = 0; i < n; ++i) {
        int64_t off = kv_row_offset(&p, s, i, h / (num_q_heads / num_kv_heads));
        /* with head_dim 1, off = (block * block_size + slot) * num_kv_heads + g */
        counts[off / num_kv_heads] += 1;
      }
  }
  return ORACLE_OK;
}

/*
 * KV-cache write: store this step's new key and value rows of every token in
 * the paged cache, where the attention above will read them.
 *
 * Token t is row j of request s (request of t from query_start_loc, or s = t
 * for a decode batch when query_start_loc is NULL; q_len = 1 then). Its
 * absolute position is pos = ctx - q_len + j, with ctx = context_lens[s]
 * counting the request's cached tokens including this step's (the same
 * reading as the attention rows). Logical block pos / block_size of the
 * request is physical block block_tables[s][pos / block_size], slot
 * pos % block_size ("Continuous batching" page, section 2.2, the block table;
 * "in practice" page, logical/physical blocks: a new token goes to the slot
 * after the last filled one, in a block allocated on demand). The slot row
 * [num_kv_heads][head_dim] of k_new[t] and v_new[t] is copied element by
 * element (elem_bytes each) into k_cache and v_cache; nothing else changes.
 */
int pa_oracle_cache_write(int elem_bytes, int num_seqs, int num_tokens, int num_kv_heads, int head_dim,
                          int block_size, int num_blocks, int max_blocks_per_seq, void* k_cache, void* v_cache,
                          const void* k_new, const void* v_new, const int32_t* block_tables,
                          const int32_t* context_lens, const int32_t* query_start_loc) {
  if (elem_bytes < 1 || num_seqs < 0 || num_tokens < 0 || num_kv_heads < 1 || head_dim < 1 ||
      block_size < 1 || num_blocks < 1 || max_blocks_per_seq < 1)
    return ORACLE_BAD_ARGUMENT;
  if (query_start_loc == NULL && num_tokens != num_seqs) return ORACLE_BAD_ARGUMENT;
  const size_t row_elems = (size_t)num_kv_heads * head_dim;
  for (int t = 0; t < num_tokens; ++t) {
    int s = t, q_len = 1;
    if (query_start_loc != NULL) {
      s = -1;
      for (int r = 0; r < num_seqs; ++r)
        if (query_start_loc[r] <= t && t < query_start_loc[r + 1]) s = r;
      if (s < 0) return ORACLE_BAD_QUERY_START_LOC;
      q_len = query_start_loc[s + 1] - query_start_loc[s];
    }
    const int j = query_start_loc != NULL ? t - query_start_loc[s] : 0;
    const int ctx = context_lens[s];
    const int pos = ctx - q_len + j;
    if (pos < 0 || ctx > max_blocks_per_seq * block_size) return ORACLE_BAD_CONTEXT_LEN;
    const int block = block_tables[(int64_t)s * max_blocks_per_seq + pos / block_size];
    const int slot = pos % block_size;
    if (block < 0 || block >= num_blocks) return ORACLE_BAD_BLOCK_ID;
    for (size_t e = 0; e < row_elems; ++e) {
      const size_t dst = (((size_t)block * block_size + slot) * row_elems + e) * elem_bytes;
      const size_t src = ((size_t)t * row_elems + e) * elem_bytes;
      for (int b = 0; b < elem_bytes; ++b) {
        ((unsigned char*)k_cache)[dst + b] = ((const unsigned char*)k_new)[src + b];
        ((unsigned char*)v_cache)[dst + b] = ((const unsigned char*)v_new)[src + b];
      }
    }
  }
  return ORACLE_OK;
}

/*
 * Block copy: copy whole physical blocks, keys and values, from a source pool
 * to a destination pool. Pair i copies source block mapping[2i] to destination
 * block mapping[2i+1]; the pairs are applied one after another in the listed
 * order. Each block is [block_size][num_kv_heads][head_dim] elements of
 * elem_bytes bytes, copied element by element.
 *
 * The two uses the pages describe are one operation:
 *   - copy-on-write: the source and destination pools are the same pool; a
 *     block shared by several requests (reference count above one) is copied to
 *     a fresh block before one of them writes into it ("PagedAttention memory
 *     paging and continuous batching in practice" page, comparison table:
 *     copy-on-write and shared blocks for multi-branch decoding; "Continuous
 *     batching" page, section 4.2, prefix sharing);
 *   - swap: one pool is on the GPU and the other in host memory; preemption
 *     moves a request's blocks out and resumption moves them back, block by
 *     block ("Continuous batching" page, section 3.3, preemption by swapping;
 *     "The PagedAttention mechanism in vLLM and memory optimisation practice"
 *     page, section 2.1, block-granular swap on separate copy streams).
 * A block id outside its pool is rejected (ORACLE_BAD_BLOCK_ID) before any
 * byte is copied; nothing but the destination blocks changes.
 */
int pa_oracle_copy_blocks(int elem_bytes, int num_pairs, int block_size, int num_kv_heads, int head_dim,
                          int src_num_blocks, int dst_num_blocks, const void* src_k, const void* src_v,
                          void* dst_k, void* dst_v, const int32_t* mapping) {
  if (elem_bytes < 1 || num_pairs < 0 || block_size < 1 || num_kv_heads < 1 || head_dim < 1 ||
      src_num_blocks < 0 || dst_num_blocks < 0)
    return ORACLE_BAD_ARGUMENT;
  for (int i = 0; i < num_pairs; ++i) {
    const int32_t from = mapping[2 * i], to = mapping[2 * i + 1];
    if (from < 0 || from >= src_num_blocks || to < 0 || to >= dst_num_blocks) return ORACLE_BAD_BLOCK_ID;
  }
  for (int i = 0; i < num_pairs; ++i) {
    const int32_t from = mapping[2 * i], to = mapping[2 * i + 1];
    for (int slot = 0; slot < block_size; ++slot) {
      for (int g = 0; g < num_kv_heads; ++g) {
        for (int d = 0; d < head_dim; ++d) {
          const size_t src = ((((size_t)from * block_size + slot) * num_kv_heads + g) * head_dim + d) * elem_bytes;
          const size_t dst = ((((size_t)to * block_size + slot) * num_kv_heads + g) * head_dim + d) * elem_bytes;
          for (int b = 0; b < elem_bytes; ++b) {
            ((unsigned char*)dst_k)[dst + b] = ((const unsigned char*)src_k)[src + b];
            ((unsigned char*)dst_v)[dst + b] = ((const unsigned char*)src_v)[src + b];
          }
        }
      }
    }
  }
  return ORACLE_OK;
}
