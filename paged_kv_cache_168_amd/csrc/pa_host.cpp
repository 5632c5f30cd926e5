// Host side of the C ABI that needs no GPU: the error detail, argument validation and the checkers of the
// device-data preconditions on host copies (pa_check_*_host). Plain C++; the entry points that launch kernels
// are in pa_api.cpp.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <vector>

#include "pa.h"
#include "pa_host.h"

namespace pa {

namespace {
thread_local char g_detail[kDetailBytes] = "";
}  // namespace

char* error_detail() { return g_detail; }

pa_status fail(pa_status st, const char* what) {
  std::snprintf(g_detail, sizeof g_detail, "%s", what);
  return st;
}

pa_status validate_params(const pa_params* p) {
  if (p == nullptr) return fail(PA_ERR_NULL_POINTER, "params is NULL");
  if (p->num_q_heads < 1 || p->num_kv_heads < 1 || p->num_q_heads % p->num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_q_heads must be a positive multiple of num_kv_heads >= 1");
  if (p->head_dim < 1) return fail(PA_ERR_INVALID_ARGUMENT, "head_dim must be positive");
  if (p->head_dim != 64 && p->head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (p->block_size < 1 || p->num_blocks < 1 || p->max_blocks_per_seq < 1)
    return fail(PA_ERR_INVALID_ARGUMENT, "block_size, num_blocks and max_blocks_per_seq must be >= 1");
  if ((int64_t)p->max_blocks_per_seq * p->block_size > INT32_MAX)
    return fail(PA_ERR_INVALID_ARGUMENT, "max_blocks_per_seq * block_size overflows int32");
  if (p->dtype != PA_DTYPE_FP32 && p->dtype != PA_DTYPE_BF16)
    return fail(PA_ERR_INVALID_ARGUMENT, "dtype must be PA_DTYPE_FP32 or PA_DTYPE_BF16");
  if (!std::isfinite(p->scale)) return fail(PA_ERR_INVALID_ARGUMENT, "scale must be finite");
  const int pt = p->partition_tokens;
  if (pt != 0 && (pt % kTileTokens != 0 || pt < kTileTokens || pt > kMaxPartitionTokens))
    return fail(PA_ERR_INVALID_ARGUMENT, "partition_tokens must be 0 or a multiple of 16 in [16, 1024]");
  if ((p->flags & ~PA_FLAG_SHARED_BLOCKS) != 0) return fail(PA_ERR_INVALID_ARGUMENT, "flags has unknown bits");
  if (p->layout != PA_LAYOUT_TOKEN_MAJOR && p->layout != PA_LAYOUT_HEAD_MAJOR)
    return fail(PA_ERR_INVALID_ARGUMENT, "layout must be PA_LAYOUT_TOKEN_MAJOR or PA_LAYOUT_HEAD_MAJOR");
  return PA_OK;
}

}  // namespace pa

using pa::fail;
using pa::validate_params;

extern "C" {

pa_status pa_check_groups_host(const pa_params* params, int32_t num_seqs, int32_t num_groups,
                               const int32_t* group_start, const int32_t* group_prefix,
                               const int32_t* block_tables, const int32_t* context_lens, int64_t* first_bad) {
  if (first_bad) *first_bad = -1;
  pa_status st = validate_params(params);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_groups < 0) return fail(PA_ERR_INVALID_ARGUMENT, "negative count");
  if (num_groups == 0) return PA_OK;
  if (!group_start || !group_prefix || (num_seqs > 0 && (!block_tables || !context_lens)))
    return fail(PA_ERR_NULL_POINTER, "an array is NULL");
  if (group_start[0] != 0 || group_start[num_groups] != num_seqs)
    return fail(PA_ERR_INVALID_ARGUMENT, "group_start must run from 0 to num_seqs");
  const int32_t BS = params->block_size, W = params->max_blocks_per_seq;
  for (int32_t g = 0; g < num_groups; ++g) {
    const int32_t a = group_start[g], b = group_start[g + 1];
    int32_t pre = group_prefix[g];
    bool bad = b < a || b > num_seqs || pre < 0 || pre % BS != 0;
    if (!bad && b > a && pre > 0) {
      pre = std::min(pre, std::max(context_lens[a], 0));  // the prefix pass reads the first request's table
      pre -= pre % BS;
      for (int32_t s = a + 1; s < b && !bad; ++s) {
        const int32_t seen = std::min(pre, std::max(context_lens[s], 0));
        const int32_t nb = std::min((seen + BS - 1) / BS, W);
        for (int32_t e = 0; e < nb && !bad; ++e)
          bad = block_tables[(int64_t)s * W + e] != block_tables[(int64_t)a * W + e];
      }
    }
    if (bad) {
      if (first_bad) *first_bad = g;
      return fail(PA_ERR_INVALID_ARGUMENT, "a group does not share the blocks it declares");
    }
  }
  return PA_OK;
}

pa_status pa_check_copy_host(int32_t num_pairs, const int32_t* mapping, int32_t src_num_blocks, int32_t dst_num_blocks,
                             int32_t same_pool, int64_t* first_bad) {
  if (first_bad) *first_bad = -1;
  if (num_pairs < 0 || src_num_blocks < 1 || dst_num_blocks < 1)
    return fail(PA_ERR_INVALID_ARGUMENT, "negative pair count or empty pool");
  if (same_pool && src_num_blocks != dst_num_blocks)
    return fail(PA_ERR_INVALID_ARGUMENT, "one pool has one block count");
  if (num_pairs > 0 && !mapping) return fail(PA_ERR_NULL_POINTER, "mapping is NULL");
  // role of each destination-pool block: 1 = a destination so far, 2 = a source (within one pool)
  std::vector<uint8_t> role(dst_num_blocks, 0);
  int64_t bad = -1;
  for (int32_t i = 0; i < num_pairs && bad < 0; ++i) {
    const int32_t from = mapping[2 * i], to = mapping[2 * i + 1];
    if (from < 0 || from >= src_num_blocks || to < 0 || to >= dst_num_blocks) bad = i;
    else if (same_pool) role[from] |= 2;
  }
  for (int32_t i = 0; i < (bad < 0 ? num_pairs : bad); ++i) {
    const int32_t to = mapping[2 * i + 1];
    if (role[to] != 0) {
      bad = i;
      break;
    }
    role[to] = 1;
  }
  if (bad >= 0) {
    if (first_bad) *first_bad = bad;
    return fail(PA_ERR_INVALID_ARGUMENT, "a pair leaves its pool, repeats a destination or writes a source");
  }
  return PA_OK;
}

pa_status pa_check_inputs_host(const pa_params* params, int32_t num_seqs, int32_t num_tokens, int32_t max_query_len,
                               const int32_t* block_tables, const int32_t* context_lens,
                               const int32_t* query_start_loc, int64_t* first_bad) {
  if (first_bad) *first_bad = -1;
  pa_status st = validate_params(params);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_tokens < 0) return fail(PA_ERR_INVALID_ARGUMENT, "negative count");
  if (num_seqs > 0 && (!block_tables || !context_lens)) return fail(PA_ERR_NULL_POINTER, "table pointer is NULL");
  if (query_start_loc == nullptr && num_tokens != num_seqs)
    return fail(PA_ERR_INVALID_ARGUMENT, "decode batch needs num_tokens == num_seqs");
  if (query_start_loc != nullptr && (query_start_loc[0] != 0 || query_start_loc[num_seqs] != num_tokens))
    return fail(PA_ERR_INVALID_ARGUMENT, "query_start_loc must run from 0 to num_tokens");
  const int64_t max_ctx = (int64_t)params->max_blocks_per_seq * params->block_size;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t ctx = context_lens[s];
    int32_t q_len = 1;
    if (query_start_loc) q_len = query_start_loc[s + 1] - query_start_loc[s];
    bool bad = ctx < 1 || ctx > max_ctx || q_len < 0 || q_len > ctx || (max_query_len > 0 && q_len > max_query_len);
    if (!bad) {
      const int32_t used = (ctx + params->block_size - 1) / params->block_size;
      for (int32_t b = 0; b < used && !bad; ++b) {
        const int32_t id = block_tables[(int64_t)s * params->max_blocks_per_seq + b];
        bad = id < 0 || id >= params->num_blocks;
      }
    }
    if (bad) {
      if (first_bad) *first_bad = s;
      return fail(PA_ERR_INVALID_ARGUMENT, "request violates a device-data precondition");
    }
  }
  return PA_OK;
}

const char* pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL_POINTER: return "null pointer";
    case PA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case PA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* pa_last_error_detail(void) { return pa::error_detail(); }

}  // extern "C"
