// pa_step.cpp — one decode step of many single-token sequences driven from the
// host allocator: slots and copy-on-write pairs from the allocator, context
// lengths and block tables staged in one host buffer, one upload, then the
// page copies, the cache write and attention enqueued on the caller's stream.
// The per-step work of parallel sampling ("大模型部署.md" §2.1 items 3-4:
// append_slots with copy-on-write, pages shared between the samples of a
// prompt) without a round trip through the caller per operation.
//
// Host code: it calls the allocator and the launchers through their C ABI
// and the HIP runtime only for the asynchronous upload.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "pa_internal.h"

namespace {

struct StepLayout {
  size_t lens, qsl, pairs, tables, total;
};

// Byte offsets inside the staging buffer for n sequences and cap block-table
// columns: slots int64 [n] at 0, context lengths int32 [n], query starts
// int32 [n + 1], copy pairs int32 [n][2] (8-byte aligned), block tables
// int32 [n][cap].
StepLayout step_layout(int64_t n, int64_t cap) {
  StepLayout l;
  l.lens = (size_t)(8 * n);
  l.qsl = l.lens + (size_t)(4 * n);
  l.pairs = (l.qsl + (size_t)(4 * (n + 1)) + 7) & ~(size_t)7;
  l.tables = l.pairs + (size_t)(8 * n);
  l.total = l.tables + (size_t)(4 * n * cap);
  return l;
}

}  // namespace

extern "C" size_t pa_decode_step_staging_bytes(int32_t num_seqs, int32_t max_blocks_per_seq) {
  if (num_seqs <= 0 || max_blocks_per_seq <= 0) return 0;
  return step_layout(num_seqs, max_blocks_per_seq).total;
}

extern "C" pa_status pa_decode_step_stage(pa_allocator* a, int32_t num_seqs, const int64_t* seq_ids,
                                          const int32_t* token_ids, int32_t max_blocks_per_seq, void* host_staging, size_t staging_bytes,
                                          int32_t* num_cow_out, int32_t* max_context_len_out,
                                          int32_t* table_cols_out, size_t* used_bytes_out) {
  const char* fn = "pa_decode_step_stage";
  if (!a || num_seqs <= 0 || !seq_ids || !host_staging || max_blocks_per_seq <= 0 || !num_cow_out ||
      !max_context_len_out || !table_cols_out || !used_bytes_out)
    return pa::fail(PA_ERR_INVALID, "%s: bad argument", fn);
  if ((uintptr_t)host_staging % 8) return pa::fail(PA_ERR_INVALID, "%s: staging buffer not 8-byte aligned", fn);
  if ((int64_t)num_seqs * max_blocks_per_seq > INT32_MAX / 4)
    return pa::fail(PA_ERR_INVALID, "%s: %d sequences x %d table columns too large", fn, num_seqs,
                   max_blocks_per_seq);
  const StepLayout bound = step_layout(num_seqs, max_blocks_per_seq);
  if (staging_bytes < bound.total)
    return pa::fail(PA_ERR_INVALID, "%s: staging buffer of %zu bytes, %zu needed", fn, staging_bytes, bound.total);
  // every sequence must exist and fit max_blocks_per_seq after one more token,
  // checked before the allocator changes
  char* h = (char*)host_staging;
  int32_t* lens = (int32_t*)(h + bound.lens);
  for (int32_t i = 0; i < num_seqs; ++i) {
    pa_status st = pa_seq_num_tokens(a, seq_ids[i], &lens[i]);
    if (st != PA_OK) return st;
    if ((int64_t)lens[i] + 1 > (int64_t)16 * max_blocks_per_seq)
      return pa::fail(PA_ERR_INVALID, "%s: sequence %lld would need more than %d blocks", fn,
                     (long long)seq_ids[i], max_blocks_per_seq);
  }
  int32_t ncow = 0;
  pa_status st = token_ids ? pa_seq_append_tokens(a, num_seqs, seq_ids, token_ids, (int64_t*)h,
                                                  (int32_t*)(h + bound.pairs), &ncow)
                            : pa_seq_append_slots(a, num_seqs, seq_ids, (int64_t*)h, (int32_t*)(h + bound.pairs), &ncow);
  if (st != PA_OK) return st;
  int32_t max_len = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    st = pa_seq_num_tokens(a, seq_ids[i], &lens[i]);
    if (st != PA_OK) return st;
    max_len = std::max(max_len, lens[i]);
  }
  int32_t* qsl = (int32_t*)(h + bound.qsl);
  for (int32_t i = 0; i <= num_seqs; ++i) qsl[i] = i;
  const int32_t cap = (max_len + 15) / 16;
  const StepLayout used = step_layout(num_seqs, cap);  // same offsets up to the tables
  st = pa_seq_block_tables(a, num_seqs, seq_ids, (int32_t*)(h + used.tables), cap);
  if (st != PA_OK) return st;
  *num_cow_out = ncow;
  *max_context_len_out = max_len;
  *table_cols_out = cap;
  *used_bytes_out = used.total;
  return pa::ok();
}

extern "C" pa_status pa_decode_step(pa_allocator* a, int32_t num_seqs, const int64_t* seq_ids,
                                    const int32_t* token_ids, void* out,
                                    const void* q, const void* new_key, const void* new_value, void* k_cache,
                                    void* v_cache, int32_t num_blocks, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, pa_dtype dtype, float scale, const int32_t* groups,
                                    int32_t num_groups, int32_t max_blocks_per_seq, void* host_staging,
                                    void* dev_staging, size_t staging_bytes, void* workspace,
                                    size_t workspace_bytes, int32_t* dev_status, void* stream) {
  const char* fn = "pa_decode_step";
  if (!out || !q || !new_key || !new_value || !k_cache || !v_cache || !dev_staging || !workspace)
    return pa::fail(PA_ERR_INVALID, "%s: NULL device pointer", fn);
  if ((uintptr_t)dev_staging % 8) return pa::fail(PA_ERR_INVALID, "%s: device staging not 8-byte aligned", fn);
  if ((uintptr_t)workspace % 256) return pa::fail(PA_ERR_INVALID, "%s: workspace not 256-byte aligned", fn);
  if (num_groups < 0 || (num_groups > 0 && !groups)) return pa::fail(PA_ERR_INVALID, "%s: bad group list", fn);
  if (num_blocks <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads)
    return pa::fail(PA_ERR_INVALID, "%s: bad pool or head counts", fn);
  if (dtype != PA_F32 && dtype != PA_BF16) return pa::fail(PA_ERR_UNSUPPORTED, "%s: dtype %d", fn, (int)dtype);
  if (head_dim != 64 && head_dim != 128)
    return pa::fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d (64 or 128 supported)", fn, head_dim);
  if (num_groups > 0 && (dtype != PA_BF16 || 2 * (num_q_heads / num_kv_heads) > 16))
    return pa::fail(PA_ERR_UNSUPPORTED, "%s: shared prefixes need bfloat16 and at most 8 query heads per KV head",
                   fn);
  if (num_groups > num_seqs) return pa::fail(PA_ERR_INVALID, "%s: %d groups for %d sequences", fn, num_groups, num_seqs);
  if (!std::isfinite(scale)) return pa::fail(PA_ERR_INVALID, "%s: scale is not finite", fn);
  if (num_seqs <= 0 || max_blocks_per_seq <= 0 || (int64_t)max_blocks_per_seq * 16 > INT32_MAX)
    return pa::fail(PA_ERR_INVALID, "%s: bad sequence count or table width", fn);
  // the workspace must hold a batch whose longest context fills max_blocks_per_seq
  const int32_t ctx_bound = 16 * max_blocks_per_seq;
  const size_t ws_need =
      num_groups > 0 ? pa_forward_shared_workspace_bytes(num_seqs, num_groups, num_seqs, 1, num_q_heads,
                                                         num_kv_heads, head_dim, ctx_bound, dtype)
                     : pa_forward_workspace_bytes(num_seqs, num_seqs, 1, num_q_heads, num_kv_heads, head_dim,
                                                  ctx_bound, dtype);
  if (workspace_bytes < ws_need)
    return pa::fail(PA_ERR_INVALID, "%s: workspace of %zu bytes, %zu needed for contexts up to %d", fn,
                   workspace_bytes, ws_need, ctx_bound);

  int32_t ncow = 0, max_len = 0, cap = 0;
  size_t used = 0;
  pa_status st = pa_decode_step_stage(a, num_seqs, seq_ids, token_ids, max_blocks_per_seq, host_staging,
                                      staging_bytes, &ncow, &max_len, &cap, &used);
  if (st != PA_OK) return st;
  const StepLayout l = step_layout(num_seqs, cap);
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  hipError_t e = hipMemcpyAsync(dev_staging, host_staging, used, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return pa::fail(PA_ERR_HIP, "%s: upload failed: %s", fn, hipGetErrorString(e));
  char* d = (char*)dev_staging;
  if (ncow > 0) {
    st = pa_copy_blocks(k_cache, v_cache, (const int32_t*)(d + l.pairs), ncow, num_blocks, num_kv_heads, head_dim, 16,
                        dtype, dev_status, stream);
    if (st != PA_OK) return st;
  }
  st = pa_reshape_and_cache(new_key, new_value, k_cache, v_cache, (const int64_t*)d, num_seqs, num_blocks,
                            num_kv_heads, head_dim, 16, dtype, dev_status, stream);
  if (st != PA_OK) return st;
  const int32_t* tables = (const int32_t*)(d + l.tables);
  const int32_t* lens = (const int32_t*)(d + l.lens);
  const int32_t* qsl = (const int32_t*)(d + l.qsl);
  if (num_groups > 0)
    return pa_forward_shared(out, q, k_cache, v_cache, tables, cap, lens, qsl, groups, num_groups, num_seqs, num_seqs,
                             1, max_len, num_q_heads, num_kv_heads, head_dim, 16, num_blocks, scale, dtype, workspace,
                             workspace_bytes, dev_status, stream);
  return pa_forward(out, q, k_cache, v_cache, tables, cap, lens, qsl, num_seqs, num_seqs, 1, max_len, num_q_heads,
                    num_kv_heads, head_dim, 16, num_blocks, scale, dtype, workspace, workspace_bytes, dev_status,
                    stream);
}
