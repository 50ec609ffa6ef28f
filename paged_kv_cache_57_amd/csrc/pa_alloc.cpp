// Host-side reference-counted block allocator and per-sequence block tables.
//
// Follows the block manager the pages describe: "大模型部署.md" §2.1 item 3
// (BlockSpaceManagerV1: _allocate_sequence gives a prompt ceil(L/P) blocks with
// reference counts; can_allocate compares free blocks with a watermark and
// answers NEVER / OK / LATER; append_slots takes a new block when the table is
// one short and copies the last block on write when it is shared, returning
// the (old, new) pair) and "第7章：大模型部署实战" §2.3 (the free list is popped
// from its end on allocation and appended to on release).  Forking shares
// every block of the parent ("大模型部署.md" §2.1 item 4, sharing between the
// samples of one prompt); the pages print no fork code, so the plain reading
// is used: copy the table, add one reference per block.
//
// Every mutation checks all its preconditions before touching any state, so a
// failing call leaves the allocator exactly as it was.
#include <algorithm>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_internal.h"

struct pa_allocator {
  struct Seq {
    std::vector<int32_t> table;
    int32_t ntok = 0;
  };
  int32_t num_blocks = 0;
  int32_t block_size = 16;
  int32_t watermark_blocks = 0;
  std::vector<int32_t> free_stack;  // top = back()
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, Seq> seqs;

  int64_t blocks_for(int64_t n) const { return (n + block_size - 1) / block_size; }
  int32_t take() {
    int32_t b = free_stack.back();
    free_stack.pop_back();
    ref[b] = 1;
    return b;
  }
};

using pa::fail;
using pa::ok;

extern "C" {

pa_status pa_alloc_create(int32_t num_blocks, int32_t block_size, double watermark,
                          const int32_t* initial_free_order, pa_allocator** out) {
  if (!out) return fail(PA_ERR_INVALID, "pa_alloc_create: out is NULL");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0)
    return fail(PA_ERR_INVALID, "pa_alloc_create: num_blocks %d and block_size %d must be > 0",
                num_blocks, block_size);
  if (!(watermark >= 0.0) || watermark > 1.0)
    return fail(PA_ERR_INVALID, "pa_alloc_create: watermark %g outside [0, 1]", (double)watermark);
  auto* a = new (std::nothrow) pa_allocator();
  if (!a) return fail(PA_ERR_INVALID, "pa_alloc_create: out of host memory");
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  // int(watermark * num_blocks), truncated toward zero
  a->watermark_blocks = (int32_t)(watermark * (double)num_blocks);
  a->ref.assign(num_blocks, 0);
  a->free_stack.resize(num_blocks);
  if (initial_free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = initial_free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete a;
        return fail(PA_ERR_INVALID, "pa_alloc_create: initial_free_order is not a permutation");
      }
      seen[b] = 1;
      a->free_stack[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) a->free_stack[i] = i;
  }
  *out = a;
  return ok();
}

void pa_alloc_destroy(pa_allocator* a) { delete a; }

int32_t pa_alloc_num_free(const pa_allocator* a) {
  return a ? (int32_t)a->free_stack.size() : -1;
}

int32_t pa_alloc_ref_count(const pa_allocator* a, int32_t block) {
  if (!a || block < 0 || block >= a->num_blocks) return -1;
  return a->ref[block];
}

pa_status pa_alloc_can_allocate(const pa_allocator* a, int32_t num_tokens, pa_alloc_status* out) {
  if (!a || !out) return fail(PA_ERR_INVALID, "pa_alloc_can_allocate: NULL argument");
  if (num_tokens < 0) return fail(PA_ERR_INVALID, "pa_alloc_can_allocate: negative length");
  int64_t req = a->blocks_for(num_tokens);
  if ((int64_t)a->num_blocks - req < a->watermark_blocks)
    *out = PA_ALLOC_NEVER;
  else if ((int64_t)a->free_stack.size() - req >= a->watermark_blocks)
    *out = PA_ALLOC_OK;
  else
    *out = PA_ALLOC_LATER;
  return ok();
}

pa_status pa_seq_create(pa_allocator* a, int64_t seq_id, int32_t num_tokens) {
  if (!a) return fail(PA_ERR_INVALID, "pa_seq_create: NULL allocator");
  if (num_tokens < 0) return fail(PA_ERR_INVALID, "pa_seq_create: negative length");
  if (a->seqs.count(seq_id))
    return fail(PA_ERR_INVALID, "pa_seq_create: sequence %lld exists", (long long)seq_id);
  int64_t req = a->blocks_for(num_tokens);
  if (req > (int64_t)a->free_stack.size())
    return fail(PA_ERR_NO_BLOCKS, "pa_seq_create: %lld blocks needed, %zu free", (long long)req,
                a->free_stack.size());
  pa_allocator::Seq s;
  s.table.reserve(req);
  for (int64_t j = 0; j < req; ++j) s.table.push_back(a->take());
  s.ntok = num_tokens;
  a->seqs.emplace(seq_id, std::move(s));
  return ok();
}

pa_status pa_seq_fork(pa_allocator* a, int64_t parent_id, int64_t child_id) {
  if (!a) return fail(PA_ERR_INVALID, "pa_seq_fork: NULL allocator");
  auto it = a->seqs.find(parent_id);
  if (it == a->seqs.end())
    return fail(PA_ERR_NOT_FOUND, "pa_seq_fork: unknown parent %lld", (long long)parent_id);
  if (a->seqs.count(child_id))
    return fail(PA_ERR_INVALID, "pa_seq_fork: child %lld exists", (long long)child_id);
  pa_allocator::Seq child = it->second;
  for (int32_t b : child.table) a->ref[b] += 1;
  a->seqs.emplace(child_id, std::move(child));
  return ok();
}

pa_status pa_seq_append_slot(pa_allocator* a, int64_t seq_id, int64_t* slot_out, int32_t* cow_src,
                             int32_t* cow_dst) {
  if (!a || !slot_out || !cow_src || !cow_dst)
    return fail(PA_ERR_INVALID, "pa_seq_append_slot: NULL argument");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end())
    return fail(PA_ERR_NOT_FOUND, "pa_seq_append_slot: unknown sequence %lld", (long long)seq_id);
  auto& s = it->second;
  const int64_t L = s.ntok;
  if (L >= INT32_MAX) return fail(PA_ERR_INVALID, "pa_seq_append_slot: sequence too long");
  const int64_t need = a->blocks_for(L + 1);
  int32_t src = -1, dst = -1;
  if ((int64_t)s.table.size() < need) {
    if ((int64_t)s.table.size() != need - 1)
      return fail(PA_ERR_INVALID, "pa_seq_append_slot: table of %zu blocks for %lld tokens",
                  s.table.size(), (long long)L);
    if (a->free_stack.empty())
      return fail(PA_ERR_NO_BLOCKS, "pa_seq_append_slot: no free block for a new page");
    s.table.push_back(a->take());
  } else if (a->ref[s.table.back()] > 1) {
    if (a->free_stack.empty())
      return fail(PA_ERR_NO_BLOCKS, "pa_seq_append_slot: no free block for copy-on-write");
    src = s.table.back();
    dst = a->take();
    s.table.back() = dst;
    a->ref[src] -= 1;  // > 1 before, so still held by another sequence
  }
  s.ntok = (int32_t)(L + 1);
  *slot_out = (int64_t)s.table[L / a->block_size] * a->block_size + L % a->block_size;
  *cow_src = src;
  *cow_dst = dst;
  return ok();
}

pa_status pa_seq_append_slots(pa_allocator* a, int32_t n, const int64_t* seq_ids, int64_t* slots_out,
                              int32_t* cow_pairs_out, int32_t* num_cow_out) {
  if (!a || n < 0 || (n > 0 && (!seq_ids || !slots_out || !cow_pairs_out)) || !num_cow_out)
    return fail(PA_ERR_INVALID, "pa_seq_append_slots: bad argument");
  int32_t ncow = 0;
  *num_cow_out = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t src, dst;
    pa_status st = pa_seq_append_slot(a, seq_ids[i], &slots_out[i], &src, &dst);
    if (st != PA_OK) {
      *num_cow_out = ncow;
      return st;
    }
    if (src >= 0) {
      cow_pairs_out[2 * ncow] = src;
      cow_pairs_out[2 * ncow + 1] = dst;
      ++ncow;
    }
  }
  *num_cow_out = ncow;
  return ok();
}

pa_status pa_seq_slots(const pa_allocator* a, int64_t seq_id, int32_t start, int32_t n,
                       int64_t* slots_out) {
  if (!a || (n > 0 && !slots_out)) return fail(PA_ERR_INVALID, "pa_seq_slots: NULL argument");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end())
    return fail(PA_ERR_NOT_FOUND, "pa_seq_slots: unknown sequence %lld", (long long)seq_id);
  const auto& s = it->second;
  if (start < 0 || n < 0 || (int64_t)start + n > s.ntok)
    return fail(PA_ERR_INVALID, "pa_seq_slots: positions [%d, %lld) outside the sequence of %d",
                start, (long long)start + n, s.ntok);
  for (int32_t i = 0; i < n; ++i) {
    int64_t p = (int64_t)start + i;
    slots_out[i] = (int64_t)s.table[p / a->block_size] * a->block_size + p % a->block_size;
  }
  return ok();
}

pa_status pa_seq_num_tokens(const pa_allocator* a, int64_t seq_id, int32_t* out) {
  if (!a || !out) return fail(PA_ERR_INVALID, "pa_seq_num_tokens: NULL argument");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end())
    return fail(PA_ERR_NOT_FOUND, "pa_seq_num_tokens: unknown sequence %lld", (long long)seq_id);
  *out = it->second.ntok;
  return ok();
}

pa_status pa_seq_block_table(const pa_allocator* a, int64_t seq_id, int32_t* out, int32_t cap,
                             int32_t* n_out) {
  if (!a || !n_out || (cap > 0 && !out)) return fail(PA_ERR_INVALID, "pa_seq_block_table: NULL argument");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end())
    return fail(PA_ERR_NOT_FOUND, "pa_seq_block_table: unknown sequence %lld", (long long)seq_id);
  const auto& t = it->second.table;
  *n_out = (int32_t)t.size();
  if ((int64_t)t.size() > cap)
    return fail(PA_ERR_INVALID, "pa_seq_block_table: %zu blocks, capacity %d", t.size(), cap);
  std::copy(t.begin(), t.end(), out);
  return ok();
}

pa_status pa_seq_block_tables(const pa_allocator* a, int32_t n, const int64_t* seq_ids, int32_t* out,
                              int32_t cap) {
  if (!a || n < 0 || cap < 0 || (n > 0 && (!seq_ids || (cap > 0 && !out))))
    return fail(PA_ERR_INVALID, "pa_seq_block_tables: bad argument");
  for (int32_t i = 0; i < n; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end())
      return fail(PA_ERR_NOT_FOUND, "pa_seq_block_tables: unknown sequence %lld", (long long)seq_ids[i]);
    if ((int64_t)it->second.table.size() > cap)
      return fail(PA_ERR_INVALID, "pa_seq_block_tables: sequence %lld has %zu blocks, capacity %d",
                  (long long)seq_ids[i], it->second.table.size(), cap);
  }
  for (int32_t i = 0; i < n; ++i) {
    const auto& t = a->seqs.find(seq_ids[i])->second.table;
    int32_t* row = out + (int64_t)i * cap;
    std::copy(t.begin(), t.end(), row);
    std::fill(row + t.size(), row + cap, -1);
  }
  return ok();
}

pa_status pa_seq_free(pa_allocator* a, int64_t seq_id) {
  if (!a) return fail(PA_ERR_INVALID, "pa_seq_free: NULL allocator");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end())
    return fail(PA_ERR_NOT_FOUND, "pa_seq_free: unknown sequence %lld", (long long)seq_id);
  for (int32_t b : it->second.table)
    if (a->ref[b] <= 0) return fail(PA_ERR_REFCOUNT, "pa_seq_free: block %d has no reference", b);
  for (int32_t b : it->second.table) {
    if (--a->ref[b] == 0) a->free_stack.push_back(b);
  }
  a->seqs.erase(it);
  return ok();
}

}  // extern "C"
