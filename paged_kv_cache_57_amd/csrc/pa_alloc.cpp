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
// Prefix caching ("大模型部署.md" §2.1 item 3, CachedBlockAllocator and
// LRUEvictor; "【自用】AI infra相关" part 二.4(2)), switched on per allocator:
// every full block of a sequence made from token ids carries a hash chained
// from the previous block's hash and its own tokens; a block whose hash is
// already cached (in use, or released and waiting in the evictor) is shared
// instead of allocated; a released hashed block waits in the evictor until a
// new block is needed and the free stack is empty, and the evictor gives up
// its least recently released block, among equally old ones the one whose
// hash covers the most tokens.  A hit compares the block's own tokens and its
// parent's hash too, so a 64-bit hash collision can only ever cost a miss.
//
// Every mutation checks all its preconditions before touching any state, so a
// failing call leaves the allocator exactly as it was.
#include <algorithm>
#include <cstring>
#include <list>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_internal.h"

struct pa_allocator {
  struct Seq {
    std::vector<int32_t> table;
    int32_t ntok = 0;
    bool hashed = false;            // made from token ids on a caching allocator
    std::vector<int32_t> tokens;    // all tokens (hashed sequences)
    std::vector<uint64_t> chain;    // hash of every full block, in order (hashed sequences)
    int32_t sinks = -1;             // streaming sequences (sinks >= 0): sink tokens kept,
    int32_t window = 0;             // then the most recent `window` tokens;
    int64_t seen = 0;               // tokens appended so far (ntok stops at sinks + window)
  };
  int32_t num_blocks = 0;
  int32_t block_size = 16;
  int32_t watermark_blocks = 0;
  std::vector<int32_t> free_stack;  // top = back()
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, Seq> seqs;

  // prefix caching
  bool caching = false;
  uint64_t clock = 0;                        // advances at every mutating call
  std::vector<char> has_hash;
  std::vector<uint64_t> hash, parent, accessed;
  std::vector<int32_t> hashed_tokens;
  std::vector<int32_t> block_tokens;         // [num_blocks][block_size], hashed blocks
  std::unordered_map<uint64_t, int32_t> cached;
  std::list<int32_t> evictor;                // insertion order
  std::vector<std::list<int32_t>::iterator> evictor_pos;
  std::vector<char> in_evictor;

  int64_t blocks_for(int64_t n) const { return (n + block_size - 1) / block_size; }
  int64_t available() const { return (int64_t)free_stack.size() + (int64_t)evictor.size(); }

  void forget(int32_t b) {
    cached.erase(hash[b]);
    has_hash[b] = 0;
    hashed_tokens[b] = 0;
  }
  // LRUEvictor.evict: the first block in insertion order, replaced by a later
  // one with more hashed tokens while the access times are equal
  int32_t evict() {
    auto best = evictor.begin();
    for (auto it = evictor.begin(); it != evictor.end(); ++it) {
      if (accessed[*best] < accessed[*it]) break;
      if (hashed_tokens[*best] < hashed_tokens[*it]) best = it;
    }
    const int32_t b = *best;
    evictor.erase(best);
    in_evictor[b] = 0;
    forget(b);
    return b;
  }
  // a fresh block: the free stack's top, else one evicted block (caller checked available())
  int32_t take() {
    int32_t b;
    if (!free_stack.empty()) {
      b = free_stack.back();
      free_stack.pop_back();
    } else {
      b = evict();
    }
    ref[b] = 1;
    return b;
  }
  // one more reference to a cached block (it leaves the evictor if it waits there)
  void share(int32_t b) {
    if (ref[b] == 0) {
      evictor.erase(evictor_pos[b]);
      in_evictor[b] = 0;
    }
    ref[b] += 1;
  }
  void release(int32_t b) {
    if (--ref[b] == 0) {
      if (caching && has_hash[b]) {
        accessed[b] = clock;
        evictor.push_back(b);
        evictor_pos[b] = std::prev(evictor.end());
        in_evictor[b] = 1;
      } else {
        free_stack.push_back(b);
      }
    }
  }
  static uint64_t mix(uint64_t x) {  // splitmix64 finaliser
    x ^= x >> 30;
    x *= 0xbf58476d1ce4e5b9ull;
    x ^= x >> 27;
    x *= 0x94d049bb133111ebull;
    return x ^ (x >> 31);
  }
  uint64_t block_hash(uint64_t prev, const int32_t* toks) const {
    uint64_t h = mix(prev ^ 0x9e3779b97f4a7c15ull);
    for (int32_t i = 0; i < block_size; ++i) h = mix(h + (uint32_t)toks[i] + 0x632be59bd9b4e019ull);
    return h;
  }
  static constexpr uint64_t kRootHash = 0x243f6a8885a308d3ull;
  // the cached block holding exactly these tokens after a prefix hashed `prev`, or -1
  int32_t lookup(uint64_t h, uint64_t prev, const int32_t* toks) const {
    auto it = cached.find(h);
    if (it == cached.end()) return -1;
    const int32_t b = it->second;
    if (parent[b] != prev ||
        std::memcmp(&block_tokens[(size_t)b * block_size], toks, sizeof(int32_t) * block_size) != 0)
      return -1;
    return b;
  }
  void register_block(int32_t b, uint64_t h, uint64_t prev, const int32_t* toks, int32_t ntok) {
    if (cached.count(h)) return;  // a colliding hash: the block stays uncached
    has_hash[b] = 1;
    hash[b] = h;
    parent[b] = prev;
    hashed_tokens[b] = ntok;
    std::memcpy(&block_tokens[(size_t)b * block_size], toks, sizeof(int32_t) * block_size);
    cached.emplace(h, b);
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
  return a ? (int32_t)a->available() : -1;
}

int32_t pa_alloc_num_evictable(const pa_allocator* a) {
  return a ? (int32_t)a->evictor.size() : -1;
}

pa_status pa_alloc_enable_prefix_caching(pa_allocator* a) {
  if (!a) return fail(PA_ERR_INVALID, "pa_alloc_enable_prefix_caching: NULL allocator");
  if (!a->seqs.empty() || (int32_t)a->free_stack.size() != a->num_blocks)
    return fail(PA_ERR_INVALID, "pa_alloc_enable_prefix_caching: the allocator is in use");
  if (a->caching) return ok();
  const size_t n = (size_t)a->num_blocks;
  try {
    a->has_hash.assign(n, 0);
    a->hash.assign(n, 0);
    a->parent.assign(n, 0);
    a->accessed.assign(n, 0);
    a->hashed_tokens.assign(n, 0);
    a->block_tokens.assign(n * (size_t)a->block_size, 0);
    a->evictor_pos.assign(n, a->evictor.end());
    a->in_evictor.assign(n, 0);
  } catch (const std::bad_alloc&) {
    return fail(PA_ERR_INVALID, "pa_alloc_enable_prefix_caching: out of host memory");
  }
  a->caching = true;
  return ok();
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
  else if (a->available() - req >= a->watermark_blocks)
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
  if (req > a->available())
    return fail(PA_ERR_NO_BLOCKS, "pa_seq_create: %lld blocks needed, %lld free", (long long)req,
                (long long)a->available());
  a->clock += 1;
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
  a->clock += 1;
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
  if (s.hashed)
    return fail(PA_ERR_INVALID, "pa_seq_append_slot: sequence %lld was made from token ids: use pa_seq_append_tokens",
                (long long)seq_id);
  if (s.sinks >= 0 && s.seen >= (int64_t)s.sinks + s.window) {
    // a full streaming cache: the new token replaces the oldest window token (a ring over the
    // window positions; attention does not depend on the order of its keys)
    const int64_t pos = s.sinks + (s.seen - s.sinks) % s.window;
    const int64_t j = pos / a->block_size;
    int32_t src = -1, dst = -1;
    if (a->ref[s.table[j]] > 1) {
      if (a->available() == 0)
        return fail(PA_ERR_NO_BLOCKS, "pa_seq_append_slot: no free block for copy-on-write");
      a->clock += 1;
      src = s.table[j];
      dst = a->take();
      a->ref[src] -= 1;  // > 1 before, so still held by another sequence
      s.table[j] = dst;
    } else {
      a->clock += 1;
    }
    s.seen += 1;
    *slot_out = (int64_t)s.table[j] * a->block_size + pos % a->block_size;
    *cow_src = src;
    *cow_dst = dst;
    return ok();
  }
  const int64_t L = s.ntok;
  if (L >= INT32_MAX) return fail(PA_ERR_INVALID, "pa_seq_append_slot: sequence too long");
  const int64_t need = a->blocks_for(L + 1);
  int32_t src = -1, dst = -1;
  if ((int64_t)s.table.size() < need) {
    if ((int64_t)s.table.size() != need - 1)
      return fail(PA_ERR_INVALID, "pa_seq_append_slot: table of %zu blocks for %lld tokens",
                  s.table.size(), (long long)L);
    if (a->available() == 0)
      return fail(PA_ERR_NO_BLOCKS, "pa_seq_append_slot: no free block for a new page");
    a->clock += 1;
    s.table.push_back(a->take());
  } else if (a->ref[s.table.back()] > 1) {
    if (a->available() == 0)
      return fail(PA_ERR_NO_BLOCKS, "pa_seq_append_slot: no free block for copy-on-write");
    a->clock += 1;
    src = s.table.back();
    dst = a->take();
    s.table.back() = dst;
    a->ref[src] -= 1;  // > 1 before, so still held by another sequence
  } else {
    a->clock += 1;
  }
  s.ntok = (int32_t)(L + 1);
  if (s.sinks >= 0) s.seen += 1;
  *slot_out = (int64_t)s.table[L / a->block_size] * a->block_size + L % a->block_size;
  *cow_src = src;
  *cow_dst = dst;
  return ok();
}

pa_status pa_seq_create_streaming(pa_allocator* a, int64_t seq_id, int32_t num_sinks, int32_t window,
                                  int32_t num_tokens) {
  if (!a) return fail(PA_ERR_INVALID, "pa_seq_create_streaming: NULL allocator");
  if (num_sinks < 0 || window <= 0 || (int64_t)num_sinks + window > INT32_MAX || num_tokens < 0 ||
      (int64_t)num_tokens > (int64_t)num_sinks + window)
    return fail(PA_ERR_INVALID, "pa_seq_create_streaming: sinks %d, window %d, %d tokens", num_sinks, window,
                num_tokens);
  pa_status st = pa_seq_create(a, seq_id, num_tokens);
  if (st != PA_OK) return st;
  auto& s = a->seqs.find(seq_id)->second;
  s.sinks = num_sinks;
  s.window = window;
  s.seen = num_tokens;
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
  a->clock += 1;
  for (int32_t b : it->second.table) a->release(b);
  a->seqs.erase(it);
  return ok();
}

pa_status pa_seq_create_tokens(pa_allocator* a, int64_t seq_id, const int32_t* token_ids, int32_t num_tokens,
                               int32_t* num_cached_tokens) {
  const char* fn = "pa_seq_create_tokens";
  if (!a || !num_cached_tokens || (num_tokens > 0 && !token_ids))
    return fail(PA_ERR_INVALID, "%s: NULL argument", fn);
  if (!a->caching) return fail(PA_ERR_INVALID, "%s: prefix caching is not enabled", fn);
  if (num_tokens < 0) return fail(PA_ERR_INVALID, "%s: negative length", fn);
  if (a->seqs.count(seq_id)) return fail(PA_ERR_INVALID, "%s: sequence %lld exists", fn, (long long)seq_id);
  const int32_t P = a->block_size;
  const int64_t nblk = a->blocks_for(num_tokens);
  const int64_t nfull = num_tokens / P;
  pa_allocator::Seq s;
  s.hashed = true;
  s.tokens.assign(token_ids, token_ids + num_tokens);
  s.chain.resize(nfull);
  std::vector<int32_t> hit(nfull, -1);
  int64_t nhit = 0, revive = 0;
  uint64_t prev = pa_allocator::kRootHash;
  for (int64_t j = 0; j < nfull; ++j) {
    const int32_t* t = token_ids + j * P;
    s.chain[j] = a->block_hash(prev, t);
    hit[j] = a->lookup(s.chain[j], prev, t);
    if (hit[j] >= 0) {
      ++nhit;
      revive += a->ref[hit[j]] == 0;
    }
    prev = s.chain[j];
  }
  if (nblk - nhit > a->available() - revive)
    return fail(PA_ERR_NO_BLOCKS, "%s: %lld new blocks needed, %lld free", fn, (long long)(nblk - nhit),
                (long long)(a->available() - revive));
  a->clock += 1;
  s.table.assign(nblk, -1);
  for (int64_t j = 0; j < nfull; ++j)  // reused blocks first, so no eviction can take one of them
    if (hit[j] >= 0) {
      a->share(hit[j]);
      s.table[j] = hit[j];
    }
  for (int64_t j = 0; j < nblk; ++j) {
    if (s.table[j] >= 0) continue;
    s.table[j] = a->take();
    if (j < nfull)
      a->register_block(s.table[j], s.chain[j], j ? s.chain[j - 1] : pa_allocator::kRootHash,
                        token_ids + j * P, (int32_t)((j + 1) * P));
  }
  int64_t lead = 0;
  while (lead < nfull && hit[lead] >= 0) ++lead;
  s.ntok = num_tokens;
  a->seqs.emplace(seq_id, std::move(s));
  *num_cached_tokens = (int32_t)(lead * P);
  return ok();
}

// One token appended to a sequence made from token ids (see the header).
static pa_status append_token(pa_allocator* a, int64_t seq_id, int32_t token, int64_t* slot_out,
                              int32_t* cow_src, int32_t* cow_dst) {
  const char* fn = "pa_seq_append_tokens";
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return fail(PA_ERR_NOT_FOUND, "%s: unknown sequence %lld", fn, (long long)seq_id);
  auto& s = it->second;
  if (!s.hashed)
    return fail(PA_ERR_INVALID, "%s: sequence %lld was not made from token ids", fn, (long long)seq_id);
  const int32_t P = a->block_size;
  const int64_t L = s.ntok;
  if (L >= INT32_MAX) return fail(PA_ERR_INVALID, "%s: sequence too long", fn);
  const int64_t need = a->blocks_for(L + 1);
  const bool fills = (L + 1) % P == 0;
  uint64_t h = 0, prev = 0;
  std::vector<int32_t> blk;
  int32_t hit = -1;
  if (fills) {
    blk.assign(s.tokens.end() - (P - 1), s.tokens.end());
    blk.push_back(token);
    prev = s.chain.empty() ? pa_allocator::kRootHash : s.chain.back();
    h = a->block_hash(prev, blk.data());
    hit = a->lookup(h, prev, blk.data());
  }
  int32_t src = -1, dst = -1;
  if ((int64_t)s.table.size() < need) {
    if (a->available() == 0) return fail(PA_ERR_NO_BLOCKS, "%s: no free block for a new page", fn);
    a->clock += 1;
    s.table.push_back(a->take());  // holds one token: full only when P == 1
    if (fills) {
      if (hit >= 0) {
        a->release(s.table.back());
        a->share(hit);
        s.table.back() = hit;
      } else {
        a->register_block(s.table.back(), h, prev, blk.data(), (int32_t)(L + 1));
      }
    }
  } else if (a->ref[s.table.back()] > 1) {
    if (hit < 0 && a->available() == 0) return fail(PA_ERR_NO_BLOCKS, "%s: no free block for copy-on-write", fn);
    a->clock += 1;
    const int32_t old = s.table.back();
    if (hit >= 0) {
      a->share(hit);
      a->ref[old] -= 1;  // > 1 before, so still held by another sequence
      s.table.back() = hit;
    } else {
      src = old;
      dst = a->take();
      a->ref[old] -= 1;
      s.table.back() = dst;
      if (fills) a->register_block(dst, h, prev, blk.data(), (int32_t)(L + 1));
    }
  } else {
    a->clock += 1;
    if (fills) {
      if (hit >= 0) {
        a->share(hit);
        a->release(s.table.back());
        s.table.back() = hit;
      } else {
        a->register_block(s.table.back(), h, prev, blk.data(), (int32_t)(L + 1));
      }
    }
  }
  s.tokens.push_back(token);
  if (fills) s.chain.push_back(h);
  s.ntok = (int32_t)(L + 1);
  *slot_out = (int64_t)s.table[L / P] * P + L % P;
  *cow_src = src;
  *cow_dst = dst;
  return ok();
}

pa_status pa_seq_append_tokens(pa_allocator* a, int32_t n, const int64_t* seq_ids, const int32_t* token_ids,
                               int64_t* slots_out, int32_t* cow_pairs_out, int32_t* num_cow_out) {
  if (!a || n < 0 || (n > 0 && (!seq_ids || !token_ids || !slots_out || !cow_pairs_out)) || !num_cow_out)
    return fail(PA_ERR_INVALID, "pa_seq_append_tokens: bad argument");
  if (!a->caching) return fail(PA_ERR_INVALID, "pa_seq_append_tokens: prefix caching is not enabled");
  int32_t ncow = 0;
  *num_cow_out = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t src, dst;
    pa_status st = append_token(a, seq_ids[i], token_ids[i], &slots_out[i], &src, &dst);
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

}  // extern "C"
