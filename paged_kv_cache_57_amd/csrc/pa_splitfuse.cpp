// Dynamic SplitFuse token-budget composer ("DeepSpeed-FastGen 深度解析"
// §3.1-§3.2: split long prompts, fuse short ones, keep every forward pass at
// the same token count; "第 15 章：推理引擎与部署", chunked prefill: decodes
// count one token each and prompt chunks take what is left of the budget).
//
// A pass takes every running decode (one token each, in the order the
// sequences started decoding; those past the budget wait), then prompt chunks
// in arrival order, each min(tokens remaining, budget left), until the budget
// is used.  A prompt whose last chunk ran decodes from the next pass on.  The
// pass lists the chunks first, then the decodes, with each row's query token
// count and the context length after the pass — the query_start_loc /
// context_lens of one pa_forward.
#include <algorithm>
#include <deque>
#include <new>
#include <vector>

#include "pa_internal.h"

struct pa_splitfuse {
  struct Prompt {
    int64_t id;
    int32_t len, done;
  };
  struct Running {
    int64_t id;
    int32_t ctx;
  };
  int32_t budget = 0;
  std::vector<Prompt> queue;
  std::vector<Running> running;

  bool known(int64_t id) const {
    for (const auto& q : queue)
      if (q.id == id) return true;
    for (const auto& r : running)
      if (r.id == id) return true;
    return false;
  }
};

using pa::fail;
using pa::ok;

extern "C" {

pa_status pa_sf_create(int32_t token_budget, pa_splitfuse** out) {
  if (!out) return fail(PA_ERR_INVALID, "pa_sf_create: out is NULL");
  *out = nullptr;
  if (token_budget <= 0) return fail(PA_ERR_INVALID, "pa_sf_create: budget %d must be > 0", token_budget);
  auto* c = new (std::nothrow) pa_splitfuse();
  if (!c) return fail(PA_ERR_INVALID, "pa_sf_create: out of host memory");
  c->budget = token_budget;
  *out = c;
  return ok();
}

void pa_sf_destroy(pa_splitfuse* c) { delete c; }

pa_status pa_sf_add_prompt(pa_splitfuse* c, int64_t seq_id, int32_t prompt_len) {
  if (!c) return fail(PA_ERR_INVALID, "pa_sf_add_prompt: NULL composer");
  if (prompt_len <= 0) return fail(PA_ERR_INVALID, "pa_sf_add_prompt: prompt length %d", prompt_len);
  if (c->known(seq_id)) return fail(PA_ERR_INVALID, "pa_sf_add_prompt: sequence %lld exists", (long long)seq_id);
  c->queue.push_back({seq_id, prompt_len, 0});
  return ok();
}

pa_status pa_sf_finish(pa_splitfuse* c, int64_t seq_id) {
  if (!c) return fail(PA_ERR_INVALID, "pa_sf_finish: NULL composer");
  for (size_t i = 0; i < c->running.size(); ++i)
    if (c->running[i].id == seq_id) {
      c->running.erase(c->running.begin() + i);
      return ok();
    }
  for (size_t i = 0; i < c->queue.size(); ++i)
    if (c->queue[i].id == seq_id) {
      c->queue.erase(c->queue.begin() + i);
      return ok();
    }
  return fail(PA_ERR_NOT_FOUND, "pa_sf_finish: unknown sequence %lld", (long long)seq_id);
}

pa_status pa_sf_step(pa_splitfuse* c, int32_t cap, int64_t* seq_ids, int32_t* q_lens, int32_t* context_lens,
                     int32_t* num_rows_out, int32_t* num_tokens_out) {
  if (!c || !num_rows_out || !num_tokens_out || cap < 0 || (cap > 0 && (!seq_ids || !q_lens || !context_lens)))
    return fail(PA_ERR_INVALID, "pa_sf_step: bad argument");
  // size the pass first, so a too-small output leaves the composer unchanged
  const int32_t nd = (int32_t)std::min<int64_t>((int64_t)c->running.size(), c->budget);
  int64_t left = c->budget - nd;
  int32_t nchunks = 0;
  for (const auto& q : c->queue) {
    if (left == 0) break;
    left -= std::min<int64_t>(q.len - q.done, left);
    ++nchunks;
  }
  *num_rows_out = nchunks + nd;
  if (nchunks + nd > cap)
    return fail(PA_ERR_INVALID, "pa_sf_step: %d rows do not fit a capacity of %d", nchunks + nd, cap);
  left = c->budget - nd;
  int32_t row = 0, tokens = 0;
  std::vector<pa_splitfuse::Running> started;
  size_t qi = 0;
  for (; qi < c->queue.size() && left > 0; ++qi) {
    auto& q = c->queue[qi];
    const int32_t take = (int32_t)std::min<int64_t>(q.len - q.done, left);
    q.done += take;
    left -= take;
    seq_ids[row] = q.id;
    q_lens[row] = take;
    context_lens[row] = q.done;
    ++row;
    tokens += take;
    if (q.done == q.len) started.push_back({q.id, q.len});
  }
  for (int32_t i = 0; i < nd; ++i) {
    auto& r = c->running[i];
    r.ctx += 1;
    seq_ids[row] = r.id;
    q_lens[row] = 1;
    context_lens[row] = r.ctx;
    ++row;
    tokens += 1;
  }
  // prompts whose last chunk ran leave the queue and decode from the next pass on
  c->queue.erase(std::remove_if(c->queue.begin(), c->queue.end(),
                                [](const pa_splitfuse::Prompt& q) { return q.done == q.len; }),
                 c->queue.end());
  c->running.insert(c->running.end(), started.begin(), started.end());
  *num_tokens_out = tokens;
  return ok();
}

}  // extern "C"
