// Command-line driver of the host allocator for sanitizer runs.
// Reads one operation per line from stdin and prints one result line each:
//   new N P W           -> pa_alloc_create (free order 0..N-1)      prints status
//   order N P W b0 ...  -> pa_alloc_create with an explicit order    prints status
//   create id n         -> pa_seq_create                             prints status
//   fork p c            -> pa_seq_fork                               prints status
//   append id           -> pa_seq_append_slot                        prints status slot src dst
//   free id             -> pa_seq_free                               prints status
//   can n               -> pa_alloc_can_allocate                     prints status answer
//   table id            -> pa_seq_block_table                        prints status n b0 b1 ...
//   nfree               -> pa_alloc_num_free                         prints count
//   caching             -> pa_alloc_enable_prefix_caching            prints status
//   ctok id t0 t1 ...   -> pa_seq_create_tokens                      prints status cached
//   atok id t           -> pa_seq_append_tokens (one sequence)       prints status slot src dst
//   nevict              -> pa_alloc_num_evictable                    prints count
//   stream id k w n     -> pa_seq_create_streaming                   prints status
#include <cstdio>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "pa.h"

int main() {
  pa_allocator* a = nullptr;
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string op;
    in >> op;
    if (op == "new" || op == "order") {
      int n, p;
      double w;
      in >> n >> p >> w;
      std::vector<int32_t> ord;
      int32_t b;
      while (in >> b) ord.push_back(b);
      if (a) pa_alloc_destroy(a);
      a = nullptr;
      std::printf("%d\n", pa_alloc_create(n, p, w, op == "order" ? ord.data() : nullptr, &a));
    } else if (op == "create") {
      long long id;
      int n;
      in >> id >> n;
      std::printf("%d\n", pa_seq_create(a, id, n));
    } else if (op == "fork") {
      long long p, c;
      in >> p >> c;
      std::printf("%d\n", pa_seq_fork(a, p, c));
    } else if (op == "append") {
      long long id;
      in >> id;
      int64_t slot = -1;
      int32_t s = -1, d = -1;
      int st = pa_seq_append_slot(a, id, &slot, &s, &d);
      std::printf("%d %lld %d %d\n", st, (long long)slot, s, d);
    } else if (op == "free") {
      long long id;
      in >> id;
      std::printf("%d\n", pa_seq_free(a, id));
    } else if (op == "can") {
      int n;
      in >> n;
      pa_alloc_status r = PA_ALLOC_NEVER;
      int st = pa_alloc_can_allocate(a, n, &r);
      std::printf("%d %d\n", st, (int)r);
    } else if (op == "table") {
      long long id;
      in >> id;
      int32_t n = 0;
      std::vector<int32_t> buf(4096);
      int st = pa_seq_block_table(a, id, buf.data(), (int32_t)buf.size(), &n);
      std::printf("%d %d", st, st == 0 ? n : 0);
      for (int i = 0; st == 0 && i < n; ++i) std::printf(" %d", buf[i]);
      std::printf("\n");
    } else if (op == "nfree") {
      std::printf("%d\n", pa_alloc_num_free(a));
    } else if (op == "caching") {
      std::printf("%d\n", pa_alloc_enable_prefix_caching(a));
    } else if (op == "ctok") {
      long long id;
      in >> id;
      std::vector<int32_t> toks;
      int32_t t;
      while (in >> t) toks.push_back(t);
      int32_t cached = -1;
      int st = pa_seq_create_tokens(a, id, toks.data(), (int32_t)toks.size(), &cached);
      std::printf("%d %d\n", st, cached);
    } else if (op == "atok") {
      long long id;
      int32_t t;
      in >> id >> t;
      int64_t sid = id, slot = -1;
      int32_t pair[2] = {-1, -1}, ncow = 0;
      int st = pa_seq_append_tokens(a, 1, &sid, &t, &slot, pair, &ncow);
      std::printf("%d %lld %d %d\n", st, (long long)slot, ncow ? pair[0] : -1, ncow ? pair[1] : -1);
    } else if (op == "stream") {
      long long id;
      int k, w, n;
      in >> id >> k >> w >> n;
      std::printf("%d\n", pa_seq_create_streaming(a, id, k, w, n));
    } else if (op == "nevict") {
      std::printf("%d\n", pa_alloc_num_evictable(a));
    }
  }
  if (a) pa_alloc_destroy(a);
  return 0;
}
