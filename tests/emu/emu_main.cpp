// Runs libpa's C-ABI entry points with the emulated kernels on host memory.
// Every buffer is a separate exact-size heap allocation, so AddressSanitizer
// reports any access outside it with the kernel source line.
//
//   emu_main forward <in> <out>   in: i32 dtype,S,T,max_q_len,max_ctx,Hq,Hkv,D,NB,mbps; f32 scale;
//                                     q, k_cache, v_cache (element bytes by dtype),
//                                     i32 block_tables[S*mbps], context_lens[S], qsl[S+1]
//                                 out: output [T*Hq*D] then i32 status
//   emu_main reshape <in> <out>   in: i32 dtype,T,NB,Hkv,D; key, value, k_cache, v_cache; i64 slots[T]
//                                 out: k_cache, v_cache, i32 status
//   emu_main copy <in> <out>      in: i32 dtype,P,NB,Hkv,D; k_cache, v_cache; i32 pairs[2P]
//                                 out: k_cache, v_cache, i32 status
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "pa.h"

namespace {

FILE* fin;
FILE* fout;

int32_t rd_i32() {
  int32_t v;
  if (std::fread(&v, 4, 1, fin) != 1) std::abort();
  return v;
}
float rd_f32() {
  float v;
  if (std::fread(&v, 4, 1, fin) != 1) std::abort();
  return v;
}
// exact-size allocation so that any overrun is caught
void* rd_buf(size_t bytes) {
  void* p = std::malloc(bytes ? bytes : 1);
  if (bytes && std::fread(p, 1, bytes, fin) != bytes) std::abort();
  return p;
}
void wr(const void* p, size_t bytes) { std::fwrite(p, 1, bytes, fout); }

}  // namespace

int main(int argc, char** argv) {
  if (argc != 4) return 2;
  fin = std::fopen(argv[2], "rb");
  fout = std::fopen(argv[3], "wb");
  if (!fin || !fout) return 2;
  int32_t status = 0;
  if (!std::strcmp(argv[1], "forward_sparse")) {
    // Same as forward, but the pools are described by the blocks the tables use:
    // i32 nused, i32 ids[nused], then the K pages and the V pages of those blocks.
    // The full pools are allocated zeroed at their real size (large pools test
    // 64-bit page offsets) and only the given blocks are filled in.
    const int dt = rd_i32(), S = rd_i32(), T = rd_i32(), mq = rd_i32(), mc = rd_i32();
    const int Hq = rd_i32(), Hkv = rd_i32(), D = rd_i32(), NB = rd_i32(), mbps = rd_i32();
    const float scale = rd_f32();
    const size_t es = dt == PA_F32 ? 4 : 2;
    const size_t page = (size_t)Hkv * 16 * D * es;
    void* q = rd_buf((size_t)T * Hq * D * es);
    const int nused = rd_i32();
    auto* ids = (int32_t*)rd_buf((size_t)nused * 4);
    auto* kc = (char*)std::calloc((size_t)NB * page, 1);
    auto* vc = (char*)std::calloc((size_t)NB * page, 1);
    if (!kc || !vc) return 4;
    for (int i = 0; i < nused; ++i)
      if (std::fread(kc + (size_t)ids[i] * page, 1, page, fin) != page) std::abort();
    for (int i = 0; i < nused; ++i)
      if (std::fread(vc + (size_t)ids[i] * page, 1, page, fin) != page) std::abort();
    auto* tab = (int32_t*)rd_buf((size_t)S * mbps * 4);
    auto* lens = (int32_t*)rd_buf((size_t)S * 4);
    auto* qsl = (int32_t*)rd_buf((size_t)(S + 1) * 4);
    void* out = std::malloc((size_t)T * Hq * D * es);
    const size_t wsb = pa_forward_workspace_bytes(S, T, mq, Hq, Hkv, D, mc, (pa_dtype)dt);
    void* ws = std::aligned_alloc(256, wsb);
    pa_status st = pa_forward(out, q, kc, vc, tab, mbps, lens, qsl, S, T, mq, mc, Hq, Hkv, D, 16, NB,
                              scale, (pa_dtype)dt, ws, wsb, &status, nullptr);
    if (st != PA_OK) {
      std::fprintf(stderr, "pa_forward: %d %s\n", st, pa_last_error());
      return 3;
    }
    wr(out, (size_t)T * Hq * D * es);
    std::free(ws); std::free(out); std::free(q); std::free(ids); std::free(kc); std::free(vc);
    std::free(tab); std::free(lens); std::free(qsl);
  } else if (!std::strcmp(argv[1], "forward")) {
    const int dt = rd_i32(), S = rd_i32(), T = rd_i32(), mq = rd_i32(), mc = rd_i32();
    const int Hq = rd_i32(), Hkv = rd_i32(), D = rd_i32(), NB = rd_i32(), mbps = rd_i32();
    const float scale = rd_f32();
    const size_t es = dt == PA_F32 ? 4 : 2;
    void* q = rd_buf((size_t)T * Hq * D * es);
    void* kc = rd_buf((size_t)NB * Hkv * 16 * D * es);
    void* vc = rd_buf((size_t)NB * Hkv * 16 * D * es);
    auto* tab = (int32_t*)rd_buf((size_t)S * mbps * 4);
    auto* lens = (int32_t*)rd_buf((size_t)S * 4);
    auto* qsl = (int32_t*)rd_buf((size_t)(S + 1) * 4);
    void* out = std::malloc((size_t)T * Hq * D * es);
    std::memset(out, 0xff, (size_t)T * Hq * D * es);
    const size_t wsb = pa_forward_workspace_bytes(S, T, mq, Hq, Hkv, D, mc, (pa_dtype)dt);
    void* ws = std::aligned_alloc(256, wsb);
    std::memset(ws, 0xa5, wsb);
    pa_status st = pa_forward(out, q, kc, vc, tab, mbps, lens, qsl, S, T, mq, mc, Hq, Hkv, D, 16, NB,
                              scale, (pa_dtype)dt, ws, wsb, &status, nullptr);
    if (st != PA_OK) {
      std::fprintf(stderr, "pa_forward: %d %s\n", st, pa_last_error());
      return 3;
    }
    wr(out, (size_t)T * Hq * D * es);
    std::free(ws);
    std::free(out);
    std::free(q); std::free(kc); std::free(vc); std::free(tab); std::free(lens); std::free(qsl);
  } else if (!std::strcmp(argv[1], "forward_shared")) {
    // forward, then i32 num_groups and the groups [num_groups][3]
    const int dt = rd_i32(), S = rd_i32(), T = rd_i32(), mq = rd_i32(), mc = rd_i32();
    const int Hq = rd_i32(), Hkv = rd_i32(), D = rd_i32(), NB = rd_i32(), mbps = rd_i32();
    const float scale = rd_f32();
    const size_t es = dt == PA_F32 ? 4 : 2;
    void* q = rd_buf((size_t)T * Hq * D * es);
    void* kc = rd_buf((size_t)NB * Hkv * 16 * D * es);
    void* vc = rd_buf((size_t)NB * Hkv * 16 * D * es);
    auto* tab = (int32_t*)rd_buf((size_t)S * mbps * 4);
    auto* lens = (int32_t*)rd_buf((size_t)S * 4);
    auto* qsl = (int32_t*)rd_buf((size_t)(S + 1) * 4);
    const int NG = rd_i32();
    auto* groups = (int32_t*)rd_buf((size_t)NG * 12);
    void* out = std::malloc((size_t)T * Hq * D * es);
    std::memset(out, 0xff, (size_t)T * Hq * D * es);
    const size_t wsb = pa_forward_shared_workspace_bytes(S, NG, T, mq, Hq, Hkv, D, mc, (pa_dtype)dt);
    void* ws = std::aligned_alloc(256, wsb);
    std::memset(ws, 0xa5, wsb);
    pa_status st = pa_forward_shared(out, q, kc, vc, tab, mbps, lens, qsl, NG ? groups : nullptr, NG, S, T, mq, mc,
                                     Hq, Hkv, D, 16, NB, scale, (pa_dtype)dt, ws, wsb, &status, nullptr);
    if (st != PA_OK) {
      std::fprintf(stderr, "pa_forward_shared: %d %s\n", st, pa_last_error());
      return 3;
    }
    wr(out, (size_t)T * Hq * D * es);
    std::free(ws);
    std::free(out);
    std::free(q); std::free(kc); std::free(vc); std::free(tab); std::free(lens); std::free(qsl); std::free(groups);
  } else if (!std::strcmp(argv[1], "reshape")) {
    const int dt = rd_i32(), T = rd_i32(), NB = rd_i32(), Hkv = rd_i32(), D = rd_i32();
    const size_t es = dt == PA_F32 ? 4 : 2;
    void* key = rd_buf((size_t)T * Hkv * D * es);
    void* val = rd_buf((size_t)T * Hkv * D * es);
    const size_t pool = (size_t)NB * Hkv * 16 * D * es;
    void* kc = rd_buf(pool);
    void* vc = rd_buf(pool);
    auto* slots = (int64_t*)rd_buf((size_t)T * 8);
    pa_status st = pa_reshape_and_cache(key, val, kc, vc, slots, T, NB, Hkv, D, 16, (pa_dtype)dt, &status, nullptr);
    if (st != PA_OK) {
      std::fprintf(stderr, "pa_reshape_and_cache: %d %s\n", st, pa_last_error());
      return 3;
    }
    wr(kc, pool);
    wr(vc, pool);
    std::free(key); std::free(val); std::free(kc); std::free(vc); std::free(slots);
  } else if (!std::strcmp(argv[1], "copy")) {
    const int dt = rd_i32(), P = rd_i32(), NB = rd_i32(), Hkv = rd_i32(), D = rd_i32();
    const size_t es = dt == PA_F32 ? 4 : 2;
    const size_t pool = (size_t)NB * Hkv * 16 * D * es;
    void* kc = rd_buf(pool);
    void* vc = rd_buf(pool);
    auto* pairs = (int32_t*)rd_buf((size_t)P * 8);
    pa_status st = pa_copy_blocks(kc, vc, pairs, P, NB, Hkv, D, 16, (pa_dtype)dt, &status, nullptr);
    if (st != PA_OK) {
      std::fprintf(stderr, "pa_copy_blocks: %d %s\n", st, pa_last_error());
      return 3;
    }
    wr(kc, pool);
    wr(vc, pool);
    std::free(kc); std::free(vc); std::free(pairs);
  } else if (!std::strcmp(argv[1], "rope")) {
    const int dt = rd_i32(), T = rd_i32(), Hq = rd_i32(), Hkv = rd_i32(), D = rd_i32(), NB = rd_i32();
    const int maxpos = rd_i32();
    const size_t es = dt == PA_F32 ? 4 : 2;
    void* q = rd_buf((size_t)T * Hq * D * es);
    void* key = rd_buf((size_t)T * Hkv * D * es);
    void* val = rd_buf((size_t)T * Hkv * D * es);
    const size_t pool = (size_t)NB * Hkv * 16 * D * es;
    void* kc = rd_buf(pool);
    void* vc = rd_buf(pool);
    auto* slots = (int64_t*)rd_buf((size_t)T * 8);
    auto* pos = (int32_t*)rd_buf((size_t)T * 4);
    auto* cs = (float*)rd_buf((size_t)maxpos * (D / 2) * 4);
    auto* sn = (float*)rd_buf((size_t)maxpos * (D / 2) * 4);
    pa_status st = pa_rope_reshape_and_cache(q, q, key, val, kc, vc, slots, pos, cs, sn, maxpos, T, Hq, Hkv, NB, D,
                                             16, (pa_dtype)dt, &status, nullptr);
    if (st != PA_OK) {
      std::fprintf(stderr, "pa_rope_reshape_and_cache: %d %s\n", st, pa_last_error());
      return 3;
    }
    wr(q, (size_t)T * Hq * D * es);
    wr(kc, pool);
    wr(vc, pool);
    std::free(q); std::free(key); std::free(val); std::free(kc); std::free(vc); std::free(slots);
    std::free(pos); std::free(cs); std::free(sn);
  } else {
    return 2;
  }
  wr(&status, 4);
  std::fclose(fout);
  std::fclose(fin);
  return 0;
}
