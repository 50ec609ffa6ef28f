// Cooperative lanes standing in for GPU threads (kernel emulator for CPU tests only).
//
// Workgroups run one after another.  Inside a workgroup every thread is a
// fiber (ucontext) on one host thread; a fiber runs until it reaches a
// barrier, then the next runnable fiber resumes.  Lanes of one 64-wide
// wavefront meet at a per-wavefront barrier for every cross-lane operation,
// which gives the lockstep behaviour those operations assume.  A lane that
// leaves the kernel drops out of its barriers.  If no fiber can run while some
// are still waiting, a barrier was reached by only part of its lanes (a
// cross-lane operation in divergent code): the emulator aborts and says so.
#include <sanitizer/common_interface_defs.h>
#include <setjmp.h>
#include <ucontext.h>

#include <cstdio>
#include <cstdlib>
#include <memory>
#include <vector>

#include "hip/hip_runtime.h"

namespace emu {

thread_local dim3 tl_threadIdx, tl_blockIdx, tl_blockDim, tl_gridDim;
thread_local int tl_lane;

namespace {

constexpr size_t kStack = 256 * 1024;

struct Barrier {
  int members = 0;   // lanes still in the kernel
  int arrived = 0;
  unsigned phase = 0;
};

struct Wave {
  Barrier bar;
  uint64_t slot[64];
  uint16_t a[64][8], b[64][8];
  float c[64][4];
  float c16[64][16];
};

struct Fiber {
  ucontext_t ctx;      // first entry only
  jmp_buf env;         // where the fiber resumes after it has started
  bool started = false;
  char* stack = nullptr;  // from g_stacks, reused by every workgroup
  dim3 tid;
  int wave = 0;
  bool done = false;
  Barrier* waiting_on = nullptr;
  unsigned waiting_phase = 0;
};

struct Block {
  std::vector<Fiber> fibers;
  std::vector<Wave> waves;
  Barrier bar;
  ucontext_t sched;
  jmp_buf sched_env;  // the scheduler's resumption point (switches use _setjmp/_longjmp: no signal-mask syscall)
  void (*body)(void*) = nullptr;
  void* ctx = nullptr;
  int current = -1;
  const void* sched_stack_bottom = nullptr;
  size_t sched_stack_size = 0;
};

Block* g_block = nullptr;
std::vector<std::unique_ptr<char[]>> g_stacks;  // one per thread slot, kept for the next workgroup

void switch_to_sched(Fiber& f) {
  void* fake = nullptr;
  if (_setjmp(f.env) == 0) {
    __sanitizer_start_switch_fiber(&fake, g_block->sched_stack_bottom, g_block->sched_stack_size);
    _longjmp(g_block->sched_env, 1);
  }
  __sanitizer_finish_switch_fiber(fake, nullptr, nullptr);
}

void set_lane_state(Fiber& f, int index) {
  tl_threadIdx = f.tid;
  tl_lane = index % 64;
}

void arrive(Barrier& b) {
  Fiber& f = g_block->fibers[g_block->current];
  if (++b.arrived == b.members) {
    b.arrived = 0;
    ++b.phase;
    return;
  }
  f.waiting_on = &b;
  f.waiting_phase = b.phase;
  switch_to_sched(f);
  f.waiting_on = nullptr;
  set_lane_state(f, g_block->current);
}

void leave(Barrier& b) {
  --b.members;
  if (b.members > 0 && b.arrived == b.members) {
    b.arrived = 0;
    ++b.phase;
  }
}

void fiber_main(unsigned lo, unsigned hi) {
  // first entry: learn the scheduler's stack (the one this fiber came from)
  __sanitizer_finish_switch_fiber(nullptr, &g_block->sched_stack_bottom, &g_block->sched_stack_size);
  (void)lo;
  (void)hi;
  Block& blk = *g_block;
  Fiber& f = blk.fibers[blk.current];
  set_lane_state(f, blk.current);
  blk.body(blk.ctx);
  Fiber& me = blk.fibers[blk.current];
  me.done = true;
  leave(blk.waves[me.wave].bar);
  leave(blk.bar);
  __sanitizer_start_switch_fiber(nullptr, blk.sched_stack_bottom, blk.sched_stack_size);
  _longjmp(blk.sched_env, 1);
}

Wave& my_wave() { return g_block->waves[g_block->fibers[g_block->current].wave]; }

}  // namespace

void wave_sync() { arrive(my_wave().bar); }

void block_sync() { arrive(g_block->bar); }

uint64_t exchange(uint64_t mine, int src) {
  if (src < 0 || src >= 64) {
    std::fprintf(stderr, "emu: cross-lane read of lane %d\n", src);
    std::abort();
  }
  Wave& w = my_wave();
  const int l = tl_lane;
  w.slot[l] = mine;
  arrive(w.bar);
  const uint64_t r = w.slot[src];
  arrive(w.bar);
  return r;
}

uint64_t ballot(bool pred) {
  Wave& w = my_wave();
  const int l = tl_lane;
  w.slot[l] = pred ? 1 : 0;
  arrive(w.bar);
  uint64_t m = 0;
  for (int k = 0; k < 64; ++k) m |= (w.slot[k] & 1) << k;
  arrive(w.bar);
  return m;
}

static float bf(uint16_t u) {
  uint32_t x = (uint32_t)u << 16;
  float f;
  std::memcpy(&f, &x, 4);
  return f;
}

// D = A(16x32) B(32x16) + C with the lane layout of v_mfma_f32_16x16x32_bf16:
// lane l holds A[l%16][8(l/16)..+8], B[8(l/16)..+8][l%16], D[4(l/16)+i][l%16].
void mfma_16x16x32_bf16(const uint16_t a[8], const uint16_t b[8], const float c[4], float d[4]) {
  Wave& w = my_wave();
  const int l = tl_lane;
  std::memcpy(w.a[l], a, 16);
  std::memcpy(w.b[l], b, 16);
  std::memcpy(w.c[l], c, 16);
  arrive(w.bar);
  const int n = l % 16;
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * (l / 16) + i;
    double acc = 0;
    for (int k = 0; k < 32; ++k) acc += (double)bf(w.a[m + 16 * (k / 8)][k % 8]) * bf(w.b[n + 16 * (k / 8)][k % 8]);
    d[i] = (float)(acc + w.c[l][i]);
  }
  arrive(w.bar);
}

static float hf(uint16_t u) {
  _Float16 h;
  std::memcpy(&h, &u, 2);
  return (float)h;
}

// The same product for IEEE half operands (v_mfma_f32_16x16x32_f16).
void mfma_16x16x32_f16(const uint16_t a[8], const uint16_t b[8], const float c[4], float d[4]) {
  Wave& w = my_wave();
  const int l = tl_lane;
  std::memcpy(w.a[l], a, 16);
  std::memcpy(w.b[l], b, 16);
  std::memcpy(w.c[l], c, 16);
  arrive(w.bar);
  const int n = l % 16;
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * (l / 16) + i;
    double acc = 0;
    for (int k = 0; k < 32; ++k) acc += (double)hf(w.a[m + 16 * (k / 8)][k % 8]) * hf(w.b[n + 16 * (k / 8)][k % 8]);
    d[i] = (float)(acc + w.c[l][i]);
  }
  arrive(w.bar);
}

// D = A(32x16) B(16x32) + C with the lane layout of v_mfma_f32_32x32x16_{bf16,f16}
// (checked on the GPU): lane l holds A[l%32][8(l/32)..+8], B[8(l/32)..+8][l%32],
// D[8(j/4) + 4(l/32) + j%4][l%32] in its accumulator j.
static void mfma_32x32x16(const uint16_t a[8], const uint16_t b[8], const float c[16], float d[16], bool half) {
  Wave& w = my_wave();
  const int l = tl_lane;
  std::memcpy(w.a[l], a, 16);
  std::memcpy(w.b[l], b, 16);
  std::memcpy(w.c16[l], c, 64);
  arrive(w.bar);
  const int n = l % 32;
  for (int j = 0; j < 16; ++j) {
    const int m = 8 * (j / 4) + 4 * (l / 32) + j % 4;
    double acc = 0;
    for (int k = 0; k < 16; ++k) {
      const uint16_t ua = w.a[m + 32 * (k / 8)][k % 8], ub = w.b[n + 32 * (k / 8)][k % 8];
      acc += half ? (double)hf(ua) * hf(ub) : (double)bf(ua) * bf(ub);
    }
    d[j] = (float)(acc + w.c16[l][j]);
  }
  arrive(w.bar);
}

void mfma_32x32x16_bf16(const uint16_t a[8], const uint16_t b[8], const float c[16], float d[16]) {
  mfma_32x32x16(a, b, c, d, false);
}

void mfma_32x32x16_f16(const uint16_t a[8], const uint16_t b[8], const float c[16], float d[16]) {
  mfma_32x32x16(a, b, c, d, true);
}

void run_grid(dim3 grid, dim3 block, void (*body)(void*), void* ctx) {
  const int n = (int)(block.x * block.y * block.z);
  for (unsigned bz = 0; bz < grid.z; ++bz)
    for (unsigned by = 0; by < grid.y; ++by)
      for (unsigned bx = 0; bx < grid.x; ++bx) {
        Block blk;
        blk.body = body;
        blk.ctx = ctx;
        blk.fibers.resize(n);
        blk.waves.resize((n + 63) / 64);
        blk.bar.members = n;
        for (int w = 0; w < (int)blk.waves.size(); ++w) blk.waves[w].bar.members = std::min(64, n - 64 * w);
        tl_blockIdx = dim3(bx, by, bz);
        tl_blockDim = block;
        tl_gridDim = grid;
        g_block = &blk;
        for (int t = 0; t < n; ++t) {
          Fiber& f = blk.fibers[t];
          f.tid = dim3(t % block.x, (t / block.x) % block.y, t / (block.x * block.y));
          f.wave = t / 64;
          if ((int)g_stacks.size() <= t) g_stacks.emplace_back(new char[kStack]);
          f.stack = g_stacks[t].get();
          getcontext(&f.ctx);
          f.ctx.uc_stack.ss_sp = f.stack;
          f.ctx.uc_stack.ss_size = kStack;
          f.ctx.uc_link = nullptr;
          makecontext(&f.ctx, (void (*)())fiber_main, 2, 0u, 0u);
        }
        // round-robin: resume every fiber that is not finished and whose barrier has moved on
        for (;;) {
          bool progressed = false, all_done = true;
          for (int t = 0; t < n; ++t) {
            Fiber& f = blk.fibers[t];
            if (f.done) continue;
            all_done = false;
            if (f.waiting_on && f.waiting_on->phase == f.waiting_phase) continue;
            blk.current = t;
            void* fake = nullptr;
            if (_setjmp(blk.sched_env) == 0) {
              __sanitizer_start_switch_fiber(&fake, f.stack, kStack);
              if (f.started) {
                _longjmp(f.env, 1);
              } else {
                f.started = true;
                swapcontext(&blk.sched, &f.ctx);  // first entry; the fiber comes back by _longjmp
              }
            }
            __sanitizer_finish_switch_fiber(fake, nullptr, nullptr);
            progressed = true;
          }
          if (all_done) break;
          if (!progressed) {
            std::fprintf(stderr, "emu: deadlock in block (%u,%u,%u): lanes wait at a barrier others never reach\n",
                         bx, by, bz);
            std::abort();
          }
        }
        g_block = nullptr;
      }
}

}  // namespace emu
