// CPU stand-in for <hip/hip_runtime.h> used only by the kernel emulator in
// tests/emu.  It lets the library's own kernel sources compile for x86 and run
// every lane of a wavefront as a host thread, so that address errors show up
// under AddressSanitizer on the CPU instead of as GPU memory faults.
//
// Cross-lane operations (shuffles, readlane, ballot, MFMA) exchange values
// through per-wavefront barriers; __shared__ variables become statics, which
// is correct because workgroups run one at a time.
#pragma once

#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstring>
#include <algorithm>

struct dim3 {
  unsigned x, y, z;
  constexpr dim3(unsigned a = 1, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {}
};

typedef struct emu_stream* hipStream_t;
typedef struct emu_event* hipEvent_t;
typedef int hipError_t;
constexpr hipError_t hipSuccess = 0;
inline hipError_t hipGetLastError() { return hipSuccess; }
inline const char* hipGetErrorString(hipError_t) { return "emulated"; }
inline hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
inline hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
#define HIP_SYMBOL(x) (&(x))
inline hipError_t hipGetSymbolAddress(void** p, const void* sym) { *p = const_cast<void*>(sym); return hipSuccess; }

#define __global__
#define __device__
#define __host__
#define __shared__ static
#define __launch_bounds__(...)
#define __align__(n) __attribute__((aligned(n)))

namespace emu {
extern thread_local dim3 tl_threadIdx, tl_blockIdx, tl_blockDim, tl_gridDim;
extern thread_local int tl_lane;

void wave_sync();
void block_sync();
uint64_t exchange(uint64_t mine, int src_lane);          // value of src_lane
uint64_t ballot(bool pred);
void mfma_16x16x32_bf16(const uint16_t a[8], const uint16_t b[8], const float c[4], float d[4]);
void mfma_16x16x32_f16(const uint16_t a[8], const uint16_t b[8], const float c[4], float d[4]);
void mfma_32x32x16_bf16(const uint16_t a[8], const uint16_t b[8], const float c[16], float d[16]);
void mfma_32x32x16_f16(const uint16_t a[8], const uint16_t b[8], const float c[16], float d[16]);
void run_grid(dim3 grid, dim3 block, void (*body)(void*), void* ctx);

template <typename T>
inline uint64_t to_bits(T v) {
  static_assert(sizeof(T) <= 8, "lane values are at most 64 bits");
  uint64_t u = 0;
  std::memcpy(&u, &v, sizeof(T));
  return u;
}
template <typename T>
inline T from_bits(uint64_t u) {
  T v;
  std::memcpy(&v, &u, sizeof(T));
  return v;
}

template <typename K, typename... A>
struct Launch {
  K k;
  std::tuple<A...> args;
  static void body(void* p) {
    auto* self = static_cast<Launch*>(p);
    std::apply(self->k, self->args);
  }
};

template <typename K, typename... A>
void launch(K k, dim3 g, dim3 b, A... args) {
  Launch<K, A...> l{k, std::tuple<A...>(args...)};
  run_grid(g, b, &Launch<K, A...>::body, &l);
}
}  // namespace emu

#include <tuple>

#define threadIdx (emu::tl_threadIdx)
#define blockIdx (emu::tl_blockIdx)
#define blockDim (emu::tl_blockDim)
#define gridDim (emu::tl_gridDim)

#define hipLaunchKernelGGL(kernel, grid, block, shmem, stream, ...) \
  emu::launch(kernel, dim3(grid), dim3(block), __VA_ARGS__)

using std::max;
using std::min;

inline float __uint_as_float(uint32_t u) { return emu::from_bits<float>(u); }
inline uint32_t __float_as_uint(float f) { return (uint32_t)emu::to_bits(f); }

inline void __syncthreads() { emu::block_sync(); }

template <typename T>
inline T __shfl_xor(T v, int mask, int width = 64) {
  (void)width;
  return emu::from_bits<T>(emu::exchange(emu::to_bits(v), emu::tl_lane ^ mask));
}

// Value of lane (src mod width) of the caller's width-lane segment.
template <typename T>
inline T __shfl(T v, int src, int width = 64) {
  const int lane = (emu::tl_lane & ~(width - 1)) | (src & (width - 1));
  return emu::from_bits<T>(emu::exchange(emu::to_bits(v), lane));
}

template <typename T>
inline T __shfl_up(T v, unsigned delta, int width = 64) {
  (void)width;
  const int src = emu::tl_lane - (int)delta;
  return emu::from_bits<T>(emu::exchange(emu::to_bits(v), src < 0 ? emu::tl_lane : src));
}

inline int atomicAdd(int* p, int v) { return __atomic_fetch_add(p, v, __ATOMIC_SEQ_CST); }
inline unsigned long long atomicAdd(unsigned long long* p, unsigned long long v) {
  return __atomic_fetch_add(p, v, __ATOMIC_SEQ_CST);
}
inline unsigned long long atomicCAS(unsigned long long* p, unsigned long long cmp, unsigned long long val) {
  __atomic_compare_exchange_n(p, &cmp, val, false, __ATOMIC_SEQ_CST, __ATOMIC_SEQ_CST);
  return cmp;  // the old value (cmp is overwritten with it on failure)
}
inline void __threadfence() { __atomic_thread_fence(__ATOMIC_SEQ_CST); }
inline int atomicOr(int* p, int v) { return __atomic_fetch_or(p, v, __ATOMIC_SEQ_CST); }

// The device builtins take and return a 32-bit int: any other argument type is
// converted to int on the way in, as on the device (a float is truncated, not
// reinterpreted), so a kernel that passes a float sees the same result here.
inline int emu_readlane(int v, int lane) {
  return emu::from_bits<int>(emu::exchange(emu::to_bits(v), lane));
}
inline int emu_readfirstlane(int v) { return emu_readlane(v, 0); }
inline uint64_t emu_ballot(bool p) { return emu::ballot(p); }

// v_permlane16_swap / v_permlane32_swap with old = a, src = b: returns
// {first, second} = ([a.R0, b.R0, a.R2, b.R2], [a.R1, b.R1, a.R3, b.R3]) for
// 16-lane rows R, and ([a.lo, b.lo], [a.hi, b.hi]) for 32-lane halves.
typedef uint32_t emu_u32x2 __attribute__((ext_vector_type(2)));
inline emu_u32x2 emu_permlane_swap(uint32_t a, uint32_t b, int width) {
  const int l = emu::tl_lane;
  const bool upper = (l / width) & 1;
  const uint64_t a_src = emu::exchange(a, upper ? l : l + width);   // partner for the second result
  const uint64_t b_src = emu::exchange(b, upper ? l - width : l);   // partner for the first result
  emu_u32x2 r;
  r[0] = upper ? (uint32_t)b_src : a;
  r[1] = upper ? b : (uint32_t)a_src;
  return r;
}
#define __builtin_amdgcn_permlane16_swap(a, b, fi, bc) emu_permlane_swap((a), (b), 16)
#define __builtin_amdgcn_permlane32_swap(a, b, fi, bc) emu_permlane_swap((a), (b), 32)

template <typename V2>
inline float emu_fdot2(V2 a, V2 b, float c, bool) {
  return (float)a[0] * (float)b[0] + (float)a[1] * (float)b[1] + c;
}

template <typename V8, typename F4>
inline F4 emu_mfma(V8 a, V8 b, F4 c, int, int, int) {
  uint16_t ua[8], ub[8];
  float fc[4], fd[4];
  std::memcpy(ua, &a, 16);
  std::memcpy(ub, &b, 16);
  for (int i = 0; i < 4; ++i) fc[i] = c[i];
  emu::mfma_16x16x32_bf16(ua, ub, fc, fd);
  F4 d;
  for (int i = 0; i < 4; ++i) d[i] = fd[i];
  return d;
}

template <typename V8, typename F4>
inline F4 emu_mfma_f16(V8 a, V8 b, F4 c, int, int, int) {
  uint16_t ua[8], ub[8];
  float fc[4], fd[4];
  std::memcpy(ua, &a, 16);
  std::memcpy(ub, &b, 16);
  for (int i = 0; i < 4; ++i) fc[i] = c[i];
  emu::mfma_16x16x32_f16(ua, ub, fc, fd);
  F4 d;
  for (int i = 0; i < 4; ++i) d[i] = fd[i];
  return d;
}

#define __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, x, y, z) emu_mfma_f16((a), (b), (c), (x), (y), (z))

template <typename V8, typename F16>
inline F16 emu_mfma32(V8 a, V8 b, F16 c, bool half) {
  uint16_t ua[8], ub[8];
  float fc[16], fd[16];
  std::memcpy(ua, &a, 16);
  std::memcpy(ub, &b, 16);
  for (int i = 0; i < 16; ++i) fc[i] = c[i];
  if (half) emu::mfma_32x32x16_f16(ua, ub, fc, fd);
  else emu::mfma_32x32x16_bf16(ua, ub, fc, fd);
  F16 d;
  for (int i = 0; i < 16; ++i) d[i] = fd[i];
  return d;
}
#define __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, x, y, z) emu_mfma32((a), (b), (c), false)
#define __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, x, y, z) emu_mfma32((a), (b), (c), true)
#define __builtin_amdgcn_fdot2(a, b, c, cl) emu_fdot2((a), (b), (c), (cl))
// hardware register reads: only XCC_ID (hwreg 20) is used; workgroups go to the eight XCDs in turn
inline int emu_getreg(int) { return (int)(emu::tl_blockIdx.x % 8); }
#define __builtin_amdgcn_s_getreg(r) emu_getreg((r))
#define __builtin_amdgcn_s_setprio(p) ((void)0)
#define __builtin_amdgcn_sched_barrier(m) ((void)0)
#define __HIP_MEMORY_SCOPE_AGENT 3  // the host compiler knows __hip_atomic_load/store, not the macro
#define __builtin_amdgcn_s_waitcnt(x) ((void)(x))
#define __builtin_amdgcn_readlane(v, l) emu_readlane((v), (l))
#define __builtin_amdgcn_readfirstlane(v) emu_readfirstlane((v))
#define __builtin_amdgcn_ballot_w64(p) emu_ballot((p))
#define __builtin_amdgcn_fdot2_f32_bf16(a, b, c, cl) emu_fdot2((a), (b), (c), (cl))
#define __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, x, y, z) emu_mfma((a), (b), (c), (x), (y), (z))
// v_exp_f32: 2^x with results below the smallest normal float flushed to 0
inline float emu_exp2(float x) {
  const float r = std::exp2(x);
  return std::fabs(r) < 1.17549435e-38f ? 0.f : r;
}
#define __builtin_amdgcn_exp2f(x) emu_exp2((x))
#define __builtin_amdgcn_fence(...) ((void)0)
#define __builtin_amdgcn_wave_barrier() emu::wave_sync()
// device queries for launch sizing: a small device (the emulator runs workgroups one at a time)
enum { hipDeviceAttributeMultiprocessorCount = 16 };
inline hipError_t hipDeviceGetAttribute(int* v, int attr, int) {
  *v = attr == hipDeviceAttributeMultiprocessorCount ? 4 : 0;
  return hipSuccess;
}
template <typename F>
inline hipError_t hipOccupancyMaxActiveBlocksPerMultiprocessor(int* n, F, int, size_t) {
  *n = 2;
  return hipSuccess;
}
