// Device-side types and helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pa.h"

namespace pa {

constexpr int kBlock = 16;  // tokens per page
constexpr int kWave = 64;   // CDNA wavefront width

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

typedef uint16_t bf16_t;  // storage type of one bfloat16

// Element traits: storage type, 16-byte group width X, load/convert helpers.
template <typename T>
struct Elem;

template <>
struct Elem<float> {
  static constexpr int X = 4;  // elements per 16 bytes
  __device__ static inline float to_f32(float v) { return v; }
  __device__ static inline float from_f32(float v) { return v; }
};

template <>
struct Elem<bf16_t> {
  static constexpr int X = 8;
  __device__ static inline float to_f32(bf16_t v) { return __uint_as_float((uint32_t)v << 16); }
  // Round to nearest even, NaN stays NaN (v_cvt_pk_bf16_f32 on gfx950, no branch).
  __device__ static inline bf16_t from_f32(float f) {
    const __bf16 b = (__bf16)f;
    return __builtin_bit_cast(bf16_t, b);
  }
};

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats rounded to bfloat16 and packed (low half = a), one instruction.
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 v = __builtin_convertvector(f32x2{a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

// Two floats rounded to IEEE half (to nearest even) and packed (low half = a).
__device__ inline uint32_t pack_f16x2(float a, float b) {
  const f16x2 v = __builtin_convertvector(f32x2{a, b}, f16x2);
  return __builtin_bit_cast(uint32_t, v);
}

// Low / high bfloat16 of a packed pair, widened to float32 (exact).
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// a.lo*b.lo + a.hi*b.hi + c on two packed bfloat16 pairs (v_dot2_f32_bf16).
// The pairs arrive as 32-bit words copied into locals: a bit cast applied
// directly to an element of a vector-typed value reinterprets the vector's
// first word instead of the element, so only plain scalars are cast here.
__device__ inline float dot2_bf16(uint32_t a, uint32_t b, float c) {
  const uint32_t ua = a, ub = b;
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ua), __builtin_bit_cast(bf16x2, ub), c,
                                         false);
}

__device__ inline u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// 16 / 8 bytes loaded with the non-temporal hint: for data read once per pass
// (a decode row's key and value pages), which streams through the caches
// without displacing what is reused; random 4 KiB page reads reach a higher
// HBM rate this way on gfx950.
__device__ inline u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ inline u32x2 ld8_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}

// A KV page load: non-temporal when each page of the pass is read once (kStream),
// plain when other sequences of the same pass read the same pages, so that their
// reads can hit in L2 or the Infinity Cache.
template <bool kStream>
__device__ inline u32x4 ld16_page(const void* p) {
  if constexpr (kStream) return ld16_stream(p);
  else return ld16(p);
}
template <bool kStream>
__device__ inline u32x2 ld8_page(const void* p) {
  if constexpr (kStream) return ld8_stream(p);
  else return *reinterpret_cast<const u32x2*>(p);
}

__device__ inline void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// One word stored / loaded coherently for the whole GPU (relaxed, agent scope): the
// instruction itself carries the scope bit, so values handed between workgroups of one
// dispatch that run on different XCDs (each with its own L2) need no fence that writes
// back or invalidates a whole L2.  Ordering is the caller's: see wait_stores.
__device__ inline void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float ld_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until every store this wavefront has issued is acknowledged (s_waitcnt with all
// counts zero): an agent-scope store is then visible to the whole GPU.  The signal fences
// keep the compiler from moving memory accesses across the wait.
__device__ inline void wait_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Lane `lane`'s value of v (lane wave-uniform).  The builtin works on 32-bit
// integers, so a float travels as its bit pattern (a plain call would convert
// the value to an integer and back).
__device__ inline int readlane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }
__device__ inline float readlane(float v, int lane) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), lane));
}

__device__ inline float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, kWave); }

// 2^x with one v_exp_f32.  Results below 2^-126 come out as 0 (exp2f spends
// five more instructions to produce them as denormals); softmax weights that
// small relative to the running maximum contribute nothing measurable.
// 2^-inf = 0, 2^NaN = NaN.
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max / sum over the four 16-lane rows of a wavefront: every lane gets the
// result for lanes l%16, l%16 + 16, l%16 + 32, l%16 + 48.  Two VALU lane
// swaps (v_permlane16_swap: rows 0,1 and 2,3; v_permlane32_swap: halves)
// instead of two exchanges through LDS.  Called with the same value in both
// operands, a swap returns the two partners' values in its two results, so
// every lane combines the same two values in the same order.
__device__ inline float max_over_rows(float v) {
  typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
  u32x2v s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
  s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ inline float sum_over_rows(float v) {
  typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
  u32x2v s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(s[0]) + __uint_as_float(s[1]);
  s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Scalar broadcast of lane 0's value (the compiler keeps the result uniform).
__device__ inline int first_lane(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ inline void flag_status(int32_t* dev_status, int bits) {
  if (dev_status) atomicOr(dev_status, bits);
}

}  // namespace pa
