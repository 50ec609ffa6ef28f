// Cache write through a slot mapping and copy-on-write page copies (gfx950).
//
// Both are pure data movement: exact byte copies, no arithmetic on values.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

// Workgroup (i, h) moves new tokens 16i .. 16i+15 of KV head h; thread (j, c) =
// (tid % 16, tid / 16) takes token 16i + j's 16-byte group c of the key row
// and of the value row.  Lanes that share c write their tokens' page offsets
// side by side, so a run of tokens that fills a page in order (a prefill
// chunk) leaves every value store instruction with whole 32-byte runs (16
// tokens of one column) and every key store with a 256-byte run, and all of
// a page's bytes pass through one L2 (a page split over several L2s would be
// written back in pieces).  A token alone in its page (a decode step) still
// writes one element per value column: the value page keeps each column's 16
// tokens together for the attention kernels' operand loads.
template <typename T, int D>
__global__ __launch_bounds__(512) void reshape_and_cache_kernel(
    const T* __restrict__ key, const T* __restrict__ value, T* __restrict__ k_cache,
    T* __restrict__ v_cache, const int64_t* __restrict__ slot_mapping, int32_t num_tokens, int32_t num_blocks,
    int32_t num_kv_heads, int32_t* dev_status) {
  constexpr int X = Elem<T>::X;  // elements per 16 bytes; blockDim.x = 16 D / X
  const int j = threadIdx.x & 15, c = threadIdx.x >> 4;
  const int h = blockIdx.y;
  const int t = blockIdx.x * kBlock + j;
  if (t >= num_tokens) return;  // the last group's missing tokens (no barrier follows)
  const int64_t slot = slot_mapping[t];
  if (slot < 0) return;  // padding token
  if (slot >= (int64_t)num_blocks * kBlock) {
    if (c == 0 && h == 0) flag_status(dev_status, PA_DEV_BAD_SLOT);
    return;
  }
  const int64_t b = slot / kBlock;
  const int o = (int)(slot % kBlock);
  const int64_t src = ((int64_t)t * num_kv_heads + h) * D + c * X;
  const int64_t page = (b * num_kv_heads + h) * (int64_t)(kBlock * D);
  // key: 16-byte run c of token o
  st16(k_cache + page + ((int64_t)c * kBlock + o) * X, ld16(key + src));
  // value: X consecutive columns of token o
  union {
    u32x4 v;
    T e[X];
  } u;
  u.v = ld16(value + src);
#pragma unroll
  for (int x = 0; x < X; ++x) v_cache[page + (int64_t)(c * X + x) * kBlock + o] = u.e[x];
}

// Rotary embedding fused with the cache write.  Workgroup (i, y) takes new
// tokens 16i .. 16i+15 and head y: query head y < num_q_heads, else KV head
// y - num_q_heads.  Thread (j, c) takes token 16i + j's unit c < head_dim/(2X):
// 16-byte group c together with its partner group c + head_dim/(2X), which
// hold the pairs (i, i + d/2) that one rotation mixes.  A query unit rotates q
// into q_out (which may be q: every element is read and written by the same
// thread); a key unit rotates the key, stores both groups into the page and
// copies the same two value groups, with the page-offset layout of the plain
// cache write above.  Rotation in float32: x' = x c − y s, y' = y c + x s,
// each with one rounded product and one fused multiply-add, then rounded to T.
template <typename T, int D>
__global__ __launch_bounds__(256) void rope_cache_kernel(
    T* q_out, const T* q, const T* __restrict__ key, const T* __restrict__ value, T* __restrict__ k_cache,
    T* __restrict__ v_cache, const int64_t* __restrict__ slot_mapping, const int32_t* __restrict__ positions,
    const float* __restrict__ cos_t, const float* __restrict__ sin_t, int32_t max_position, int32_t num_tokens,
    int32_t num_blocks, int32_t num_q_heads, int32_t num_kv_heads, int32_t* dev_status) {
  constexpr int X = Elem<T>::X;
  constexpr int HC = D / X / 2;  // units per head; blockDim.x = 16 HC
  const int j = threadIdx.x & 15, c = threadIdx.x >> 4;
  const int y = blockIdx.y;
  const int t = blockIdx.x * kBlock + j;
  if (t >= num_tokens) return;  // the last group's missing tokens (no barrier follows)
  const int pos = positions[t];
  if (pos < 0 || pos >= max_position) {
    if (c == 0 && y == 0) flag_status(dev_status, PA_DEV_BAD_POSITION);
    return;
  }
  const bool isq = y < num_q_heads;
  const int h = isq ? y : y - num_q_heads;
  int64_t b = 0;
  int o = 0;
  if (!isq) {
    const int64_t slot = slot_mapping[t];
    if (slot >= (int64_t)num_blocks * kBlock) {
      if (c == 0 && h == 0) flag_status(dev_status, PA_DEV_BAD_SLOT);
      return;
    }
    if (slot < 0) return;  // padding token: nothing to store
    b = slot / kBlock;
    o = (int)(slot % kBlock);
  }
  const float* crow = cos_t + (int64_t)pos * (D / 2);
  const float* srow = sin_t + (int64_t)pos * (D / 2);
  const int64_t src = ((int64_t)t * (isq ? num_q_heads : num_kv_heads) + h) * D + c * X;
  const T* in = isq ? q : key;
  union Grp {
    u32x4 v;
    T e[X];
  } lo, hi;
  lo.v = ld16(in + src);
  hi.v = ld16(in + src + D / 2);
#pragma unroll
  for (int x = 0; x < X; ++x) {
    const float cs = crow[c * X + x], sn = srow[c * X + x];
    const float a = Elem<T>::to_f32(lo.e[x]), bb = Elem<T>::to_f32(hi.e[x]);
    const float bs = bb * sn, as = a * sn;
    lo.e[x] = Elem<T>::from_f32(__builtin_fmaf(a, cs, -bs));
    hi.e[x] = Elem<T>::from_f32(__builtin_fmaf(bb, cs, as));
  }
  if (isq) {
    st16(q_out + src, lo.v);
    st16(q_out + src + D / 2, hi.v);
  } else {
    const int64_t page = (b * num_kv_heads + h) * (int64_t)(kBlock * D);
    st16(k_cache + page + ((int64_t)c * kBlock + o) * X, lo.v);
    st16(k_cache + page + ((int64_t)(c + HC) * kBlock + o) * X, hi.v);
    Grp v0, v1;
    v0.v = ld16(value + src);
    v1.v = ld16(value + src + D / 2);
#pragma unroll
    for (int x = 0; x < X; ++x) {
      v_cache[page + (int64_t)(c * X + x) * kBlock + o] = v0.e[x];
      v_cache[page + (int64_t)(D / 2 + c * X + x) * kBlock + o] = v1.e[x];
    }
  }
}

// grid (num_pairs, slices): each workgroup copies one 4 KiB slice of the key
// page and of the value page of one (src, dst) pair.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint8_t* __restrict__ k_cache,
                                                          uint8_t* __restrict__ v_cache,
                                                          const int32_t* __restrict__ pairs,
                                                          int32_t num_blocks, int64_t page_bytes,
                                                          int32_t* dev_status) {
  const int i = blockIdx.x;
  const int32_t src = pairs[2 * i], dst = pairs[2 * i + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) {
    if (threadIdx.x == 0 && blockIdx.y == 0) flag_status(dev_status, PA_DEV_BAD_BLOCK);
    return;
  }
  const int64_t off = (int64_t)blockIdx.y * 4096 + (int64_t)threadIdx.x * 16;
  if (off >= page_bytes) return;
  const int64_t s = (int64_t)src * page_bytes + off, d = (int64_t)dst * page_bytes + off;
  st16(k_cache + d, ld16(k_cache + s));
  st16(v_cache + d, ld16(v_cache + s));
}

pa_status check_pool_args(const char* fn, int32_t num_blocks, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, pa_dtype dtype) {
  if (num_blocks <= 0 || num_kv_heads <= 0)
    return fail(PA_ERR_INVALID, "%s: num_blocks %d and num_kv_heads %d must be > 0", fn,
                num_blocks, num_kv_heads);
  if (block_size != kBlock)
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d (only 16 is supported)", fn, block_size);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d (64 or 128 supported)", fn, head_dim);
  if (dtype != PA_F32 && dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "%s: dtype %d", fn, (int)dtype);
  return PA_OK;
}

template <typename T, int D>
void launch_reshape(const void* key, const void* value, void* k_cache, void* v_cache,
                    const int64_t* slots, int32_t T_, int32_t nb, int32_t hkv, int32_t* st,
                    hipStream_t stream) {
  hipLaunchKernelGGL((reshape_and_cache_kernel<T, D>), dim3((T_ + kBlock - 1) / kBlock, hkv),
                     dim3(kBlock * (D / Elem<T>::X)), 0, stream, (const T*)key, (const T*)value, (T*)k_cache,
                     (T*)v_cache, slots, T_, nb, hkv, st);
}

}  // namespace
}  // namespace pa

using namespace pa;

extern "C" pa_status pa_rope_reshape_and_cache(void* q_out, const void* q, const void* key, const void* value,
                                               void* k_cache, void* v_cache, const int64_t* slot_mapping,
                                               const int32_t* positions, const float* cos_table,
                                               const float* sin_table, int32_t max_position, int32_t num_tokens,
                                               int32_t num_q_heads, int32_t num_kv_heads, int32_t num_blocks,
                                               int32_t head_dim, int32_t block_size, pa_dtype dtype,
                                               int32_t* dev_status, void* stream) {
  const char* fn = "pa_rope_reshape_and_cache";
  pa_status st = check_pool_args(fn, num_blocks, num_kv_heads, head_dim, block_size, dtype);
  if (st != PA_OK) return st;
  if (num_tokens < 0 || num_q_heads <= 0 || max_position <= 0)
    return fail(PA_ERR_INVALID, "%s: num_tokens %d, num_q_heads %d, max_position %d", fn, num_tokens,
                num_q_heads, max_position);
  if (num_tokens == 0) return ok();
  if (num_tokens > 2147483647 / 2 || (int64_t)num_q_heads * head_dim > (1 << 24) ||
      (int64_t)num_q_heads + num_kv_heads > 65535)
    return fail(PA_ERR_INVALID, "%s: too large", fn);
  if (!q_out || !q || !key || !value || !k_cache || !v_cache || !slot_mapping || !positions || !cos_table ||
      !sin_table)
    return fail(PA_ERR_INVALID, "%s: NULL device pointer", fn);
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
#define PA_ROPE_LAUNCH(T, D)                                                                                   \
  hipLaunchKernelGGL((rope_cache_kernel<T, D>), dim3((num_tokens + kBlock - 1) / kBlock, num_q_heads + num_kv_heads), \
                     dim3(kBlock * (D / Elem<T>::X / 2)), 0, s, (T*)q_out, (const T*)q, (const T*)key,           \
                     (const T*)value, (T*)k_cache, (T*)v_cache, slot_mapping, positions, cos_table, sin_table,  \
                     max_position, num_tokens, num_blocks, num_q_heads, num_kv_heads, dev_status)
  if (dtype == PA_BF16) {
    if (head_dim == 64) PA_ROPE_LAUNCH(bf16_t, 64);
    else PA_ROPE_LAUNCH(bf16_t, 128);
  } else {
    if (head_dim == 64) PA_ROPE_LAUNCH(float, 64);
    else PA_ROPE_LAUNCH(float, 128);
  }
#undef PA_ROPE_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

extern "C" pa_status pa_reshape_and_cache(const void* key, const void* value, void* k_cache,
                                          void* v_cache, const int64_t* slot_mapping,
                                          int32_t num_tokens, int32_t num_blocks,
                                          int32_t num_kv_heads, int32_t head_dim,
                                          int32_t block_size, pa_dtype dtype, int32_t* dev_status,
                                          void* stream) {
  const char* fn = "pa_reshape_and_cache";
  pa_status st = check_pool_args(fn, num_blocks, num_kv_heads, head_dim, block_size, dtype);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return fail(PA_ERR_INVALID, "%s: negative num_tokens", fn);
  if (num_kv_heads > 65535) return fail(PA_ERR_INVALID, "%s: num_kv_heads %d (at most 65535)", fn, num_kv_heads);
  if (num_tokens == 0) return ok();
  if (!key || !value || !k_cache || !v_cache || !slot_mapping)
    return fail(PA_ERR_INVALID, "%s: NULL device pointer", fn);
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  if (dtype == PA_F32) {
    if (head_dim == 64)
      launch_reshape<float, 64>(key, value, k_cache, v_cache, slot_mapping, num_tokens, num_blocks, num_kv_heads, dev_status, s);
    else
      launch_reshape<float, 128>(key, value, k_cache, v_cache, slot_mapping, num_tokens, num_blocks, num_kv_heads, dev_status, s);
  } else {
    if (head_dim == 64)
      launch_reshape<bf16_t, 64>(key, value, k_cache, v_cache, slot_mapping, num_tokens, num_blocks, num_kv_heads, dev_status, s);
    else
      launch_reshape<bf16_t, 128>(key, value, k_cache, v_cache, slot_mapping, num_tokens, num_blocks, num_kv_heads, dev_status, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

extern "C" pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs,
                                    int32_t num_pairs, int32_t num_blocks, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size, pa_dtype dtype,
                                    int32_t* dev_status, void* stream) {
  const char* fn = "pa_copy_blocks";
  pa_status st = check_pool_args(fn, num_blocks, num_kv_heads, head_dim, block_size, dtype);
  if (st != PA_OK) return st;
  if (num_pairs < 0) return fail(PA_ERR_INVALID, "%s: negative num_pairs", fn);
  if (num_pairs == 0) return ok();
  if (!k_cache || !v_cache || !block_pairs) return fail(PA_ERR_INVALID, "%s: NULL device pointer", fn);
  if (num_pairs > 65535 * 64) return fail(PA_ERR_INVALID, "%s: too many pairs", fn);
  const int64_t page_bytes =
      (int64_t)num_kv_heads * kBlock * head_dim * (dtype == PA_F32 ? 4 : 2);
  const int slices = (int)((page_bytes + 4095) / 4096);
  if (slices > 65535) return fail(PA_ERR_INVALID, "%s: page too large", fn);
  (void)hipGetLastError();
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, slices), dim3(256), 0, (hipStream_t)stream,
                     (uint8_t*)k_cache, (uint8_t*)v_cache, block_pairs, num_blocks, page_bytes,
                     dev_status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}
