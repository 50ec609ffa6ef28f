// libpa_probe: measurement kernels that are not part of the attention path.
//
// pa_probe_read_pages reads listed 4 KiB pages with the access pattern of the
// decode workers (whole pages, 16-byte loads, pages in the order of a list)
// and no arithmetic, so that the random page-read rate this GPU attains can be
// set beside the workers' rates.  The number of pages each wavefront keeps in
// flight and the kind of load are parameters, so the same probe maps where
// the read rate saturates.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../../include/pa_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

thread_local char g_err[256];

pa_status probe_fail(pa_status st, const char* msg) {
  int i = 0;
  for (; msg[i] && i < 255; ++i) g_err[i] = msg[i];
  g_err[i] = 0;
  return st;
}

// Wavefront w (of W) reads its pages PIF w .. PIF w + PIF-1, then PIF (w + W) .., all
// PIF pages' 16 loads issued before any is used; lane l XORs 16-byte piece
// l, l+64, l+128, l+192 of every page it reads into one word.  Ids outside the pool
// read page 0 and set bit 1 of the status word.
// MODE 0: plain loads; 1: non-temporal loads (streamed past the caches);
// 2: loads straight into LDS (global_load_lds_dwordx4), read back after a wait;
// kBufferMode + a (a = 0..7): buffer loads through a 4 KiB resource per page with the
// cache-policy bits kCpol[a] (bit 0 SC0, bit 1 NT, bit 4 SC1).
constexpr int kBufferMode = 3;
constexpr int kCpol[8] = {0, 1, 2, 3, 16, 17, 18, 19};

template <int PIF, int MODE>
__global__ __launch_bounds__(256) void read_pages_kernel(const u32x4* __restrict__ pool, int64_t pool_pages,
                                                         const int32_t* __restrict__ page_ids, int32_t n,
                                                         uint32_t* __restrict__ sink, int32_t* dev_status) {
  __shared__ u32x4 lds[MODE == 2 ? 4 * (PIF < 4 ? PIF : 4) * 4 * 64 : 1];  // 4 wavefronts x pages x 4 KiB
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * 4 + wv));
  const int nwaves = (int)gridDim.x * 4;
  u32x4 acc = {0, 0, 0, 0};
  for (int p0 = PIF * wave; p0 < n; p0 += PIF * nwaves) {
    u32x4 v[PIF][4];
    bool have[PIF];
#pragma unroll
    for (int j = 0; j < PIF; ++j) {
      have[j] = p0 + j < n;
      const int64_t id = page_ids[min(p0 + j, n - 1)];
      const bool bad = id < 0 || id >= pool_pages;
      if (__builtin_amdgcn_ballot_w64(bad) && dev_status) atomicOr(dev_status, 1);
      const int64_t page = bad ? 0 : id;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const u32x4* src = pool + page * 256 + k * 64 + lane;
        if constexpr (MODE == 0) {
          v[j][k] = *src;
        } else if constexpr (MODE >= kBufferMode) {
          // a resource of exactly this page: every offset below is inside it
          const __amdgpu_buffer_rsrc_t rs =
              __builtin_amdgcn_make_buffer_rsrc((void*)(pool + page * 256), 0, 4096, 0x00020000);
          v[j][k] = __builtin_amdgcn_raw_buffer_load_b128(rs, (k * 64 + lane) * 16, 0, kCpol[MODE - kBufferMode]);
        } else if constexpr (MODE == 1) {
          v[j][k] = __builtin_nontemporal_load(src);
        } else {
          __builtin_amdgcn_global_load_lds((const void*)src,
                                           (__attribute__((address_space(3))) void*)(lds + ((wv * PIF + j) * 4 + k) * 64),
                                           16, 0, 0);
        }
      }
    }
    if constexpr (MODE == 2) {
      __builtin_amdgcn_s_waitcnt(0);  // this wavefront's loads have landed in its own LDS slice
#pragma unroll
      for (int j = 0; j < PIF; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k) v[j][k] = lds[((wv * PIF + j) * 4 + k) * 64 + lane];
    }
#pragma unroll
    for (int j = 0; j < PIF; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k) acc ^= have[j] ? v[j][k] : u32x4{0, 0, 0, 0};
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

template <int PIF, int MODE>
void launch_mode(dim3 g, hipStream_t s, const u32x4* pool, int64_t pages, const int32_t* ids, int32_t n,
                 uint32_t* sink, int32_t* st) {
  hipLaunchKernelGGL((read_pages_kernel<PIF, MODE>), g, dim3(256), 0, s, pool, pages, ids, n, sink, st);
}

template <int PIF>
void launch(int mode, dim3 g, hipStream_t s, const u32x4* pool, int64_t pages, const int32_t* ids, int32_t n,
            uint32_t* sink, int32_t* st) {
  switch (mode) {
    case 0: launch_mode<PIF, 0>(g, s, pool, pages, ids, n, sink, st); break;
    case 1: launch_mode<PIF, 1>(g, s, pool, pages, ids, n, sink, st); break;
    case 2: launch_mode<PIF, 2>(g, s, pool, pages, ids, n, sink, st); break;
    case kBufferMode + 0: launch_mode<PIF, kBufferMode + 0>(g, s, pool, pages, ids, n, sink, st); break;
    case kBufferMode + 1: launch_mode<PIF, kBufferMode + 1>(g, s, pool, pages, ids, n, sink, st); break;
    case kBufferMode + 2: launch_mode<PIF, kBufferMode + 2>(g, s, pool, pages, ids, n, sink, st); break;
    case kBufferMode + 3: launch_mode<PIF, kBufferMode + 3>(g, s, pool, pages, ids, n, sink, st); break;
    case kBufferMode + 4: launch_mode<PIF, kBufferMode + 4>(g, s, pool, pages, ids, n, sink, st); break;
    case kBufferMode + 5: launch_mode<PIF, kBufferMode + 5>(g, s, pool, pages, ids, n, sink, st); break;
    case kBufferMode + 6: launch_mode<PIF, kBufferMode + 6>(g, s, pool, pages, ids, n, sink, st); break;
    default: launch_mode<PIF, kBufferMode + 7>(g, s, pool, pages, ids, n, sink, st); break;
  }
}

// LDS read rate: WAVES wavefronts per workgroup each read iters x 8 pieces of 16 bytes of a
// 64 KiB LDS array (lane-consecutive addresses, masked into the array), XORed into one word
// per thread written to sink[blockIdx.x * 64 * WAVES + threadIdx.x].
template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void lds_read_kernel(uint32_t* __restrict__ sink, int32_t iters) {
  __shared__ u32x4 buf[4096];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int i = tid; i < 4096; i += 64 * WAVES) buf[i] = u32x4{(uint32_t)i, (uint32_t)i * 3u, (uint32_t)i ^ 5u, 7u};
  __syncthreads();
  u32x4 acc = {0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= buf[((it * 8 + k) * 64 + wv * 512 + lane) & 4095];
  }
  sink[(int64_t)blockIdx.x * 64 * WAVES + tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

void launch8(int mode, dim3 g, hipStream_t s, const u32x4* pool, int64_t pages, const int32_t* ids, int32_t n,
             uint32_t* sink, int32_t* st) {
  if (mode == 0) hipLaunchKernelGGL((read_pages_kernel<8, 0>), g, dim3(256), 0, s, pool, pages, ids, n, sink, st);
  else hipLaunchKernelGGL((read_pages_kernel<8, 1>), g, dim3(256), 0, s, pool, pages, ids, n, sink, st);
}

}  // namespace

extern "C" const char* pa_probe_last_error(void) { return g_err; }

extern "C" pa_status pa_probe_read_pages(const void* pool, int64_t pool_bytes, const int32_t* page_ids,
                                         int32_t num_pages, uint32_t* sink, int32_t grid, int32_t pages_in_flight,
                                         int32_t mode, int32_t* dev_status, void* stream) {
  if (num_pages < 0 || grid <= 0 || pool_bytes < 4096 || pool_bytes % 4096)
    return probe_fail(PA_ERR_INVALID, "pa_probe_read_pages: bad sizes");
  if (mode < 0 || mode > kBufferMode + 7)
    return probe_fail(PA_ERR_INVALID, "pa_probe_read_pages: mode must be 0 .. 10");
  if (pages_in_flight != 1 && pages_in_flight != 2 && pages_in_flight != 4 && pages_in_flight != 8)
    return probe_fail(PA_ERR_INVALID, "pa_probe_read_pages: pages_in_flight must be 1, 2, 4 or 8");
  if (mode == 2 && pages_in_flight > 4)
    return probe_fail(PA_ERR_UNSUPPORTED, "pa_probe_read_pages: loads into LDS hold at most 4 pages per wavefront");
  if (mode >= kBufferMode && pages_in_flight != 4)
    return probe_fail(PA_ERR_UNSUPPORTED, "pa_probe_read_pages: buffer loads run with 4 pages in flight");
  if (num_pages == 0) return PA_OK;
  if (!pool || !page_ids || !sink) return probe_fail(PA_ERR_INVALID, "pa_probe_read_pages: NULL device pointer");
  (void)hipGetLastError();
  const dim3 g(grid);
  hipStream_t s = (hipStream_t)stream;
  const u32x4* p = (const u32x4*)pool;
  const int64_t pages = pool_bytes / 4096;
  switch (pages_in_flight) {
    case 1: launch<1>(mode, g, s, p, pages, page_ids, num_pages, sink, dev_status); break;
    case 2: launch<2>(mode, g, s, p, pages, page_ids, num_pages, sink, dev_status); break;
    case 4: launch<4>(mode, g, s, p, pages, page_ids, num_pages, sink, dev_status); break;
    default: launch8(mode, g, s, p, pages, page_ids, num_pages, sink, dev_status); break;
  }
  if (hipGetLastError() != hipSuccess) return probe_fail(PA_ERR_HIP, "pa_probe_read_pages: launch failed");
  return PA_OK;
}

extern "C" pa_status pa_probe_lds_read(uint32_t* sink, int32_t grid, int32_t waves_per_group, int32_t iters,
                                       void* stream) {
  if (grid <= 0 || iters <= 0 || !sink) return probe_fail(PA_ERR_INVALID, "pa_probe_lds_read: bad arguments");
  (void)hipGetLastError();
  hipStream_t s = (hipStream_t)stream;
  switch (waves_per_group) {
    case 4: hipLaunchKernelGGL(lds_read_kernel<4>, dim3(grid), dim3(256), 0, s, sink, iters); break;
    case 8: hipLaunchKernelGGL(lds_read_kernel<8>, dim3(grid), dim3(512), 0, s, sink, iters); break;
    case 16: hipLaunchKernelGGL(lds_read_kernel<16>, dim3(grid), dim3(1024), 0, s, sink, iters); break;
    default: return probe_fail(PA_ERR_INVALID, "pa_probe_lds_read: waves_per_group must be 4, 8 or 16");
  }
  if (hipGetLastError() != hipSuccess) return probe_fail(PA_ERR_HIP, "pa_probe_lds_read: launch failed");
  return PA_OK;
}
