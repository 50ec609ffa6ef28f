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
// 2: loads straight into LDS (global_load_lds_dwordx4), read back after a wait.
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

template <int PIF>
void launch(int mode, dim3 g, hipStream_t s, const u32x4* pool, int64_t pages, const int32_t* ids, int32_t n,
            uint32_t* sink, int32_t* st) {
  if (mode == 0) hipLaunchKernelGGL((read_pages_kernel<PIF, 0>), g, dim3(256), 0, s, pool, pages, ids, n, sink, st);
  else if (mode == 1) hipLaunchKernelGGL((read_pages_kernel<PIF, 1>), g, dim3(256), 0, s, pool, pages, ids, n, sink, st);
  else hipLaunchKernelGGL((read_pages_kernel<PIF, 2>), g, dim3(256), 0, s, pool, pages, ids, n, sink, st);
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
  if (mode < 0 || mode > 2) return probe_fail(PA_ERR_INVALID, "pa_probe_read_pages: mode must be 0, 1 or 2");
  if (pages_in_flight != 1 && pages_in_flight != 2 && pages_in_flight != 4 && pages_in_flight != 8)
    return probe_fail(PA_ERR_INVALID, "pa_probe_read_pages: pages_in_flight must be 1, 2, 4 or 8");
  if (mode == 2 && pages_in_flight > 4)
    return probe_fail(PA_ERR_UNSUPPORTED, "pa_probe_read_pages: loads into LDS hold at most 4 pages per wavefront");
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
