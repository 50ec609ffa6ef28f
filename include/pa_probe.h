/* pa_probe.h — measurement-only entry points (libpa_probe.so), not part of the
 * attention path: they calibrate what the GPU attains for the access pattern
 * of the decode workers, so the workers' rates can be set beside it. */
#ifndef PA_PROBE_H
#define PA_PROBE_H

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads every byte of the listed 4096-byte pages of `pool` with 16-byte
 * loads: wavefront w of W reads pages pages_in_flight*w .. +pages_in_flight-1,
 * then the same run pages_in_flight*W further on, and so on, issuing all loads
 * of its pages_in_flight pages before using any; thread l of wavefront w writes
 * to sink[64w + l] the XOR of 16-byte pieces l, l+64, l+128, l+192 of every page
 * it read, folded to one word (so nothing is optimised away).
 *   pool             device, pool_bytes bytes (a multiple of 4096)
 *   page_ids         device, int32 [num_pages]; ids outside the pool read page 0
 *                    and set bit 1 of *dev_status (device, may be NULL)
 *   sink             device, uint32 [grid * 256]
 *   grid             workgroups of 4 wavefronts
 *   pages_in_flight  1, 2, 4 or 8 pages per wavefront at a time
 *   mode             0 plain loads, 1 non-temporal loads, 2 loads into LDS
 *                    (at most 4 pages in flight); 3 + a for a = 0..7: buffer
 *                    loads through a 4096-byte resource per page with the
 *                    cache-policy bits {0, 1, 2, 3, 16, 17, 18, 19}[a] (bit 0
 *                    SC0, bit 1 NT, bit 4 SC1; 4 pages in flight only)
 * Errors: PA_ERR_INVALID / PA_ERR_UNSUPPORTED for bad arguments (nothing is
 * launched), PA_ERR_HIP for a failed launch; pa_probe_last_error() explains. */
pa_status pa_probe_read_pages(const void* pool, int64_t pool_bytes, const int32_t* page_ids, int32_t num_pages,
                              uint32_t* sink, int32_t grid, int32_t pages_in_flight, int32_t mode,
                              int32_t* dev_status, void* stream);

/* LDS read rate: `grid` workgroups of waves_per_group (4, 8 or 16) wavefronts each
 * fill a 64 KiB LDS array, then every wavefront reads iters x 8 pieces of 16 bytes
 * of it (lane-consecutive addresses) and thread t of workgroup b writes the XOR of
 * its pieces, folded to one word, to sink[b * 64 * waves_per_group + t].
 *   sink   device, uint32 [grid * 64 * waves_per_group]
 * Errors: PA_ERR_INVALID for bad arguments (nothing is launched), PA_ERR_HIP for a
 * failed launch. */
pa_status pa_probe_lds_read(uint32_t* sink, int32_t grid, int32_t waves_per_group, int32_t iters, void* stream);

const char* pa_probe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H */
