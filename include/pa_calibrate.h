/*
 * pa_calibrate.h — measurement reference of libpa.so: how fast this GPU reads the bytes a decode
 * call reads, with nothing else done.  Not part of the attention path; bench.py prints its rate
 * beside the decode kernels' roofline, so the achieved fraction of the 8 TB/s HBM peak can be set
 * against what a plain read of the same bytes achieves on the same device.
 */
#ifndef PA_CALIBRATE_H
#define PA_CALIBRATE_H

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * pa_calibrate_read — read every byte of the listed tiles of two pools and nothing else.
 *
 *   k_pool, v_pool  device buffers; tile t is bytes [t * tile_bytes, (t + 1) * tile_bytes) of
 *                  each (the layout of include/pa.h: tile (b, h) is t = b * num_kv_heads + h).
 *   tile_bytes     a positive multiple of 1024.
 *   tiles          device int32 [num_tiles] tile indices (any order; each is read once per call,
 *                  in both pools).  NULL reads tiles 0 .. num_tiles - 1 in order (a sequential
 *                  read of num_tiles * tile_bytes bytes per pool).
 *   sink           device uint32 [ceil(num_tiles / 4)]: one word per workgroup of four
 *                  wavefronts (an XOR of what they read), so that the loads are not dead code; its
 *                  value means nothing.
 * One wavefront per list entry issues all of the entry's 16-byte loads at once (tile_bytes / 512
 * per lane, each wave-wide load a whole 1 KiB, with the non-temporal hint the decode kernels use);
 * the hardware keeps as many wavefronts in flight as fit on the device.
 * Returns PA_ERR_NULL / PA_ERR_SHAPE for bad arguments (nothing enqueued), PA_ERR_LAUNCH if the
 * launch fails.  Bytes read per call: 2 * num_tiles * tile_bytes.
 */
pa_status pa_calibrate_read(const void *k_pool, const void *v_pool, int64_t tile_bytes,
                            const int32_t *tiles, int64_t num_tiles, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* PA_CALIBRATE_H */
