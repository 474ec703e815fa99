/* Measurement and testing helpers of libpkv, kept apart from pkv.h because
 * they are not part of the attention path: the streaming-read probe, and an
 * override of the balanced schedules' grid size for tests and measurements.
 * Same status codes and error reporting as pkv.h (pkv_last_error). */
#ifndef PKV_PROBE_H
#define PKV_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "pkv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming-read probe: the HBM read rate this GPU achieves for paged
 * decode's access pattern, for comparison with the decode kernels (not part
 * of the attention path).  Reads num_tiles 4 KiB tiles of buf in the order
 * tile_ids gives, with a persistent grid of `workgroups` workgroups of 4
 * waves; each wave streams one contiguous share of the list with four tiles
 * in flight, using non-temporal loads.  Each thread stores a fold of what
 * it read (per tile, in order: rotate left by one, then XOR the tile's words)
 * to sink, so that the loads cannot be dropped.
 *   buf       : device memory, buf_bytes bytes (16-byte aligned); a tile id
 *               outside [0, buf_bytes / 4096) reads tile 0.
 *   tile_ids  : device int32[num_tiles].
 *   sink      : device uint32[workgroups * 256], overwritten.
 *   workgroups: 1 .. 65535.
 *   ev_start, ev_stop: caller-created HIP events (hipEvent_t as void*, NULL =
 *               skip) stamped by the probe kernel's own dispatch at its
 *               start and end, as the decode entry points stamp theirs.
 * Asynchronous on stream.  PKV_ERR_INVALID_ARG on NULL pointers, negative
 * sizes or a bad workgroup count. */
pkv_status pkv_stream_read_probe(const void* buf, int64_t buf_bytes, const int32_t* tile_ids,
                                 int32_t num_tiles, uint32_t* sink, int32_t workgroups,
                                 void* stream, void* ev_start, void* ev_stop);

/* Workgroups (of 4 waves) the balanced decode and multi-query schedules
 * launch for calls made later by the calling thread; n = 0 restores the
 * default (the current device's compute-unit count: one wave on every
 * SIMD).  Thread-local: other threads' calls keep their own setting.  It
 * changes what pkv_decode_workspace_size and pkv_multiquery_workspace_size
 * return on this thread, so set it before sizing workspaces.  For tests (any
 * grid must give the same attention) and measurements.  PKV_ERR_INVALID_ARG
 * for n < 0 or n > 65535. */
pkv_status pkv_set_stream_workgroups(int32_t n);

#ifdef __cplusplus
}
#endif

#endif /* PKV_PROBE_H */
