/* Measurement helper of libpkv: the streaming-read probe, kept apart from
 * pkv.h because it is not part of the attention path.  Same status codes
 * and error reporting as pkv.h (pkv_last_error). */
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

#ifdef __cplusplus
}
#endif

#endif /* PKV_PROBE_H */
