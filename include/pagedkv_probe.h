/*
 * pagedkv_probe.h -- measurement aids of libpagedkv.so: the HBM bandwidth a
 * plain read reaches on this device, the practical ceiling against which the
 * bandwidth-bound paged-decode kernels are judged (decode streams each
 * sequence's K/V blocks once; page "PagedAttention 与连续批处理：LLM Serving
 * 的底层架构拆解", advice section: decode is memory-bound).  Not part of the
 * attention path.  Conventions (device pointers, stream-ordered, host-side
 * checks, status codes) are those of pagedkv.h.
 */
#ifndef PAGEDKV_PROBE_H
#define PAGEDKV_PROBE_H

#include "pagedkv.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads every byte of buf[0 .. bytes) once (16-byte loads in address order,
 * grid-stride over 2 workgroups per CU, four loads in flight per lane).  bytes must be a multiple of 16 and
 * buf 16-byte aligned (PKV_ERR_SHAPE otherwise).  sink: one 4-byte word of
 * device memory, written only for one specific fold of the data (in practice
 * never); the call writes nothing else.  bytes == 0 returns PKV_OK.
 */
pkv_status_t pkv_hbm_read_probe(const void* buf, size_t bytes, void* sink, void* stream);

/*
 * Reads num_tiles whole tiles of tile_bytes bytes (a multiple of 16) from
 * buf, tile tiles[i] at byte offset tiles[i] * tile_bytes, in list order
 * spread over the waves of the grid (four tiles in flight per wave): the
 * gather pattern of a paged decode.  Tile ids must
 * lie inside buf (the caller's contract).  sink as above.
 */
pkv_status_t pkv_hbm_gather_probe(const void* buf, const int32_t* tiles, int32_t num_tiles,
                                  int32_t tile_bytes, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_PROBE_H */
