/*
 * pagedkv_probe.h -- measuring aid shipped in libpagedkv beside the C ABI of
 * pagedkv.h.  It is not part of the attention path: it gives the HBM read rate the GPU
 * reaches for the access patterns of the path, the ceiling the kernels are compared
 * with.
 */
#ifndef PAGEDKV_PROBE_H
#define PAGEDKV_PROBE_H

#include "pagedkv.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * pkv_read_probe -- measuring aid, not part of the attention path: a read-only pass
 * over `num_tiles` tiles of `tile_bytes` bytes (a multiple of 1,024), tile i starting
 * at byte tiles[i] * tile_bytes of `base`, to measure the HBM read rate the GPU reaches
 * for an access pattern (contiguous tiles, or the scattered 2-8 KiB K/V tiles of a
 * paged decode step; the serving-engine KV page, section 2, puts a sequence's blocks
 * anywhere in the pool).  Reports nothing itself: time it on `stream`.
 *   base   DEVICE buffer of base_bytes bytes (read only).
 *   tiles  int32 [num_tiles] DEVICE tile indices; values outside
 *          [0, base_bytes / tile_bytes) are clamped into it.
 *   sink   uint32 [grid * 4] DEVICE output: one XOR of the loaded words per wave
 *          (keeps the loads from being dropped; no meaning of its own).
 *   grid   workgroups of 256 threads (4 waves); the tiles are split evenly over the
 *          grid * 4 waves in contiguous shares.
 * Errors: null pointers, num_tiles < 0, grid <= 0, tile_bytes not a positive multiple
 * of 1,024 or base_bytes < tile_bytes -> INVALID_ARG.  Asynchronous on `stream`.
 */
pkv_status pkv_read_probe(const void *base, int64_t base_bytes, const int32_t *tiles,
                          int32_t num_tiles, int32_t tile_bytes, uint32_t *sink,
                          int32_t grid, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_PROBE_H */
