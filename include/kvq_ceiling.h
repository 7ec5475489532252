/*
 * kvq_ceiling — read-bandwidth ceilings of the GPU for the decode kernel's
 * access patterns (measurement only; libkvq_ceiling.so, separate from the
 * attention library).  The decode kernel streams a quantized cache once per
 * step, so its speed is bounded by how fast the part reads; these calls
 * measure that bound with plain reads.
 *
 * Ownership: the caller owns every buffer.  All work is queued on `stream`
 * (a hipStream_t as void*).  Returns 0 on success, -1 for invalid arguments
 * (nothing queued), -5 if the launch failed.
 */
#ifndef KVQ_CEILING_H
#define KVQ_CEILING_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Geometry of a contiguous cache for kvq_ceiling_tiles: `units`
 * (sequence, KV head) pairs of `tiles` 64-token tiles each; each tile is
 * k_tile_bytes of K codes, v_tile_bytes of V codes (both multiples of 1024,
 * at most 16 KiB together) and s_tile_bytes (16..512, a multiple of 16) in
 * each scale plane.  Planes are laid out [unit][tile][bytes], device
 * pointers 16-byte aligned. */
typedef struct kvq_ceiling_tiles_args {
  const void* k_codes;
  const void* v_codes;
  const void* k_scales;
  const void* v_scales;
  int32_t units, tiles;
  int32_t k_tile_bytes, v_tile_bytes, s_tile_bytes;
} kvq_ceiling_tiles_args;

/* Read `bytes` (a multiple of 16) of device memory at `buf` (16-byte
 * aligned) once: `blocks` workgroups of 256 lanes, grid-stride, `unroll`
 * (1, 4, 8 or 16) 16-byte loads per lane in flight; nontemporal != 0 uses
 * non-temporal loads.  sink: device uint32 of at least
 * kvq_ceiling_sink_words(blocks, 1) words. */
int kvq_ceiling_stream(const void* buf, size_t bytes, int32_t blocks, int32_t unroll,
                       int32_t nontemporal, uint32_t* sink, void* stream);

/* Read every tile of every unit once in the decode kernel's pattern: grid
 * (splits, units) workgroups of 8 waves; a workgroup takes a contiguous
 * range of its unit's tiles (mode bit 1 clear) or every splits-th chunk of 8
 * tiles (mode bit 1 set), its waves pull tiles from an LDS counter and keep
 * `ahead` (1 or 2) tiles of loads in flight; mode bit 0 makes the loads
 * non-temporal.  sink: device uint32 of at least
 * kvq_ceiling_sink_words(splits, units) words. */
int kvq_ceiling_tiles(const kvq_ceiling_tiles_args* args, int32_t splits, int32_t ahead,
                      int32_t mode, uint32_t* sink, void* stream);

/* Words of `sink` the two calls above need. */
size_t kvq_ceiling_sink_words(int32_t blocks_or_splits, int32_t units);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_CEILING_H */
