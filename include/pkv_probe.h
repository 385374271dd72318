/* Measurement probes (libpkv_probe.so) -- aids, not part of the paged-attention path.
 *
 * Read bandwidth.  bench.py --ceiling uses them to measure what HBM delivers on this chip for the two
 * access patterns that bound the decode kernel: one contiguous stream, and whole fixed-size
 * tiles visited in a given (random) order, which is how decode gathers K/V through a block
 * table ("PagedAttention: Efficient LLM Serving with vLLM", "The PagedAttention Algorithm":
 * blocks sit anywhere in the pool and are reached through the table).  The figures they give
 * are the achievable ceilings that decode's bandwidth is compared with, beside the spec peak.
 */
#ifndef PKV_PROBE_H
#define PKV_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueue one read of device memory on `stream` (a hipStream_t; NULL = default stream).
 *
 *   buf, bytes      device buffer of `bytes` bytes (16-byte aligned, bytes a multiple of 16);
 *                   read only.
 *   tile_bytes      0: read the whole buffer, each workgroup one contiguous span of it;
 *                   2048, 4096 or 8192: read num_tiles whole tiles of that size, tile i of the
 *                   visit being the tile at byte offset order[i] * tile_bytes.
 *   order           device int32 [num_tiles], each entry in [0, bytes / tile_bytes); unused
 *                   when tile_bytes = 0.  Entries are not checked on the device.
 *   num_tiles       tiles to visit (0 < num_tiles, num_tiles * tile_bytes <= bytes).
 *   nontemporal     nonzero: nontemporal loads (the decode kernel's), else ordinary loads.
 *   split           0, or with tiles 1..1023: the share (of 1024) of the visit that the waves
 *                   of the even XCDs read (workgroup b runs on XCD b % 8; the first
 *                   num_tiles * split / 1024 entries of `order`), the odd XCDs reading the
 *                   rest -- the decode launches' weighting of the two halves; workgroups must
 *                   then be a multiple of 8.
 *   sink            device uint32 [1]; written only when a data-dependent hash takes one
 *                   particular value, which keeps the loads from being removed.
 *   workgroups      grid size (1 .. 65536), 256 threads each.
 *
 * Returns 0 on success, 1 for invalid arguments (nothing enqueued), 2 when the launch fails.
 */
int32_t pkv_probe_read(const void* buf, int64_t bytes, int32_t tile_bytes, const int32_t* order,
                       int64_t num_tiles, int32_t nontemporal, int32_t split, uint32_t* sink,
                       int32_t workgroups, void* stream);

/* Sustained matrix-core rate: enqueue one launch of `workgroups` workgroups of 256 threads,
 * each wave running `iters` rounds of eight back-to-back v_mfma_f32_16x16x32_f16 products on
 * independent accumulators (16 x 16 x 32 x 2 flops each).  mode:
 *   0  operands in registers;
 *   1  every product's A operand one 16-byte-per-lane LDS read, 1 KiB per wave and product --
 *      the LDS-to-product ratio of the multi-query kernel's K and V fragment reads;
 *   2, 3, 4  every product followed by 2, 4, 8 independent v_fma_f32;
 *   5, 6     every product followed by 1, 2 independent (v_mul_f32, v_exp_f32) pairs.
 *
 *   out     device float [workgroups * 256], written (keeps the products live).
 *
 * Returns 0 on success, 1 for invalid arguments (nothing enqueued), 2 when the launch fails.
 */
int32_t pkv_probe_mfma(int32_t mode, int32_t iters, int32_t workgroups, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_PROBE_H */
