/*
 * stream_ceiling.h -- a plain in-place HBM stream on AMD Instinct MI355X
 * (gfx950), the measured ceiling for the rotation kernels' access pattern.
 * C ABI, built as libstream_ceiling.so beside librope_qk.so.
 *
 * Not part of the rotation path: a measurement aid.  The rotation reads every
 * 16-byte chunk of q and k once and writes it back once, in place ("Chronicals:
 * A High-Performance Framework for LLM Fine-Tuning with 3.51x Speedup over
 * Unsloth", abstract, optimisation (1): the fused kernels are judged by the
 * memory traffic they remove).  This stream does the same traffic with no
 * arithmetic: each 16-byte chunk of a buffer is loaded, XOR-ed with a key
 * that is 0 (so the buffer keeps its contents) and stored back, so its time
 * bounds what any kernel with that traffic can reach on the part, at that
 * size, launch ramp and tail included.
 */
#ifndef STREAM_CEILING_H
#define STREAM_CEILING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define STREAM_CEILING_OK 0
#define STREAM_CEILING_ERR_NULL -1    /* buf is NULL with bytes > 0 */
#define STREAM_CEILING_ERR_SIZE -2    /* bytes negative or not a multiple of 16, or more than 2^31 chunks */
#define STREAM_CEILING_ERR_SHAPE -3   /* chunks_per_lane not 1, 2, 4, 8 or 16, groups or groups_per_cu out of range */
#define STREAM_CEILING_ERR_ALIGN -4   /* buf not 16-byte aligned */
#define STREAM_CEILING_ERR_LAUNCH -6  /* the HIP launch failed */

/*
 * One launch of the stream over buf[0, bytes) on `stream` (a hipStream_t),
 * asynchronous.  Workgroups of 256 threads; each thread loads
 * chunks_per_lane 16-byte chunks 256 chunks apart (a wave-wide load covers
 * 1 KiB of consecutive bytes), then stores them all back, as the rotation
 * kernels order their loads and stores.
 *
 *   buf              device memory owned by the caller, 16-byte aligned;
 *                    every byte is read and written back unchanged
 *   bytes            size of buf, a multiple of 16 (0: no launch)
 *   chunks_per_lane  1, 2, 4, 8 or 16
 *   groups           0: one tile of 256 * chunks_per_lane chunks per
 *                    workgroup (one-shot grid); > 0: that many workgroups,
 *                    each looping over every groups-th tile (persistent),
 *                    with the next two tiles' loads issued before a tile's
 *                    stores
 *   nontemporal      non-zero: non-temporal loads and stores (as the
 *                    rotation kernels use), else ordinary ones
 *   groups_per_cu    0: as many resident workgroups per compute unit as
 *                    fit; 1..32: at most that many (the launch reserves
 *                    LDS it does not use, as the rotation kernels do to cap
 *                    their occupancy)
 *
 * Returns STREAM_CEILING_OK or a negative status; nothing is launched on error.
 */
int stream_ceiling_launch(void* buf, int64_t bytes, int chunks_per_lane, int64_t groups, int nontemporal,
                          int groups_per_cu, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* STREAM_CEILING_H */
