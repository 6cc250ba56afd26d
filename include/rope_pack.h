/*
 * rope_pack.h -- host-side packing of variable-length sequences into bins,
 * and a cache of the packed batch's metadata, for the rotation kernels of
 * rope_qk.h.  C ABI: plain pointers and sizes.
 *
 * What it does
 * ------------
 * "Chronicals: A High-Performance Framework for LLM Fine-Tuning with 3.51x
 * Speedup over Unsloth", abstract, optimisation (4): Best-Fit Decreasing
 * sequence packing recovers most of the compute that padding wastes.  The
 * reading implemented is the textbook algorithm: lengths in decreasing
 * order (equal lengths by index); each goes into the open bin whose
 * remaining room is the smallest that still holds it (equal rooms: the bin
 * opened first), or into a new bin; within a bin, sequences follow one
 * another from token 0 in the order placed.
 *
 * "Unsloth und NVIDIA optimieren LLM-Training um zusätzliche 25%"
 * (lumeric.app), item (1): caching the packed-sequence metadata removes
 * repeated GPU-CPU synchronisations in the packed path.  Here the cache
 * builds a batch's plan once, uploads its cu_seqlens once (asynchronously),
 * and every later lookup of the same batch -- one per layer, forward and
 * backward -- is answered on the host with no device work at all.
 *
 * The packed batch: bin b holds tokens [b * capacity, (b + 1) * capacity) of
 * one token axis.  Its cu_seqlens lists every bin's sequences in token order
 * and, after them, the bin's unused tail as one padding segment (the caller
 * masks it; the rotation kernels rotate it like any segment), so it covers
 * [0, nbins * capacity) and one kernel launch handles the whole batch.
 *
 * Status codes are those of rope_qk.h.
 */
#ifndef ROPE_PACK_H
#define ROPE_PACK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Best-Fit-Decreasing packing of n sequence lengths into bins of `capacity`
 * tokens.  Host memory, synchronous, O(n log n).
 *
 *   lengths      host int32[n], each in [0, capacity]
 *   bin_of       host int32[n] out: the bin of sequence i
 *   offset_of    host int32[n] out: its first token inside the bin
 *   nbins        out: bins used
 *
 * Returns ROPE_QK_OK, ROPE_QK_ERR_NULL (a pointer NULL while n > 0, or
 * nbins NULL) or ROPE_QK_ERR_SHAPE (n < 0, capacity < 1 or > 2^31 - 1, a
 * length outside [0, capacity]).
 */
int rope_pack_bfd(const int32_t* lengths, int64_t n, int64_t capacity, int32_t* bin_of, int32_t* offset_of,
                  int64_t* nbins);

/*
 * cu_seqlens of the packed batch over nbins * capacity tokens (host): every
 * bin's sequences in token order, then its unused tail as one segment.
 *
 *   cu_out       host int32[n + nbins + 1] out; cu_out[0 .. *nseg] are written
 *   nseg         out: segments (sequences plus padding tails)
 *
 * The placement must be one that rope_pack_bfd could return (each bin's
 * sequences contiguous from token 0); else ROPE_QK_ERR_SHAPE, as for
 * nbins * capacity > 2^31 - 1.
 */
int rope_pack_cu_seqlens(const int32_t* lengths, const int32_t* bin_of, const int32_t* offset_of, int64_t n,
                         int64_t nbins, int64_t capacity, int32_t* cu_out, int64_t* nseg);

/* The packed-metadata cache (opaque). */
typedef struct rope_pack_cache rope_pack_cache;

/* One packed batch, as the cache holds it.  Every pointer is owned by the
 * cache and stays valid until this plan is evicted (after max_entries other
 * distinct batches have been looked up) or the cache is destroyed. */
typedef struct rope_pack_plan {
  const int32_t* cu_seqlens_device;  /* device int32[nseg + 1]; NULL in a host-only cache */
  const int32_t* cu_seqlens_host;    /* host int32[nseg + 1] */
  const int32_t* bin_of;             /* host int32[n] */
  const int32_t* offset_of;          /* host int32[n] */
  int64_t n;                         /* sequences */
  int64_t nseg;                      /* segments of cu_seqlens (sequences + padding tails) */
  int64_t nbins;
  int64_t T;                         /* tokens of the packed batch: nbins * capacity */
  int32_t max_seqlen;                /* longest segment */
  int32_t hit;                       /* 1: this lookup found the plan cached */
} rope_pack_plan;

/*
 * A cache of up to max_entries (>= 1) packed batches for one device.  device
 * >= 0: plans are uploaded to that HIP device; device == -1: host-only
 * (no device memory, cu_seqlens_device stays NULL).  Returns ROPE_QK_OK,
 * ROPE_QK_ERR_NULL or ROPE_QK_ERR_SHAPE (max_entries < 1 or device < -1).
 */
int rope_pack_cache_create(int64_t max_entries, int device, rope_pack_cache** out);

/*
 * The plan of the batch `lengths` packed into bins of `capacity` tokens.
 * A hit only looks the batch up (hashing its lengths) and copies the plan
 * description: no device call, no synchronisation.  A miss packs the batch
 * (rope_pack_bfd, rope_pack_cu_seqlens), allocates its device buffer and
 * enqueues the upload of cu_seqlens from pinned host memory on `stream`
 * (hipStream_t; kernels on other streams must be ordered after it by the
 * caller), evicting the least recently used plan when the cache is full.
 * Freeing an evicted plan's buffers waits for the device (hipFree), so size
 * the cache for the batches in use.  Thread-safe.
 *
 * Returns ROPE_QK_OK, ROPE_QK_ERR_NULL, ROPE_QK_ERR_SHAPE (as rope_pack_bfd)
 * or ROPE_QK_ERR_LAUNCH (a HIP allocation or copy failed).
 */
int rope_pack_cache_get(rope_pack_cache* cache, const int32_t* lengths, int64_t n, int64_t capacity, void* stream,
                        rope_pack_plan* out);

/* Lookups answered from the cache, lookups that packed, plans held. */
int rope_pack_cache_stats(const rope_pack_cache* cache, int64_t* hits, int64_t* misses, int64_t* entries);

/* Frees every plan (waiting for the device) and the cache itself; NULL is a no-op. */
void rope_pack_cache_destroy(rope_pack_cache* cache);

#ifdef __cplusplus
}
#endif

#endif /* ROPE_PACK_H */
