// A plain in-place 16-byte stream for AMD Instinct MI355X (gfx950): the
// ceiling that the rotation kernels' HBM traffic is measured against.  The
// contract is in include/stream_ceiling.h.
//
// Each thread loads its chunks (256 chunks apart, so a wave-wide load covers
// 1 KiB of consecutive bytes), XORs them with a key that is 0, and only then
// stores them all back: the load/store order of the rotation kernels, without
// their arithmetic.  Every access stays below the buffer's chunk count.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "stream_ceiling.h"

namespace {

constexpr int kThreads = 256;
constexpr int64_t kGridX = 65536;
constexpr int64_t kLdsPerCu = 163840;  // MI355X: 160 KiB of LDS per compute unit

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) u32x4 gu32x4;

template <int kTPL, bool kNT>
__device__ __forceinline__ void stream_tile(gu32x4* buf, int64_t nchunks, int64_t tile, uint32_t key) {
  const int64_t base = tile * (kThreads * kTPL) + threadIdx.x;
  // Loads are never under a branch (a branch around each load made the
  // compiler wait for it before the next one was issued): a tile that ends
  // past the buffer re-reads its last chunk and stores only what is inside.
  const bool full = (tile + 1) * (kThreads * kTPL) <= nchunks;  // wave-uniform
  u32x4 v[kTPL];
#pragma unroll
  for (int u = 0; u < kTPL; ++u) {
    int64_t i = base + static_cast<int64_t>(u) * kThreads;
    if (!full) i = i < nchunks ? i : nchunks - 1;
    v[u] = kNT ? __builtin_nontemporal_load(buf + i) : buf[i];
  }
#pragma unroll
  for (int u = 0; u < kTPL; ++u) v[u] ^= key;
#pragma unroll
  for (int u = 0; u < kTPL; ++u) {
    const int64_t i = base + static_cast<int64_t>(u) * kThreads;
    if (full || i < nchunks) {
      if (kNT)
        __builtin_nontemporal_store(v[u], buf + i);
      else
        buf[i] = v[u];
    }
  }
}

// One tile per workgroup on a two-dimensional grid.
template <int kTPL, bool kNT>
__global__ __launch_bounds__(kThreads) void stream_oneshot(u32x4* data, int64_t nchunks, int64_t ntiles,
                                                           uint32_t key) {
  gu32x4* buf = (gu32x4*)data;  // address-space cast (C-style: reinterpret_cast cannot change it)
  const int64_t tile = static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x;
  if (tile < ntiles) stream_tile<kTPL, kNT>(buf, nchunks, tile, key);
}

// One tile's chunks into registers and back.  Chunks past the buffer use
// its last chunk: they re-read it and store back the value its own lane of
// the same tile stores, so every store instruction is issued and the
// compiler's wait counts stay exact.
template <int kTPL, bool kNT>
__device__ __forceinline__ void load_tile(gu32x4* buf, int64_t nchunks, int64_t tile, u32x4* v) {
  const int64_t base = tile * (kThreads * kTPL) + threadIdx.x;
#pragma unroll
  for (int u = 0; u < kTPL; ++u) {
    int64_t i = base + static_cast<int64_t>(u) * kThreads;
    i = i < nchunks ? i : nchunks - 1;
    v[u] = kNT ? __builtin_nontemporal_load(buf + i) : buf[i];
  }
}

template <int kTPL, bool kNT>
__device__ __forceinline__ void store_tile(gu32x4* buf, int64_t nchunks, int64_t tile, u32x4* v, uint32_t key) {
  const int64_t base = tile * (kThreads * kTPL) + threadIdx.x;
#pragma unroll
  for (int u = 0; u < kTPL; ++u) {
    int64_t i = base + static_cast<int64_t>(u) * kThreads;
    i = i < nchunks ? i : nchunks - 1;
    v[u] ^= key;
    if (kNT)
      __builtin_nontemporal_store(v[u], buf + i);
    else
      buf[i] = v[u];
  }
}

// gridDim.x workgroups, each taking every gridDim.x-th tile, with the next
// two tiles' loads in flight while a tile is stored: three register sets in
// turn (the loop unrolled by three), the loads ahead issued unconditionally
// (past the last tile they re-read it) so that the compiler's wait counts
// are exact, and only real tiles stored.
template <int kTPL, bool kNT>
__global__ __launch_bounds__(kThreads) void stream_persistent(u32x4* data, int64_t nchunks, int64_t ntiles,
                                                              uint32_t key) {
  gu32x4* buf = (gu32x4*)data;
  const int64_t step = gridDim.x;
  int64_t t = blockIdx.x;
  if (t >= ntiles) return;
  const auto ahead = [&](int64_t x) { return x < ntiles ? x : ntiles - 1; };
  u32x4 a[kTPL], b[kTPL], c[kTPL];
  load_tile<kTPL, kNT>(buf, nchunks, t, a);
  load_tile<kTPL, kNT>(buf, nchunks, ahead(t + step), b);
  for (;;) {
    load_tile<kTPL, kNT>(buf, nchunks, ahead(t + 2 * step), c);
    __builtin_amdgcn_sched_barrier(0);
    store_tile<kTPL, kNT>(buf, nchunks, t, a, key);
    __builtin_amdgcn_sched_barrier(0);
    t += step;
    if (t >= ntiles) break;
    load_tile<kTPL, kNT>(buf, nchunks, ahead(t + 2 * step), a);
    __builtin_amdgcn_sched_barrier(0);
    store_tile<kTPL, kNT>(buf, nchunks, t, b, key);
    __builtin_amdgcn_sched_barrier(0);
    t += step;
    if (t >= ntiles) break;
    load_tile<kTPL, kNT>(buf, nchunks, ahead(t + 2 * step), b);
    __builtin_amdgcn_sched_barrier(0);
    store_tile<kTPL, kNT>(buf, nchunks, t, c, key);
    __builtin_amdgcn_sched_barrier(0);
    t += step;
    if (t >= ntiles) break;
  }
}

template <int kTPL>
const void* pick(bool persistent, bool nt) {
  if (persistent)
    return nt ? reinterpret_cast<const void*>(&stream_persistent<kTPL, true>)
              : reinterpret_cast<const void*>(&stream_persistent<kTPL, false>);
  return nt ? reinterpret_cast<const void*>(&stream_oneshot<kTPL, true>)
            : reinterpret_cast<const void*>(&stream_oneshot<kTPL, false>);
}

}  // namespace

extern "C" int stream_ceiling_launch(void* buf, int64_t bytes, int chunks_per_lane, int64_t groups, int nontemporal,
                                     int groups_per_cu, void* stream) {
  if (bytes < 0 || bytes % 16 || bytes / 16 > (int64_t(1) << 31)) return STREAM_CEILING_ERR_SIZE;
  if (groups < 0 || groups > INT32_MAX || groups_per_cu < 0 || groups_per_cu > 32) return STREAM_CEILING_ERR_SHAPE;
  const void* fn = nullptr;
  const bool persistent = groups > 0, nt = nontemporal != 0;
  switch (chunks_per_lane) {
    case 1: fn = pick<1>(persistent, nt); break;
    case 2: fn = pick<2>(persistent, nt); break;
    case 4: fn = pick<4>(persistent, nt); break;
    case 8: fn = pick<8>(persistent, nt); break;
    case 16: fn = pick<16>(persistent, nt); break;
    default: return STREAM_CEILING_ERR_SHAPE;
  }
  if (bytes == 0) return STREAM_CEILING_OK;
  if (buf == nullptr) return STREAM_CEILING_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(buf) % 16) return STREAM_CEILING_ERR_ALIGN;
  int64_t nchunks = bytes / 16;
  const int64_t per_tile = int64_t(kThreads) * chunks_per_lane;
  int64_t ntiles = (nchunks + per_tile - 1) / per_tile;
  dim3 grid;
  if (persistent) {
    grid = dim3(static_cast<uint32_t>(groups < ntiles ? groups : ntiles));
  } else {
    const int64_t gx = ntiles < kGridX ? ntiles : kGridX;
    grid = dim3(static_cast<uint32_t>(gx), static_cast<uint32_t>((ntiles + gx - 1) / gx));
  }
  u32x4* p = static_cast<u32x4*>(buf);
  uint32_t key = 0;
  void* args[] = {&p, &nchunks, &ntiles, &key};
  // unused LDS so that groups_per_cu + 1 workgroups do not fit on a compute unit
  const size_t lds = groups_per_cu > 0 ? static_cast<size_t>(kLdsPerCu / (groups_per_cu + 1) + 1) : 0;
  const hipError_t err = hipLaunchKernel(fn, grid, dim3(kThreads), args, lds, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? STREAM_CEILING_OK : STREAM_CEILING_ERR_LAUNCH;
}
