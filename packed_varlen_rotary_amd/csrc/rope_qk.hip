// Fused in-place QK rotary position embedding over packed variable-length
// batches, forward and backward, for AMD Instinct MI355X (CDNA4, gfx950).
//
// The operation, its arguments and its contract are documented in
// include/rope_qk.h.  Sources on the pages: the fused QK RoPE kernel paragraph
// of "Unsloth prétend accélérer 5 fois l'entraînement des LLM avec de nouveaux
// noyaux Triton et un auto-packing" (seventnews.com: q and k in one kernel,
// variable length, fully in place), its auto-packing paragraph (length
// metadata keeps samples apart), its LONG_INDEXING paragraph (500K-token
// contexts need wide offsets) and its kernel-history paragraph (blocks launched
// for groups of heads share the rotary factors); "Chronicals: A
// High-Performance Framework for LLM Fine-Tuning with 3.51x Speedup over
// Unsloth", abstract, optimisation (1) (QK-RoPE fusion removes memory traffic).
//
// Design (one launch per call, HBM-bound: every element of q and k is read
// once and written once, ~0.75 flop per byte, so there is no MFMA here):
//
//  * A workgroup owns a tile of consecutive tokens (one tile per workgroup;
//    measured on MI355X, a one-shot grid streams better than a persistent
//    one).  The work of a tile is a flat list of "tasks"; a task is one
//    16-byte chunk of the first half of a head together with the matching
//    16-byte chunk of its second half (the rotate_half partner i + D/2), over
//    the heads of q followed by those of k.  Consecutive lanes take
//    consecutive chunks of a head, so each load/store instruction of a wave
//    covers whole 64-128 byte runs.  Each lane keeps 4 tasks (128 bytes of
//    loads) in flight.
//  * First the workgroup finds each token's position -- a wave-uniform
//    binary search over cu_seqlens through the scalar cache, then a uniform
//    scan of the boundaries inside the tile -- and evaluates cos/sin once per
//    (token, pair) in float64 into LDS, where all heads of q and k read them.
//    Then it streams its q/k chunks with non-temporal loads and stores; the
//    other workgroups resident on the CU overlap each other's phases.
//  * The rotation is done in float64 and rounded once: fp32 output is the
//    correctly rounded fp32; bf16 output is the correctly rounded bf16 (fast
//    float64->fp32->bf16 path, and an exact re-rounding for the rare values
//    whose fp32 rounding lands exactly on a bf16 midpoint).
//  * All offsets are 64-bit; one build covers every tensor size.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "rope_qk.h"
#include "rope_sincos.h"

namespace {

constexpr int kThreads = 256;          // 4 wave64s per workgroup
constexpr int kMaxHalf = 256;          // D <= 512
constexpr int kMaxTileTokens = 64;
constexpr int kMaxTableBytes = 16384;  // cos/sin table per workgroup
constexpr uint32_t kMaxTasksPerToken = 65535;
constexpr int64_t kMaxGrid = int64_t(1) << 20;  // grid * 256 work-items stays below 2^32

// Two instances of the rotation kernel, by the number of 16-byte chunk pairs
// each lane keeps in flight: 2 (occupancy 4 waves/SIMD) or 4 (occupancy 3).
// Tiles hold whole tokens, so a tile of 256 * tpt tasks is only partly used
// when a token's task count does not divide it.  Measured on MI355X, the
// 2-task instance is faster whenever its tiles are at least ~90% full
// (e.g. 16 heads x D 64: +5-11% at every batch size), otherwise the 4-task
// instance is (e.g. 40 heads x D 128: 62.5% full tiles, 4-task +10-18%).
constexpr double kMinTileFill = 0.9;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef double f64x2 __attribute__((ext_vector_type(2)));
// cu_seqlens is only read, with wave-uniform indices: through the constant
// address space these become scalar loads, which the vector-memory counter
// does not order behind the tile's in-flight HBM loads.
typedef const __attribute__((address_space(4))) int32_t* cu_ptr;

struct RopeParams {
  char* q;                 // base of q (bytes)
  char* k;                 // base of k (bytes)
  const int32_t* cu;       // cu_seqlens[nseq + 1]
  int64_t T;
  int64_t q_st, q_sh;      // byte strides of q along tokens / heads
  int64_t k_st, k_sh;      // byte strides of k along tokens / heads
  int64_t ntiles;          // ceil(T / tile_tokens)
  uint64_t magic_task;     // ceil(2^32 / tasks_per_tok)
  uint64_t magic_chunk;    // ceil(2^32 / chunks)
  int32_t nseq;
  int32_t Hq;
  int32_t tasks_per_tok;   // (Hq + Hkv) * chunks
  int32_t chunks;          // 16-byte chunks per half head
  int32_t half;            // D / 2
  int32_t half_bytes;      // (D / 2) * element size
  int32_t tile_tokens;
  double sign;             // +1 forward, -1 backward
  double inv_freq[kMaxHalf];
};

// n / d for n, d < 2^16 with m = ceil(2^32 / d): exact because n * (m d - 2^32) < 2^32.
__device__ __forceinline__ uint32_t div_small(uint32_t n, uint64_t m) {
  return static_cast<uint32_t>((static_cast<uint64_t>(n) * m) >> 32);
}

// Last index s in [0, nseq] with cu[s] <= t, or -1 if cu[0] > t.  Every index
// probed lies in [0, nseq] whatever cu holds.
__device__ __forceinline__ int32_t last_start_at_or_before(cu_ptr cu, int32_t nseq, int64_t t) {
  int32_t lo = -1, hi = nseq + 1;  // cu[lo] <= t < cu[hi], with virtual -inf / +inf ends
  while (hi - lo > 1) {
    const int32_t mid = lo + ((hi - lo) >> 1);
    if (static_cast<int64_t>(cu[mid]) <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// Position of token t inside its packed sequence, or -1 when t lies outside
// [cu[0], cu[nseq]): t minus the last sequence start at or before t, so empty
// segments (repeated offsets) resolve to the sequence that holds t and the
// counter restarts at every boundary.
__device__ __forceinline__ int32_t token_position(cu_ptr cu, int32_t nseq, int64_t t) {
  if (t >= static_cast<int64_t>(cu[nseq])) return -1;
  const int32_t s = last_start_at_or_before(cu, nseq, t);
  if (s < 0) return -1;
  const int64_t p = t - static_cast<int64_t>(cu[s]);
  return p <= INT32_MAX ? static_cast<int32_t>(p) : -1;
}

// LDS slot of pair i of tile token tt.  Pairs are stored chunk-minor:
// i = c * vec + j -> (tt * vec + j) * chunks + c, so lanes working on
// different chunks of one token read adjacent 16-byte slots (no bank
// conflicts) and lanes on the same chunk read the same slot (broadcast).
__device__ __forceinline__ int cs_slot(int tt, int i, int vec, int chunks) {
  const int c = i / vec;
  const int j = i - c * vec;
  return (tt * vec + j) * chunks + c;
}

// Fast rounding of two float64 values to a packed bf16 pair: round each to
// fp32, then the pair to bf16 (both round to nearest even; one packed
// conversion).  The result equals the single correctly rounded bf16 unless
// an fp32 value is exactly a bf16 midpoint, which sets `tie`.
__device__ __forceinline__ uint32_t pack_bf16_fast(double lo, double hi, bool& tie) {
  const f32x2 f = {static_cast<float>(lo), static_cast<float>(hi)};
  tie |= (__float_as_uint(f.x) & 0xFFFFu) == 0x8000u;
  tie |= (__float_as_uint(f.y) & 0xFFFFu) == 0x8000u;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// Exact: one rounding from float64 to bf16 (the compiler's float64->bf16
// conversion rounds to odd at fp32 precision, then to nearest even).
__device__ __forceinline__ uint32_t pack_bf16_exact(double lo, double hi) {
  const f64x2 d = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(d, bf16x2));
}

__device__ __forceinline__ double bf16_lo(uint32_t w) { return static_cast<double>(__uint_as_float(w << 16)); }
__device__ __forceinline__ double bf16_hi(uint32_t w) { return static_cast<double>(__uint_as_float(w & 0xFFFF0000u)); }

// Rotate one task of bf16 data: a holds x[i .. i+7], b holds x[i+D/2 .. i+D/2+7].
template <bool kExact>
__device__ __forceinline__ bool rotate_bf16(const u32x4& a, const u32x4& b, const double2* __restrict__ cs,
                                            int chunks, u32x4& oa, u32x4& ob) {
  bool tie = false;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const double2 c0 = cs[(2 * j) * chunks];
    const double2 c1 = cs[(2 * j + 1) * chunks];
    const double x1l = bf16_lo(a[j]), x1h = bf16_hi(a[j]);
    const double x2l = bf16_lo(b[j]), x2h = bf16_hi(b[j]);
    const double y1l = fma(x1l, c0.x, -(x2l * c0.y));
    const double y2l = fma(x2l, c0.x, x1l * c0.y);
    const double y1h = fma(x1h, c1.x, -(x2h * c1.y));
    const double y2h = fma(x2h, c1.x, x1h * c1.y);
    if (kExact) {
      oa[j] = pack_bf16_exact(y1l, y1h);
      ob[j] = pack_bf16_exact(y2l, y2h);
    } else {
      oa[j] = pack_bf16_fast(y1l, y1h, tie);
      ob[j] = pack_bf16_fast(y2l, y2h, tie);
    }
  }
  return tie;
}

// Rotate one task of fp32 data: a holds x[i .. i+3], b holds x[i+D/2 .. i+D/2+3].
__device__ __forceinline__ void rotate_f32(const u32x4& a, const u32x4& b, const double2* __restrict__ cs,
                                           int chunks, u32x4& oa, u32x4& ob) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const double2 c = cs[j * chunks];
    const double x1 = static_cast<double>(__uint_as_float(a[j]));
    const double x2 = static_cast<double>(__uint_as_float(b[j]));
    oa[j] = __float_as_uint(static_cast<float>(fma(x1, c.x, -(x2 * c.y))));
    ob[j] = __float_as_uint(static_cast<float>(fma(x2, c.x, x1 * c.y)));
  }
}

// One tile of consecutive tokens per workgroup (a grid-stride loop covers
// launches with more tiles than the grid).
template <int kDtype, int kTPT, int kWavesPerSimd>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd)))
void rope_qk_kernel(const RopeParams p) {
  constexpr int kVec = (kDtype == ROPE_QK_BF16) ? 8 : 4;  // elements per 16 bytes
  __shared__ int32_t s_pos[kMaxTileTokens];                 // positions of the tile's tokens
  extern __shared__ double2 s_cs[];                         // [tile_tokens * half] {cos, sign*sin}
  const int tid = threadIdx.x;
  const cu_ptr cu = (cu_ptr)p.cu;  // address-space cast (C-style: reinterpret_cast cannot change it)
  const int32_t nseq = p.nseq;
  const int64_t cu_last = cu[nseq];

  for (int64_t tile = blockIdx.x; tile < p.ntiles; tile += gridDim.x) {
    const int64_t t0 = tile * p.tile_tokens;
    const int ntok = static_cast<int>(min(static_cast<int64_t>(p.tile_tokens), p.T - t0));
    const int64_t t_end = t0 + ntok;  // one past the tile's last token
    const uint32_t ntasks = static_cast<uint32_t>(ntok) * static_cast<uint32_t>(p.tasks_per_tok);
    const int nent = ntok * p.half;

    const int32_t s0 = last_start_at_or_before(cu, nseq, t0);  // scalar loads

    for (uint32_t base = 0; base < ntasks; base += kThreads * kTPT) {
      u32x4 a[kTPT], b[kTPT];
      char* ptr[kTPT];
      int tt_of[kTPT], c_of[kTPT];
      bool act[kTPT];

      // 1. positions and the cos/sin table (first pass of the tile only)
      if (base == 0) {
#pragma unroll 1
        for (int e0 = 0; e0 < nent; e0 += kThreads) {
          const int e = e0 + tid;
          const bool on = e < nent;
          const int tt = on ? e / p.half : 0;
          const int i = e - tt * p.half;
          const int64_t t = t0 + tt;
          // last sequence start at or before t: the tile's first start, then
          // any boundaries inside the tile (wave-uniform scan)
          int64_t start = s0 >= 0 ? static_cast<int64_t>(cu[s0]) : INT64_MIN;
          for (int32_t j = s0 + 1; j <= nseq; ++j) {
            const int64_t v = cu[j];
            if (v >= t_end) break;
            start = v <= t ? v : start;
          }
          const int64_t pos64 = t - start;
          const int32_t pos =
              (start != INT64_MIN && t < cu_last && pos64 <= INT32_MAX) ? static_cast<int32_t>(pos64) : -1;
          if (on) {
            if (i == 0) s_pos[tt] = pos;
            if (pos >= 0) {
              double sn, cs;
              rope_sincos(static_cast<double>(pos) * p.inv_freq[i], &sn, &cs);
              s_cs[cs_slot(tt, i, kVec, p.chunks)] = make_double2(cs, p.sign * sn);
            }
          }
        }
        __syncthreads();
      }

      // 2. issue every load of this pass (lanes without a task re-read task 0)
#pragma unroll
      for (int u = 0; u < kTPT; ++u) {
        const uint32_t n_raw = base + static_cast<uint32_t>(tid + u * kThreads);
        act[u] = n_raw < ntasks;
        const uint32_t n = act[u] ? n_raw : 0u;
        const uint32_t tt = div_small(n, p.magic_task);
        const uint32_t r = n - tt * static_cast<uint32_t>(p.tasks_per_tok);
        const uint32_t h = div_small(r, p.magic_chunk);
        const uint32_t c = r - h * static_cast<uint32_t>(p.chunks);
        const int64_t t = t0 + tt;
        const bool is_q = static_cast<int32_t>(h) < p.Hq;
        char* row = is_q ? p.q + t * p.q_st + static_cast<int64_t>(h) * p.q_sh
                         : p.k + t * p.k_st + static_cast<int64_t>(h - p.Hq) * p.k_sh;
        ptr[u] = row + static_cast<int64_t>(c) * 16;
        tt_of[u] = static_cast<int>(tt);
        c_of[u] = static_cast<int>(c);
        // streamed once: non-temporal, so they do not displace other data in the caches
        a[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ptr[u]));
        b[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ptr[u] + p.half_bytes));
      }

      // 3. rotate and store; tokens outside every sequence are left untouched
#pragma unroll
      for (int u = 0; u < kTPT; ++u) {
        if (!act[u] || s_pos[tt_of[u]] < 0) continue;
        const double2* cs = s_cs + tt_of[u] * kVec * p.chunks + c_of[u];
        u32x4 oa, ob;
        if constexpr (kDtype == ROPE_QK_BF16) {
          if (rotate_bf16<false>(a[u], b[u], cs, p.chunks, oa, ob))
            rotate_bf16<true>(a[u], b[u], cs, p.chunks, oa, ob);
        } else {
          rotate_f32(a[u], b[u], cs, p.chunks, oa, ob);
        }
        __builtin_nontemporal_store(oa, reinterpret_cast<u32x4*>(ptr[u]));
        __builtin_nontemporal_store(ob, reinterpret_cast<u32x4*>(ptr[u] + p.half_bytes));
      }
    }
    __syncthreads();  // a further tile of this workgroup rewrites s_pos and s_cs
  }
}

__global__ __launch_bounds__(kThreads) void rope_positions_kernel(const int32_t* __restrict__ cu_seqlens,
                                                                  int32_t nseq, int64_t T,
                                                                  int32_t* __restrict__ out) {
  const cu_ptr cu = (cu_ptr)cu_seqlens;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; t < T; t += stride)
    out[t] = token_position(cu, nseq, t);
}

// Rows of D elements at t * st + h * sh (t < T, h < H), all strides >= 0: do any two overlap?
bool rows_overlap(int64_t T, int64_t H, int64_t D, int64_t st, int64_t sh) {
  if (T <= 1 && H <= 1) return false;
  if (T <= 1) return sh < D;
  if (H <= 1) return st < D;
  const int64_t s_small = st < sh ? st : sh, n_small = st < sh ? T : H;
  const int64_t s_big = st < sh ? sh : st;
  if (s_small < D) return true;
  return s_big / s_small < n_small;  // s_big < n_small * s_small, without overflow
}

int launch_rope(void* q, void* k, const int32_t* cu, int64_t nseq, int64_t T, int64_t Hq, int64_t Hkv, int64_t D,
                int64_t q_st, int64_t q_sh, int64_t k_st, int64_t k_sh, double theta, int dtype, void* stream,
                double sign) {
  if (dtype != ROPE_QK_FP32 && dtype != ROPE_QK_BF16) return ROPE_QK_ERR_DTYPE;
  if (nseq < 0 || T < 0 || Hq < 0 || Hkv < 0 || D < 2 || (D & 1) || D > 2 * kMaxHalf || T > INT32_MAX ||
      nseq >= INT32_MAX || Hq + Hkv > INT32_MAX)
    return ROPE_QK_ERR_SHAPE;
  if (!(theta > 0.0) || !isfinite(theta)) return ROPE_QK_ERR_THETA;
  if (T == 0 || nseq == 0 || Hq + Hkv == 0) return ROPE_QK_OK;
  if (cu == nullptr || (Hq > 0 && q == nullptr) || (Hkv > 0 && k == nullptr)) return ROPE_QK_ERR_NULL;
  if ((Hq > 0 && (q_st < 0 || q_sh < 0 || rows_overlap(T, Hq, D, q_st, q_sh))) ||
      (Hkv > 0 && (k_st < 0 || k_sh < 0 || rows_overlap(T, Hkv, D, k_st, k_sh))))
    return ROPE_QK_ERR_LAYOUT;

  const int64_t esz = dtype == ROPE_QK_BF16 ? 2 : 4;
  const int64_t half = D / 2;
  if ((half * esz) % 16) return ROPE_QK_ERR_ALIGN;
  if (Hq > 0 && ((reinterpret_cast<uintptr_t>(q) % 16) || (q_st * esz) % 16 || (q_sh * esz) % 16))
    return ROPE_QK_ERR_ALIGN;
  if (Hkv > 0 && ((reinterpret_cast<uintptr_t>(k) % 16) || (k_st * esz) % 16 || (k_sh * esz) % 16))
    return ROPE_QK_ERR_ALIGN;

  const int64_t chunks = half * esz / 16;
  const int64_t tasks_per_tok = (Hq + Hkv) * chunks;
  if (tasks_per_tok > kMaxTasksPerToken) return ROPE_QK_ERR_SHAPE;

  // tokens per tile for an instance keeping tpt tasks per lane: as many whole
  // tokens as fill 256 * tpt task slots, within the LDS table and position caps
  const auto tile_tokens_for = [&](int64_t tpt) {
    int64_t tt = static_cast<int64_t>(kThreads) * tpt / tasks_per_tok;
    const int64_t lds_cap = kMaxTableBytes / (half * 16);
    if (tt > kMaxTileTokens) tt = kMaxTileTokens;
    if (tt > lds_cap) tt = lds_cap;
    return tt < 1 ? int64_t(1) : tt;
  };
  const int64_t tile2 = tile_tokens_for(2);
  const bool two_per_lane =
      tile2 * tasks_per_tok <= 2 * kThreads && tile2 * tasks_per_tok >= kMinTileFill * 2 * kThreads;
  const int64_t tile = two_per_lane ? tile2 : tile_tokens_for(4);

  RopeParams p;
  p.q = static_cast<char*>(q);
  p.k = static_cast<char*>(k);
  p.cu = cu;
  p.T = T;
  p.q_st = q_st * esz;
  p.q_sh = q_sh * esz;
  p.k_st = k_st * esz;
  p.k_sh = k_sh * esz;
  p.ntiles = (T + tile - 1) / tile;
  p.magic_task = ((uint64_t(1) << 32) + tasks_per_tok - 1) / tasks_per_tok;
  p.magic_chunk = ((uint64_t(1) << 32) + chunks - 1) / chunks;
  p.nseq = static_cast<int32_t>(nseq);
  p.Hq = static_cast<int32_t>(Hq);
  p.tasks_per_tok = static_cast<int32_t>(tasks_per_tok);
  p.chunks = static_cast<int32_t>(chunks);
  p.half = static_cast<int32_t>(half);
  p.half_bytes = static_cast<int32_t>(half * esz);
  p.tile_tokens = static_cast<int32_t>(tile);
  p.sign = sign;
  for (int64_t i = 0; i < kMaxHalf; ++i)
    p.inv_freq[i] = i < half ? pow(theta, -static_cast<double>(2 * i) / static_cast<double>(D)) : 0.0;

  const int64_t grid = p.ntiles < kMaxGrid ? p.ntiles : kMaxGrid;
  const size_t lds = static_cast<size_t>(tile * half) * sizeof(double2);
  void* args[] = {&p};
  const void* fn;
  if (dtype == ROPE_QK_BF16)
    fn = two_per_lane ? reinterpret_cast<const void*>(&rope_qk_kernel<ROPE_QK_BF16, 2, 4>)
                     : reinterpret_cast<const void*>(&rope_qk_kernel<ROPE_QK_BF16, 4, 3>);
  else
    fn = two_per_lane ? reinterpret_cast<const void*>(&rope_qk_kernel<ROPE_QK_FP32, 2, 4>)
                     : reinterpret_cast<const void*>(&rope_qk_kernel<ROPE_QK_FP32, 4, 3>);
  const hipError_t err = hipLaunchKernel(fn, dim3(static_cast<uint32_t>(grid)), dim3(kThreads), args, lds,
                                         static_cast<hipStream_t>(stream));
  return err == hipSuccess ? ROPE_QK_OK : ROPE_QK_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int rope_qk_fwd(void* q, void* k, const int32_t* cu_seqlens, int64_t nseq, int64_t T, int64_t Hq, int64_t Hkv,
                int64_t D, int64_t q_stride_t, int64_t q_stride_h, int64_t k_stride_t, int64_t k_stride_h,
                double theta, int dtype, void* stream) {
  return launch_rope(q, k, cu_seqlens, nseq, T, Hq, Hkv, D, q_stride_t, q_stride_h, k_stride_t, k_stride_h, theta,
                     dtype, stream, 1.0);
}

int rope_qk_bwd(void* dq, void* dk, const int32_t* cu_seqlens, int64_t nseq, int64_t T, int64_t Hq, int64_t Hkv,
                int64_t D, int64_t q_stride_t, int64_t q_stride_h, int64_t k_stride_t, int64_t k_stride_h,
                double theta, int dtype, void* stream) {
  return launch_rope(dq, dk, cu_seqlens, nseq, T, Hq, Hkv, D, q_stride_t, q_stride_h, k_stride_t, k_stride_h,
                     theta, dtype, stream, -1.0);
}

int rope_qk_positions(const int32_t* cu_seqlens, int64_t nseq, int64_t T, int32_t* pos_out, void* stream) {
  if (nseq < 0 || T < 0 || T > INT32_MAX || nseq >= INT32_MAX) return ROPE_QK_ERR_SHAPE;
  if (T == 0) return ROPE_QK_OK;
  if (cu_seqlens == nullptr || pos_out == nullptr) return ROPE_QK_ERR_NULL;
  const int64_t blocks = (T + kThreads - 1) / kThreads;
  const int64_t grid = blocks < 65536 ? blocks : 65536;
  int32_t n = static_cast<int32_t>(nseq);
  void* args[] = {&cu_seqlens, &n, &T, &pos_out};
  const hipError_t err =
      hipLaunchKernel(reinterpret_cast<const void*>(&rope_positions_kernel), dim3(static_cast<uint32_t>(grid)),
                      dim3(kThreads), args, 0, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? ROPE_QK_OK : ROPE_QK_ERR_LAUNCH;
}

const char* rope_qk_strerror(int status) {
  switch (status) {
    case ROPE_QK_OK: return "ok";
    case ROPE_QK_ERR_NULL: return "a required pointer is NULL";
    case ROPE_QK_ERR_SHAPE: return "unsupported shape (negative size, D odd/<2/>512, T >= 2^31, too many heads)";
    case ROPE_QK_ERR_DTYPE: return "unsupported dtype (expected ROPE_QK_FP32 or ROPE_QK_BF16)";
    case ROPE_QK_ERR_ALIGN: return "misaligned: pointers, strides and D/2 must be multiples of 16 bytes";
    case ROPE_QK_ERR_THETA: return "theta must be finite and > 0";
    case ROPE_QK_ERR_LAUNCH: return "HIP kernel launch failed";
    case ROPE_QK_ERR_LAYOUT: return "negative strides or overlapping rows";
    default: return "unknown status";
  }
}

}  // extern "C"
