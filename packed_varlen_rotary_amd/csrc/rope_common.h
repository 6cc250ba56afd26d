// Pieces shared by the rotation kernels (rope_qk.hip) and the fused
// RMSNorm + rotation kernels (rope_qk_norm.hip): limits, vector types,
// position search, the float64 -> 16-bit rounding, and the host-side argument
// checks and frequency table.  Every function is internal to the including
// file (anonymous namespace).

#ifndef ROPE_COMMON_H
#define ROPE_COMMON_H

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "rope_layout.h"
#include "rope_qk.h"
#include "rope_sincos.h"

namespace {

constexpr int kThreads = 256;                         // 4 wave64s per workgroup
constexpr int kMaxHalf = 256;                         // D <= 512
constexpr int kMaxTileTokens = 64;                    // tokens a tile may touch
constexpr int kMaxTableBytes = 16384;                 // cos/sin table per workgroup
constexpr int kEnt = kMaxTableBytes / 16 / kThreads;  // table entries per thread, at most
constexpr int64_t kGridX = 65536;                     // tiles per grid row
constexpr int64_t kLdsPerCu = 163840;                 // MI355X: 160 KiB of LDS per compute unit

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef double f64x2 __attribute__((ext_vector_type(2)));
// cu_seqlens is only read, with wave-uniform indices: through the constant
// address space these become scalar loads, which the vector-memory counter
// does not order behind the tile's in-flight HBM loads.
typedef const __attribute__((address_space(4))) int32_t* cu_ptr;
// q and k rows: explicitly global, so every load and store is a global_* (not
// flat) instruction, which the scalar-memory counter does not track.
typedef __attribute__((address_space(1))) char gchar;
typedef __attribute__((address_space(1))) u32x4 gu32x4;

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

// n / tasks_per_tok for n < 2^24 (m = ceil(2^40 / d), d < 2^16).
__device__ __forceinline__ uint32_t div_tok(uint32_t n, uint64_t m) {
  return static_cast<uint32_t>((static_cast<uint64_t>(n) * m) >> 40);
}

// ---- 16-bit storage (bf16, fp16): two elements per dword, the lower-indexed
// element in the low half ----

// Exact float64 values of the two elements of a dword.
template <int kDtype>
__device__ __forceinline__ f64x2 unpack16(uint32_t w) {
  if constexpr (kDtype == ROPE_QK_BF16) {
    return f64x2{static_cast<double>(__uint_as_float(w << 16)), static_cast<double>(__uint_as_float(w & 0xFFFF0000u))};
  } else {
    return __builtin_convertvector(__builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2), f64x2);
  }
}

// Is an fp32 value one that the fp32 -> fp16 step may round differently from
// a direct float64 -> fp16 rounding?  Midpoints of the fp16 grid in its normal
// range (low 13 of 24 significant bits 1 followed by zeros), and every value
// of magnitude below 2^-14, where the grid of fp16 subnormals is coarser
// (zero included: it only sends an exact value down the exact path too).
// The magnitude test is one float compare with an absolute-value operand.
__device__ __forceinline__ bool fp16_hard(float f) {
  return (__float_as_uint(f) & 0x1FFFu) == 0x1000u || fabsf(f) < 0x1p-14f;
}

// Fast rounding of two float64 values to a packed 16-bit pair: round each to
// fp32, then the pair to the storage format (both round to nearest even; one
// packed conversion).  The result equals the single correctly rounded value
// unless an fp32 value is exactly a midpoint of the storage grid (bf16: low 16
// bits 0x8000), or is otherwise hard (fp16_hard), which sets `tie`.
template <int kDtype>
__device__ __forceinline__ uint32_t pack16_fast(double lo, double hi, bool& tie) {
  const f32x2 f = {static_cast<float>(lo), static_cast<float>(hi)};
  if constexpr (kDtype == ROPE_QK_BF16) {
    tie |= (__float_as_uint(f.x) & 0xFFFFu) == 0x8000u;
    tie |= (__float_as_uint(f.y) & 0xFFFFu) == 0x8000u;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
  } else {
    tie |= fp16_hard(f.x);
    tie |= fp16_hard(f.y);
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
  }
}

// float64 -> fp32 rounded to odd: the fp32 neighbour of y toward zero, with
// its last bit set when y is not exactly representable.  Rounding that value
// to nearest even in a format with at least two fewer significant bits gives
// the correctly rounded y (Boldo and Melquiond, "Emulation of FMA and
// correctly rounded sums: proved algorithms using rounding to odd", IEEE
// Trans. Computers 2008).
__device__ __forceinline__ float f32_round_odd(double y) {
  const float f = static_cast<float>(y);
  const uint32_t b = __float_as_uint(f);
  const bool even_inexact = static_cast<double>(f) != y && !(b & 1u);
  // the other fp32 neighbour of y, which is odd: one step down or up in magnitude
  const uint32_t other = fabs(static_cast<double>(f)) > fabs(y) ? b - 1u : b + 1u;
  return __uint_as_float(even_inexact ? other : b);
}

// Exact: one rounding from float64 to the storage format.  bf16: the
// compiler's float64 -> bf16 conversion (rounds to odd at fp32 precision,
// then to nearest even).  fp16: round to odd at fp32, then the packed
// fp32 -> fp16 conversion (nearest even).
template <int kDtype>
__device__ __forceinline__ uint32_t pack16_exact(double lo, double hi) {
  if constexpr (kDtype == ROPE_QK_BF16) {
    const f64x2 d = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(d, bf16x2));
  } else {
    const f32x2 f = {f32_round_odd(lo), f32_round_odd(hi)};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
  }
}

// ---- host side ----

// Frequencies of a head of size r (pairs i < r/2), optionally with the Llama
// 3.1 rescaling (the rule is documented with rope_qk_options in rope_qk.h).
void make_inv_freq(double theta, int64_t r, const rope_qk_options& o, double* out) {
  const double kTwoPi = 6.283185307179586476925286766559;
  const double L = o.original_max_position;
  for (int64_t i = 0; i < kMaxHalf; ++i) {
    if (i >= r / 2) {
      out[i] = 0.0;
      continue;
    }
    const double f = pow(theta, -static_cast<double>(2 * i) / static_cast<double>(r));
    if (o.scaling != ROPE_QK_SCALING_LLAMA3) {
      out[i] = f;
      continue;
    }
    const double w = kTwoPi / f;
    if (w < L / o.high_freq_factor) {
      out[i] = f;
    } else if (w > L / o.low_freq_factor) {
      out[i] = f / o.factor;
    } else {
      const double s = (L / w - o.low_freq_factor) / (o.high_freq_factor - o.low_freq_factor);
      out[i] = (1.0 - s) * f / o.factor + s * f;
    }
  }
}

// Checks shared by every rotating entry point, in the order their status
// codes are documented: dtype, shape, theta, options.
int check_call(int dtype, int64_t nseq, int64_t T, int64_t Hq, int64_t Hkv, int64_t D, double theta,
               const rope_qk_options& o) {
  if (dtype != ROPE_QK_FP32 && dtype != ROPE_QK_BF16 && dtype != ROPE_QK_FP16) return ROPE_QK_ERR_DTYPE;
  if (nseq < 0 || T < 0 || Hq < 0 || Hkv < 0 || D < 2 || (D & 1) || D > 2 * kMaxHalf || T > INT32_MAX ||
      nseq >= INT32_MAX || Hq + Hkv > INT32_MAX)
    return ROPE_QK_ERR_SHAPE;
  if (!(theta > 0.0) || !isfinite(theta)) return ROPE_QK_ERR_THETA;
  const int64_t r = o.rotary_dim == 0 ? D : o.rotary_dim;  // elements of each head that are rotated
  if (o.pos_offset < 0 || o.pos_offset > INT32_MAX - T || r < 2 || (r & 1) || r > D ||
      (o.pairing != ROPE_QK_PAIR_HALF && o.pairing != ROPE_QK_PAIR_INTERLEAVED) ||
      (o.scaling != ROPE_QK_SCALING_NONE && o.scaling != ROPE_QK_SCALING_LLAMA3) ||
      (o.freq_precision != ROPE_QK_FREQ_FP64 && o.freq_precision != ROPE_QK_FREQ_FP32) || o.reserved != 0)
    return ROPE_QK_ERR_OPTION;
  if (o.scaling == ROPE_QK_SCALING_LLAMA3 &&
      !(o.factor > 0.0 && isfinite(o.factor) && o.original_max_position > 0.0 && isfinite(o.original_max_position) &&
        o.low_freq_factor > 0.0 && o.high_freq_factor > o.low_freq_factor && isfinite(o.high_freq_factor)))
    return ROPE_QK_ERR_OPTION;
  return ROPE_QK_OK;
}

// The frequency table of a call: make_inv_freq, then rounded to float32 for
// the float32 angle convention.
void fill_inv_freq(double theta, int64_t r, const rope_qk_options& o, double* out) {
  make_inv_freq(theta, r, o, out);
  if (o.freq_precision == ROPE_QK_FREQ_FP32)
    for (int i = 0; i < kMaxHalf; ++i) out[i] = static_cast<double>(static_cast<float>(out[i]));
}

}  // namespace

#endif  // ROPE_COMMON_H
