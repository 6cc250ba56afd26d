// Host-side layout checks of the rotation and norm calls: do a tensor's rows
// overlap each other, and do two tensors' rows share a byte.  Plain C++ with
// no HIP dependency, so the checks also build for CPU tests.

#ifndef ROPE_LAYOUT_H
#define ROPE_LAYOUT_H

#include <stdint.h>

namespace {

// Rows of D elements at t * st + h * sh (t < T, h < H), all strides >= 0: do any two overlap?
inline bool rows_overlap(int64_t T, int64_t H, int64_t D, int64_t st, int64_t sh) {
  if (T <= 1 && H <= 1) return false;
  if (T <= 1) return sh < D;
  if (H <= 1) return st < D;
  const int64_t s_small = st < sh ? st : sh, n_small = st < sh ? T : H;
  const int64_t s_big = st < sh ? sh : st;
  if (s_small < D) return true;
  return s_big / s_small < n_small;  // s_big < n_small * s_small, without overflow
}

// A [T, H] grid of rows of `row` bytes at base + t * st + h * sh (byte
// strides >= 0, T, H >= 1): its first byte and one past its last, in 128 bits.
struct Extent {
  __int128 lo, hi;
};

inline Extent rows_extent(const void* base, int64_t T, int64_t H, int64_t st, int64_t sh, int64_t row) {
  const __int128 lo = static_cast<__int128>(reinterpret_cast<uintptr_t>(base));
  return {lo, lo + static_cast<__int128>(T - 1) * st + static_cast<__int128>(H - 1) * sh + row};
}

// Do two [T, Ha] and [T, Hb] grids of rows (byte strides >= 0) share no
// byte?  Exact when their extents do not meet; otherwise true only for the
// fused-projection form: one token stride S for both, each token's rows
// within S bytes, and b's rows of a token in a gap of a's (offsets compared
// modulo S).  Any other meeting of the extents counts as an overlap.
inline bool rows_disjoint(const void* a, int64_t Ha, int64_t a_st, int64_t a_sh, const void* b, int64_t Hb,
                          int64_t b_st, int64_t b_sh, int64_t T, int64_t row) {
  if (T <= 0 || Ha <= 0 || Hb <= 0) return true;
  const Extent ea = rows_extent(a, T, Ha, a_st, a_sh, row), eb = rows_extent(b, T, Hb, b_st, b_sh, row);
  if (ea.hi <= eb.lo || eb.hi <= ea.lo) return true;
  if (T == 1 || a_st != b_st || a_st <= 0) return false;
  const __int128 S = a_st;
  const __int128 fa = static_cast<__int128>(Ha - 1) * a_sh + row;  // a token's span of a's rows
  const __int128 fb = static_cast<__int128>(Hb - 1) * b_sh + row;
  if (fa > S || fb > S) return false;
  __int128 d = (eb.lo - ea.lo) % S;
  if (d < 0) d += S;
  return d >= fa && d + fb <= S;
}

}  // namespace

#endif  // ROPE_LAYOUT_H
