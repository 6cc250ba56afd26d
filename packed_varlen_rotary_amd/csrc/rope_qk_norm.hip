// Fused per-head RMSNorm + rotary position embedding of q and k over packed
// variable-length batches, forward and backward, for AMD Instinct MI355X
// (CDNA4, gfx950).  The contract is documented with rope_qk_norm_fwd and
// rope_qk_norm_bwd in include/rope_qk.h.
//
// Sources: "Chronicals: A High-Performance Framework for LLM Fine-Tuning with
// 3.51x Speedup over Unsloth", abstract, optimisation (1) (RMSNorm and QK-RoPE
// among the fused kernels that remove memory traffic); RMSNorm as defined by
// Zhang and Sennrich (2019); its per-head placement before the rotation is
// the Qwen3 architecture's (a model family the pages name).
//
// Design (HBM-bound like the rotation: the forward reads and writes each
// element once, the backward reads x and dy and writes dx):
//
//  * Row tiles.  A row is one head of one token: D elements, 16 bytes of it
//    per lane on L = D*size/16 lanes, L a power of two from 2 to 64.  Lane l
//    of a workgroup holds part l % L of row u * (256 / L) + l / L of the
//    tile, for u < kTPT, so a row sits on L consecutive lanes of one wave and
//    each wave-wide load or store covers whole rows.  Interleaved pairs: the
//    part is chunk l % L (a pair inside a dword).  rotate_half pairs ("split"
//    rows): 8 bytes from each half of the row, so that both elements of every
//    pair sit in the lane and no lane exchange is needed.  A tile is a run of
//    whole rows in (token, head of q then k) order that may begin and end
//    inside a token.
//  * Per row: the sum of squares in float64, summed over the row's lanes by
//    a xor butterfly (ds_bpermute; every lane ends with the same bits),
//    r = 1/sqrt(mean + eps) from v_rsq_f64 and two Newton steps, then the
//    rotation; the table, built once per tile, holds one (A, B) entry per
//    element with the signs (and weights) in it, so that an element becomes
//    x_e A_e + x_p B_e.
//  * A tile holds rows of q only or of k only, so it needs one weight vector
//    and one set of weight-gradient sums.
//  * Backward: the rotation by -angle, then the RMSNorm gradient with a
//    second row sum (sum_j g_j x_j), summed over the row's lanes in the same
//    butterfly as the squares.  When every weight is finite and nonzero
//    the weights are folded into the per-element table, so the rotation of
//    dy yields g = w dn directly and the weight-gradient sums (of w dn x r)
//    are divided by w once at the end; otherwise the table has unit weights
//    and dn is multiplied by w.  A fixed number of workgroups each take a
//    contiguous run of tiles, carrying a cursor into cu_seqlens from tile to
//    tile, with one barrier per tile.  Each lane
//    keeps the weight-gradient terms of its rows in registers while the
//    tiles are of one tensor; then they are summed across the lanes of a
//    wave that hold the same chunk and across the 4 waves, into float64 sums
//    in LDS that the workgroup writes once at the end; a small kernel adds
//    the workgroups' sums in a fixed tree order, so the result is
//    deterministic.
//  * Rows of tokens in no sequence pass through unchanged; in the backward
//    they enter the arithmetic as zeros, with identity table entries.
//  * The kernels are instantiated per row width L, so the table offsets of a
//    row's elements are immediate offsets of its LDS reads.
//  * Everything is evaluated in float64 and rounded once to the storage type.

#include "rope_common.h"

#include <mutex>

namespace {

constexpr int kFwdTasks = 4;          // rows per lane per forward tile
constexpr int kBwdTasks = 2;          // rows per lane per backward tile (register-bound)
constexpr int64_t kMaxHeads = 65535;  // row -> (token, head) division limit
constexpr int kWaves = kThreads / 64;
constexpr int kFwdTableBytes = 32768;  // forward table per workgroup (one entry per element)
// Table entries (pairs, two 16-byte elements each) per thread, at most: the
// forward's one table, or each of the backward's two of kMaxTableBytes.
constexpr int kFwdEnt = kFwdTableBytes / 32 / kThreads;
constexpr int kBwdEnt = kMaxTableBytes / 32 / kThreads;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) u32x2 gu32x2;

// The elements of its row that a lane holds (kVec of them, 16 bytes).
// Interleaved pairs: chunk c, elements c kVec + j (a pair inside a dword).
// rotate_half pairs ("split" rows): kVec / 2 elements from each half, 8 bytes
// each, so that both elements of every pair sit in the lane: element j <
// kVec / 2 is c kVec / 2 + j of the first half, j >= kVec / 2 the same
// element of the second half (the partner of j is j ^ kVec / 2).  The offset
// of element j from element 0 in the row (half = kL kVec / 2):
template <bool kSplit, int kVec, int kL>
__device__ __forceinline__ constexpr int elem_off(int j) {
  return (kSplit && j >= kVec / 2) ? j - kVec / 2 + kL * kVec / 2 : j;
}

// Backward workgroups, each looping over a contiguous run of tiles: four
// times as many as the 256 compute units hold at once (3 per unit at the
// 16-bit kernels' 168 VGPRs, 4 for float32).  Units that run ahead then take
// more of the runs; with one run per resident slot the slowest unit sets the
// end (MI355X, Qwen3-8B and Qwen3-32B shapes: 3072 workgroups 3-8% faster
// than 768, level from 1536 to 6144).
constexpr int kBwdWaves16 = 3;
constexpr int64_t kBwdGroups16 = 4 * 256 * kBwdWaves16;
constexpr int64_t kBwdGroups32 = 4 * 256 * 4;
constexpr int64_t kBwdTilesPerRun = 8;   // fewer workgroups than the above when runs would be shorter
constexpr int64_t kBwdMinGroups = 768;   // ... but at least 3 per compute unit

// One of the two tensors (q, k) of a call.
struct NormTensor {
  const char* x;         // forward: input; backward: the forward's input
  const char* g;         // backward: incoming gradient of the forward's output
  char* o;               // forward: output; backward: gradient of the input
  const float* w;        // [D] weights
  int64_t x_st, x_sh;    // byte strides along tokens / heads
  int64_t g_st, g_sh;
  int64_t o_st, o_sh;
  uint64_t magic_heads;  // ceil(2^40 / H): exact n / H for n < 2^24
  double rcp_heads;      // 1 / H, rounded
  int32_t H;             // heads
  int32_t tile_rows;     // rows per tile
  uint32_t ntiles;
  int32_t copy;          // 1: tokens outside every sequence are copied to a separate output
  int32_t lin;           // 1: x, g and o are token-major (stride_t = H * stride_h), so row n sits at n * stride_h
};

struct NormParams {
  NormTensor ten[2];     // q, k; tiles [0, ten[0].ntiles) are q's, the rest k's
  double* partial;       // backward: [gridDim.x][2 D] weight-gradient sums per workgroup
  const int32_t* cu;     // cu_seqlens[nseq + 1]
  int64_t T;
  uint64_t magic_half;   // ceil(2^32 / half)
  double eps;
  double inv_d;          // 1 / D (exact: D is a power of two)
  double sign;           // +1 forward, -1 backward
  uint32_t ntiles;       // both tensors' tiles
  int32_t table_bytes;   // LDS bytes of the cos/sin table
  int32_t nseq;
  int32_t D;
  int32_t half;          // D / 2
  int32_t pos_offset;
  int32_t freq_fp32;
  double inv_freq[kMaxHalf];
  int32_t* pos_rows;     // positions hook only: [ntiles][pos_row_len] (first token, then positions)
  int64_t pos_row_len;
};

// The float64 value lane (addr / 4) holds (ds_bpermute, two dwords).
__device__ __forceinline__ double lane_f64(double v, int addr) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(addr, static_cast<int>(b)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(addr, static_cast<int>(b >> 32)));
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

// 1 / sqrt(a) for finite a > 0: the hardware estimate (relative error below
// 2^-23) refined by two Newton steps y <- y + y (1 - a y^2) / 2; the first
// leaves about 1.5 * 2^-46, the second ends at the float64 rounding, within
// one ulp of the correctly rounded value (a third step changes nothing more).
__device__ __forceinline__ double rsqrt_f64(double a) {
  double y = __builtin_amdgcn_rsq(a);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const double e = fma(-(a * y), y, 1.0);
    y = fma(0.5 * y, e, y);
  }
  return y;
}

// Elements 2d and 2d + 1 (16-bit storage) or element d (fp32) of a chunk as
// float64; for fp32 the second value is unused.
template <int kDtype>
__device__ __forceinline__ f64x2 element_pair(const u32x4& w, int d) {
  if constexpr (kDtype == ROPE_QK_FP32) {
    return f64x2{static_cast<double>(__uint_as_float(w[d])), 0.0};
  } else {
    return unpack16<kDtype>(w[d]);
  }
}

// Sum of squares of a chunk's elements, in float64.
template <int kDtype>
__device__ __forceinline__ double chunk_squares(const u32x4& a) {
  double ss = 0.0;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const f64x2 v = element_pair<kDtype>(a, d);
    ss = fma(v.x, v.x, ss);
    if constexpr (kDtype != ROPE_QK_FP32) ss = fma(v.y, v.y, ss);
  }
  return ss;
}

// The float64 value of the lane that DPP control kCtrl selects within the
// lane's row of 16 (two 32-bit DPP moves: there is no 64-bit DPP form for
// these controls on gfx950).
template <int kCtrl>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(static_cast<uint32_t>(b)), kCtrl,
                                                                     0xF, 0xF, false));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(static_cast<uint32_t>(b >> 32)),
                                                                     kCtrl, 0xF, 0xF, false));
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

// Sums over the L consecutive lanes of a row for kN rows at once (xor
// butterfly; a + b and b + a are the same float64, so every lane of a row
// ends with the same bits), so that the lane exchanges of the rows overlap.
// The first kDpp steps (at most the four inside a 16-lane DPP row) are DPP
// moves, which need no trip through the LDS crossbar: lane ^ 1 and lane ^ 2
// are quad permutations; once every quad holds one value, the half-row
// mirror (lane i with 7 - i) pairs quad 0 with quad 1 as lane ^ 4 does, and
// once every half row holds one value the row mirror (i with 15 - i) pairs
// the halves as lane ^ 8 does.  The same additions as the xor butterfly, so
// the same bits.  The remaining steps are ds_bpermute lane exchanges.
template <int kN, int kL, int kDpp>
__device__ __forceinline__ void row_sums(double* v, int lane) {
  constexpr int kQuadXor1 = 0xB1;       // quad_perm [1, 0, 3, 2]
  constexpr int kQuadXor2 = 0x4E;       // quad_perm [2, 3, 0, 1]
  constexpr int kRowHalfMirror = 0x141;
  constexpr int kRowMirror = 0x140;
  static_assert(kDpp >= 0 && kDpp <= 4, "at most the four steps inside a 16-lane row");
  if constexpr (kDpp >= 1 && kL >= 2) {
#pragma unroll
    for (int u = 0; u < kN; ++u) v[u] += dpp_f64<kQuadXor1>(v[u]);
    __builtin_amdgcn_sched_barrier(0);  // one step at a time, as measured
  }
  if constexpr (kDpp >= 2 && kL >= 4) {
#pragma unroll
    for (int u = 0; u < kN; ++u) v[u] += dpp_f64<kQuadXor2>(v[u]);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (kDpp >= 3 && kL >= 8) {
#pragma unroll
    for (int u = 0; u < kN; ++u) v[u] += dpp_f64<kRowHalfMirror>(v[u]);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (kDpp >= 4 && kL >= 16) {
#pragma unroll
    for (int u = 0; u < kN; ++u) v[u] += dpp_f64<kRowMirror>(v[u]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll 1
  for (int m = 1 << kDpp; m < kL; m <<= 1) {
    const int addr = (lane ^ m) << 2;
    double o[kN];
#pragma unroll
    for (int u = 0; u < kN; ++u) o[u] = lane_f64(v[u], addr);
#pragma unroll
    for (int u = 0; u < kN; ++u) v[u] += o[u];
  }
}

// The forward output of one lane's 16 bytes of a row from the weight-folded
// table: element e becomes r * (x_e * A_e + x_p * B_e), with p its pair
// partner (rotate_half: the same element of pr, the lane's other half of a
// split row; interleaved: its neighbour in the chunk) and (A_e, B_e) =
// (w_e cos, -w_p sin) for the first element of a pair, (w_e cos, w_p sin)
// for the second.  tab: the chunk's first entry, consecutive elements L
// entries apart.  16-bit storage: kExact selects the exact rounding; returns
// whether a value was hard for the fast one.
template <int kDtype, bool kIl, bool kExact>
__device__ __forceinline__ bool fwd_chunk(const u32x4& own, const u32x4& pr, double r, const double2* tab, int L,
                                          u32x4& out) {
  bool tie = false;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const f64x2 x = element_pair<kDtype>(own, d);
    if constexpr (kDtype == ROPE_QK_FP32) {
      const double xp = kIl ? element_pair<kDtype>(own, d ^ 1).x : element_pair<kDtype>(pr, d).x;
      const double2 c = tab[d * L];
      out[d] = __float_as_uint(static_cast<float>(r * fma(x.x, c.x, xp * c.y)));
    } else {
      double p0, p1;
      if constexpr (kIl) {
        p0 = x.y;
        p1 = x.x;
      } else {
        const f64x2 px = element_pair<kDtype>(pr, d);
        p0 = px.x;
        p1 = px.y;
      }
      const double2 c0 = tab[(2 * d) * L];
      const double2 c1 = tab[(2 * d + 1) * L];
      const double y0 = r * fma(x.x, c0.x, p0 * c0.y);
      const double y1 = r * fma(x.y, c1.x, p1 * c1.y);
      out[d] = kExact ? pack16_exact<kDtype>(y0, y1) : pack16_fast<kDtype>(y0, y1, tie);
    }
  }
  return tie;
}

// The incoming gradient of one lane's 16 bytes of a row rotated by -angle,
// from the per-element table (A_e, B_e): v_e = dy_e A_e + dy_p B_e, p the pair
// partner of element e (rotate_half: the same element of pr, the lane's other
// half of a split row; interleaved: its neighbour in the chunk).  With the weights folded into the table
// (A_e = w_e cos, B_e = -+w_e sin) v is g = w dn; with unit weights it is dn.
// tab: the chunk's first entry, consecutive elements L entries apart.
template <int kDtype, bool kIl>
__device__ __forceinline__ void bwd_chunk_rot(const u32x4& dy, const u32x4& pr, const double2* tab, int L,
                                              double* v) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const f64x2 dv = element_pair<kDtype>(dy, d);
    if constexpr (kDtype == ROPE_QK_FP32) {
      const double dp = kIl ? element_pair<kDtype>(dy, d ^ 1).x : element_pair<kDtype>(pr, d).x;
      const double2 c = tab[d * L];
      v[d] = fma(dv.x, c.x, dp * c.y);
    } else {
      double p0, p1;
      if constexpr (kIl) {
        p0 = dv.y;
        p1 = dv.x;
      } else {
        const f64x2 pv = element_pair<kDtype>(pr, d);
        p0 = pv.x;
        p1 = pv.y;
      }
      const double2 c0 = tab[(2 * d) * L];
      const double2 c1 = tab[(2 * d + 1) * L];
      v[2 * d] = fma(dv.x, c0.x, p0 * c0.y);
      v[2 * d + 1] = fma(dv.y, c1.x, p1 * c1.y);
    }
  }
}

// Backward of one chunk, first part: sum_j g_j x_j over its elements.  kFold:
// v is g already; otherwise v is dn and g = dn w, with element j's weight at
// w_own[elem_off(j)] (its offset in the row from the lane's element 0).
template <int kDtype, bool kFold, bool kSplit, int kL>
__device__ __forceinline__ double bwd_chunk_gx(const u32x4& x, const double* v, const float* w_own) {
  constexpr int kVec = kDtype == ROPE_QK_FP32 ? 4 : 8;
  double gx = 0.0;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const f64x2 xv = element_pair<kDtype>(x, d);
    if constexpr (kDtype == ROPE_QK_FP32) {
      gx = fma(kFold ? v[d] : v[d] * static_cast<double>(w_own[elem_off<kSplit, kVec, kL>(d)]), xv.x, gx);
    } else {
      gx = fma(kFold ? v[2 * d] : v[2 * d] * static_cast<double>(w_own[elem_off<kSplit, kVec, kL>(2 * d)]), xv.x,
               gx);
      gx = fma(kFold ? v[2 * d + 1] : v[2 * d + 1] * static_cast<double>(w_own[elem_off<kSplit, kVec, kL>(2 * d + 1)]),
               xv.y, gx);
    }
  }
  return gx;
}

// Backward of one chunk, second part: dx_j = r g_j - (x_j r) coef (that is
// r (g_j - x_j coef)), rounded, and (on the fast pass, not the exact redo)
// the weight-gradient term v_j x_j r added to acc: dn x r without the fold,
// w dn x r with it (the sums are divided by w once at the end).
template <int kDtype, bool kExact, bool kFold, bool kSplit, int kL>
__device__ __forceinline__ bool bwd_chunk_dx(const u32x4& x, const double* v, const float* w_own, double r,
                                             double coef, double* acc, u32x4& out) {
  constexpr int kVec = kDtype == ROPE_QK_FP32 ? 4 : 8;
  bool tie = false;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const f64x2 xv = element_pair<kDtype>(x, d);
    if constexpr (kDtype == ROPE_QK_FP32) {
      const double xr = xv.x * r;
      const double g = kFold ? v[d] : v[d] * static_cast<double>(w_own[elem_off<kSplit, kVec, kL>(d)]);
      out[d] = __float_as_uint(static_cast<float>(fma(-xr, coef, r * g)));
      if constexpr (!kExact) acc[d] = fma(v[d], xr, acc[d]);
    } else {
      const double xr0 = xv.x * r, xr1 = xv.y * r;
      const double g0 = kFold ? v[2 * d] : v[2 * d] * static_cast<double>(w_own[elem_off<kSplit, kVec, kL>(2 * d)]);
      const double g1 =
          kFold ? v[2 * d + 1] : v[2 * d + 1] * static_cast<double>(w_own[elem_off<kSplit, kVec, kL>(2 * d + 1)]);
      const double y0 = fma(-xr0, coef, r * g0);
      const double y1 = fma(-xr1, coef, r * g1);
      out[d] = kExact ? pack16_exact<kDtype>(y0, y1) : pack16_fast<kDtype>(y0, y1, tie);
      if constexpr (!kExact) {
        acc[2 * d] = fma(v[2 * d], xr0, acc[2 * d]);
        acc[2 * d + 1] = fma(v[2 * d + 1], xr1, acc[2 * d + 1]);
      }
    }
  }
  return tie;
}

// Scalar geometry of one tile: its tensor, first row n0 = t0 * H + r0, the
// tokens [t0, t_end) it touches and its table entries (tokens x pairs).
struct TileGeom {
  int sel;  // 0: q, 1: k
  uint32_t r0;
  int ntok, nent;
  int64_t n0, t0, n_end, t_end;
};

// The tensor descriptors are read by value (p.ten[sel] into registers):
// references into the kernel argument, selected between q's and k's, have
// made the compiler copy the whole argument (2.4 KB) to scratch memory.
__device__ __forceinline__ TileGeom tile_geom(const NormParams& p, uint32_t tile) {
  TileGeom gm;
  gm.sel = tile >= p.ten[0].ntiles ? 1 : 0;  // wave-uniform
  const NormTensor tn = p.ten[gm.sel];
  const uint32_t lt = tile - (gm.sel ? p.ten[0].ntiles : 0u);
  const int32_t H = tn.H;
  // n0 < 2^47 is exact in float64; the rounded quotient is off by at most one
  gm.n0 = static_cast<int64_t>(lt) * tn.tile_rows;
  int32_t t0i = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(static_cast<double>(gm.n0) * tn.rcp_heads));
  int64_t r0l = gm.n0 - static_cast<int64_t>(t0i) * H;
  if (r0l < 0) { t0i -= 1; r0l += H; }
  if (r0l >= H) { t0i += 1; r0l -= H; }
  gm.t0 = t0i;
  gm.r0 = static_cast<uint32_t>(r0l);
  gm.n_end = min(gm.n0 + tn.tile_rows, p.T * H);
  gm.ntok = static_cast<int>(div_tok(static_cast<uint32_t>(gm.n_end - gm.n0) + gm.r0 - 1, tn.magic_heads)) + 1;
  gm.t_end = gm.t0 + gm.ntok;
  gm.nent = gm.ntok * p.half;
  return gm;
}

// A lane's rows of one tile: the loaded chunks (x; backward also dy), where
// its outputs go, and which tile token each row belongs to.
template <int kTPT>
struct TileData {
  u32x4 a[kTPT], g[kTPT];
  gchar* optr[kTPT];
  int tt_of[kTPT];
  bool act[kTPT];
};

// a * b for b < 2^32 (its low word), as one 32 x 32 -> 64-bit multiply.
__device__ __forceinline__ int64_t mul_u32_wide(uint32_t a, int64_t b) {
  return static_cast<int64_t>(static_cast<uint64_t>(a) * static_cast<uint32_t>(b));
}

// One row's 16 bytes for this lane: a whole chunk, or (split rows) 8 bytes
// from each half of the row, the second kL * 8 bytes after the first.
template <bool kSplit, int kL>
__device__ __forceinline__ u32x4 row_load(const gchar* ptr) {
  if constexpr (kSplit) {
    const u32x2 lo = __builtin_nontemporal_load(reinterpret_cast<const gu32x2*>(ptr));
    const u32x2 hi = __builtin_nontemporal_load(reinterpret_cast<const gu32x2*>(ptr + kL * 8));
    return u32x4{lo.x, lo.y, hi.x, hi.y};
  } else {
    return __builtin_nontemporal_load(reinterpret_cast<const gu32x4*>(ptr));
  }
}

template <bool kSplit, int kL>
__device__ __forceinline__ void row_store(const u32x4& v, gchar* ptr) {
  if constexpr (kSplit) {
    __builtin_nontemporal_store(u32x2{v.x, v.y}, reinterpret_cast<gu32x2*>(ptr));
    __builtin_nontemporal_store(u32x2{v.z, v.w}, reinterpret_cast<gu32x2*>(ptr + kL * 8));
  } else {
    __builtin_nontemporal_store(v, reinterpret_cast<gu32x4*>(ptr));
  }
}

// Issue every load of a tile (rows past the tile's end re-read its first row).
template <bool kBwd, bool kSplit, int kTPT, int kL>
__device__ __forceinline__ void tile_loads(const NormParams& p, const TileGeom& gm, TileData<kTPT>& d) {
  const int tid = threadIdx.x;
  const NormTensor tn = p.ten[gm.sel];
  const int32_t H = tn.H;
  constexpr int rows_per_step = kThreads / kL;
  const int64_t off = static_cast<int64_t>(tid & (kL - 1)) * (kSplit ? 8 : 16);
  if (tn.lin) {
    // token-major rows: row n0 + lr at (n0 + lr) * stride_h, the tile's part
    // of it once per tile
    const gchar* xb = (const gchar*)tn.x + gm.n0 * tn.x_sh + off;
    const gchar* gb = kBwd ? (const gchar*)tn.g + gm.n0 * tn.g_sh + off : nullptr;
    gchar* ob = (gchar*)tn.o + gm.n0 * tn.o_sh + off;
#pragma unroll
    for (int u = 0; u < kTPT; ++u) {
      const int lr = u * rows_per_step + tid / kL;
      d.act[u] = gm.n0 + lr < gm.n_end;
      const uint32_t r = d.act[u] ? static_cast<uint32_t>(lr) : 0u;
      // head strides below 2^32 bytes (checked on the host for this form):
      // each row offset is one 32 x 32 -> 64-bit multiply
      d.a[u] = row_load<kSplit, kL>(xb + mul_u32_wide(r, tn.x_sh));
      if constexpr (kBwd) d.g[u] = row_load<kSplit, kL>(gb + mul_u32_wide(r, tn.g_sh));
      d.optr[u] = ob + mul_u32_wide(r, tn.o_sh);
      d.tt_of[u] = static_cast<int>(div_tok(gm.r0 + r, tn.magic_heads));
    }
    return;
  }
#pragma unroll
  for (int u = 0; u < kTPT; ++u) {
    const int lr = u * rows_per_step + tid / kL;
    d.act[u] = gm.n0 + lr < gm.n_end;
    const uint32_t l = d.act[u] ? gm.r0 + static_cast<uint32_t>(lr) : gm.r0;
    const uint32_t tt = div_tok(l, tn.magic_heads);
    const int64_t h = static_cast<int64_t>(l - tt * static_cast<uint32_t>(H));
    const int64_t t = gm.t0 + tt;
    d.a[u] = row_load<kSplit, kL>((const gchar*)tn.x + t * tn.x_st + h * tn.x_sh + off);
    if constexpr (kBwd) d.g[u] = row_load<kSplit, kL>((const gchar*)tn.g + t * tn.g_st + h * tn.g_sh + off);
    d.optr[u] = (gchar*)tn.o + t * tn.o_st + h * tn.o_sh + off;
    d.tt_of[u] = static_cast<int>(tt);
  }
}

// This thread's table entries e = tid + v * 256 of a tile: token and pair.
template <int kE>
__device__ __forceinline__ void tile_entries(const NormParams& p, const TileGeom& gm, int* tt_e, int* i_e) {
#pragma unroll
  for (int v = 0; v < kE; ++v) {
    const int e = threadIdx.x + v * kThreads;
    const int tt = e < gm.nent ? static_cast<int>(div_small(static_cast<uint32_t>(e), p.magic_half)) : 0;
    tt_e[v] = tt;
    i_e[v] = e < gm.nent ? e - tt * p.half : 0;
  }
}

// Where a tile's first token falls among the sequences: s0 is the last
// sequence that starts at or before it (-1: none), start0 = cu[s0] and next =
// cu[s0 + 1] (INT64_MIN / INT64_MAX past the ends).
struct SeqCursor {
  int32_t s0;
  int64_t start0, next;
};

__device__ __forceinline__ SeqCursor seq_cursor(const NormParams& p, int32_t s0) {
  const cu_ptr cu = (cu_ptr)p.cu;
  SeqCursor c;
  c.s0 = s0;
  c.start0 = s0 >= 0 ? static_cast<int64_t>(cu[s0]) : INT64_MIN;
  c.next = s0 < p.nseq ? static_cast<int64_t>(cu[s0 + 1]) : INT64_MAX;
  return c;
}

// The cursor moved on to token t0 >= the token it was made for (cu_seqlens
// non-decreasing): no memory read unless t0 has passed the next start.
__device__ __forceinline__ void seq_advance(const NormParams& p, SeqCursor& c, int64_t t0) {
  const cu_ptr cu = (cu_ptr)p.cu;
  while (c.next <= t0) {
    ++c.s0;
    c.start0 = c.next;
    c.next = c.s0 < p.nseq ? static_cast<int64_t>(cu[c.s0 + 1]) : INT64_MAX;
  }
}

// Positions and the table of a tile, from each entry's frequency f (and, for
// the forward, the weights w1, w2 of the pair's two elements); ends with a
// barrier.
// kPosOnly (the positions test hook): no table; the tile's first token and
// its tokens' positions go to pos_out[0 .. ntok] instead.
template <int kDtype, bool kIl, bool kBwd, int kL, bool kPosOnly = false>
__device__ __forceinline__ void tile_table(const NormParams& p, const TileGeom& gm, const int* tt_e, const int* i_e,
                                           const double* f, const float* w1, const float* w2,
                                           const SeqCursor& sc, int32_t* s_pos, double2* s_cs,
                                           int32_t* pos_out = nullptr) {
  constexpr int kVec = kDtype == ROPE_QK_FP32 ? 4 : 8;
  constexpr int L = kL;
  constexpr int kE = kBwd ? kBwdEnt : kFwdEnt;
  const cu_ptr cu = (cu_ptr)p.cu;
  const int32_t nseq = p.nseq;
  const int64_t cu_last = cu[nseq];
  const int64_t cu_first_end = nseq >= 1 ? static_cast<int64_t>(cu[1]) : INT64_MIN;  // cu[1] exists only then
  int64_t start[kE];
#pragma unroll
  for (int v = 0; v < kE; ++v) start[v] = sc.start0;
  // the sequence starts inside the tile
  int64_t cv = sc.next;
  for (int32_t j = sc.s0 + 1; cv < gm.t_end;) {
#pragma unroll
    for (int v = 0; v < kE; ++v) start[v] = cv <= gm.t0 + tt_e[v] ? cv : start[v];
    ++j;
    cv = j <= nseq ? static_cast<int64_t>(cu[j]) : INT64_MAX;
  }
#pragma unroll
  for (int v = 0; v < kE; ++v) {
    if (v > 0 && v * kThreads >= gm.nent) break;
    const int e = threadIdx.x + v * kThreads;
    const int64_t t = gm.t0 + tt_e[v];
    const bool inside = start[v] != INT64_MIN && t < cu_last;
    const int64_t pos64 = inside ? t - start[v] + (t < cu_first_end ? p.pos_offset : 0) : -1;
    const int32_t pos = pos64 <= INT32_MAX ? static_cast<int32_t>(pos64) : -1;
    if (e < gm.nent) {
      if (i_e[v] == 0) s_pos[tt_e[v]] = pos;
      if constexpr (kPosOnly) {
        if (i_e[v] == 0) pos_out[1 + tt_e[v]] = pos;
        if (e == 0) pos_out[0] = static_cast<int32_t>(gm.t0);
        continue;
      }
      // one entry per element: lane c's element j of token tt at (tt * kVec
      // + j) * L + c (lanes read consecutive slots); the pair's elements:
      // interleaved 2 i and 2 i + 1 of chunk i / (kVec / 2), rotate_half
      // (split rows) i and i + half, both in lane i / (kVec / 2)
      const int i = i_e[v];
      const int c = i / (kVec / 2);
      const int j1 = kIl ? 2 * (i % (kVec / 2)) : i % (kVec / 2);
      const int j2 = kIl ? j1 + 1 : j1 + kVec / 2;
      double2* slot1 = s_cs + (tt_e[v] * kVec + j1) * L + c;
      double2* slot2 = s_cs + (tt_e[v] * kVec + j2) * L + c;
      if (pos >= 0) {
        double sn, cs;
        const double ang = p.freq_fp32 ? static_cast<double>(static_cast<float>(pos) * static_cast<float>(f[v]))
                                       : static_cast<double>(pos) * f[v];
        rope_sincos(ang, &sn, &cs);
        const double a = static_cast<double>(w1[v]), b = static_cast<double>(w2[v]);
        if constexpr (kBwd) {
          // the rotation by -angle (p.sign = -1: the first element of a pair
          // takes +sin times its partner, the second -sin), each entry
          // scaled by its own element's weight (1 when not folded)
          const double s2 = p.sign * sn;
          *slot1 = make_double2(a * cs, -(a * s2));
          *slot2 = make_double2(b * cs, b * s2);
        } else {
          *slot1 = make_double2(a * cs, -(b * sn));
          *slot2 = make_double2(b * cs, a * sn);
        }
      } else if constexpr (kBwd) {
        // a token in no sequence: its rows enter the backward as zeros and
        // must stay zeros through the rotation, so its entries are the
        // identity rather than whatever an earlier kernel left in this LDS
        // (0 times a stale NaN would reach the weight-gradient sums)
        *slot1 = make_double2(1.0, 0.0);
        *slot2 = make_double2(1.0, 0.0);
      }
    }
  }
  __syncthreads();
}

// Every row of a tile (after its table).  Forward: r for all rows (their
// lane sums together), then the rows one at a time.  Backward, in phases:
// the squares, the rotation of dy and the lane's part of sum g x; both row
// sums of all rows in one butterfly; r; dx and the weight-gradient terms.
// Then the stores.  s_w holds both tensors' weights (q then k); acc
// (backward) receives this lane's weight-gradient terms.  kFold (backward):
// the table carries the weights, so the rotation gives g = w dn directly and
// acc receives w dn x r.
template <int kDtype, bool kIl, bool kBwd, int kTPT, int kL, bool kFold = false>
__device__ __forceinline__ void tile_compute(const NormParams& p, const TileGeom& gm, const TileData<kTPT>& d,
                                             const int32_t* s_pos, const double2* s_cs, const float* s_w,
                                             double* acc) {
  constexpr int kVec = kDtype == ROPE_QK_FP32 ? 4 : 8;  // elements per lane and row
  constexpr bool kSplit = !kIl;                         // rotate_half: split rows
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  constexpr int L = kL;
  const int c = tid & (L - 1);
  const int sel = gm.sel;
  const NormTensor tn = p.ten[sel];
  const int* tt_of = d.tt_of;
  const bool* act = d.act;
  const bool copy = tn.copy != 0;
  bool st[kTPT], inside[kTPT];
  u32x4 out[kTPT];
  double r[kTPT];
  // backward: the rows that are in no sequence (or past the tile's end)
  // enter as zeros, so they add exactly nothing to the weight gradient
  // whatever they hold; their outputs are not computed from these
  u32x4 a[kTPT], g[kTPT];
#pragma unroll
  for (int u = 0; u < kTPT; ++u) {
    inside[u] = s_pos[tt_of[u]] >= 0;
    st[u] = act[u] & (inside[u] | copy);
    const bool use = !kBwd || (act[u] & inside[u]);
    const u32x4 zero = {0u, 0u, 0u, 0u};
    a[u] = use ? d.a[u] : zero;
    if constexpr (kBwd) g[u] = use ? d.g[u] : zero;
    r[u] = chunk_squares<kDtype>(a[u]);
  }
  if constexpr (!kBwd) {
    // the two quad steps as DPP moves; the others would raise the register
    // count past 128 and cost the fourth wave (so would the quad steps on
    // interleaved 16-bit rows of 4 or 8 lanes: 125 -> 131 VGPRs)
    constexpr int kFwdDpp = kIl && kDtype != ROPE_QK_FP32 && kL < 16 ? 0 : 2;
    row_sums<kTPT, kL, kFwdDpp>(r, lane);
#pragma unroll
    for (int u = 0; u < kTPT; ++u) r[u] = rsqrt_f64(fma(r[u], p.inv_d, p.eps));
#pragma unroll
    for (int u = 0; u < kTPT; ++u) {
      // one row at a time: interleaving rows would keep several rows' float64
      // values live and cut the occupancy
      __builtin_amdgcn_sched_barrier(0);
      const double2* tab = s_cs + tt_of[u] * kVec * L + c;
      // rotate_half partners: the lane's other half (signs are in the table)
      const u32x4 pr = kSplit ? u32x4{a[u].z, a[u].w, a[u].x, a[u].y} : a[u];
      u32x4 y;
      if (fwd_chunk<kDtype, kIl, false>(a[u], pr, r[u], tab, L, y)) fwd_chunk<kDtype, kIl, true>(a[u], pr, r[u], tab, L, y);
      out[u] = inside[u] ? y : a[u];
    }
  } else {
    const float* w_own = s_w + sel * (kL * kVec) + c * (kSplit ? kVec / 2 : kVec);  // read only when not folded
    // v (g when folded, else dn) stays in registers from the first pass to
    // the second; the weight-gradient terms are added in the second, where x
    // is unpacked again anyway (in the first they kept x's float64 values
    // live longer: 185 against 168 VGPRs, 2 against 3 waves per SIMD)
    double gx[kTPT];
    double v[kTPT][kVec];
#pragma unroll
    for (int u = 0; u < kTPT; ++u) {
      __builtin_amdgcn_sched_barrier(0);
      const double2* tab = s_cs + tt_of[u] * kVec * L + c;
      const u32x4 pr = kSplit ? u32x4{g[u].z, g[u].w, g[u].x, g[u].y} : g[u];
      bwd_chunk_rot<kDtype, kIl>(g[u], pr, tab, L, v[u]);
      gx[u] = bwd_chunk_gx<kDtype, kFold, kSplit, kL>(a[u], v[u], w_own);
    }
    __builtin_amdgcn_sched_barrier(0);
    // both row sums (of x^2 and of g x; neither needs the other) go through
    // one butterfly, one chain of lane exchanges instead of two; DPP moves
    // for every step inside a 16-lane row
    double sums[2 * kTPT];
#pragma unroll
    for (int u = 0; u < kTPT; ++u) {
      sums[u] = r[u];
      sums[kTPT + u] = gx[u];
    }
    row_sums<2 * kTPT, kL, 4>(sums, lane);
#pragma unroll
    for (int u = 0; u < kTPT; ++u) {
      r[u] = rsqrt_f64(fma(sums[u], p.inv_d, p.eps));
      gx[u] = sums[kTPT + u];
    }
#pragma unroll
    for (int u = 0; u < kTPT; ++u) {
      __builtin_amdgcn_sched_barrier(0);
      const double coef = (r[u] * r[u]) * (gx[u] * p.inv_d);
      u32x4 y;
      if (bwd_chunk_dx<kDtype, false, kFold, kSplit, kL>(a[u], v[u], w_own, r[u], coef, acc, y))
        bwd_chunk_dx<kDtype, true, kFold, kSplit, kL>(a[u], v[u], w_own, r[u], coef, acc, y);
      out[u] = inside[u] ? y : d.g[u];
    }
  }
#pragma unroll
  for (int u = 0; u < kTPT; ++u) {
    if (!st[u]) continue;
    row_store<kSplit, kL>(out[u], d.optr[u]);
  }
}

// The forward tile: its frequencies and weights are loaded before its data.
// kPosOnly: the positions hook (see tile_table).
template <int kDtype, bool kIl, int kTPT, int kL, bool kPosOnly = false>
__device__ __forceinline__ void fwd_tile(const NormParams& p, uint32_t tile, int32_t* s_pos, double2* s_cs,
                                         int32_t* pos_out = nullptr) {
  const TileGeom gm = tile_geom(p, tile);
  const NormTensor tn = p.ten[gm.sel];
  int tt_e[kFwdEnt], i_e[kFwdEnt];
  tile_entries<kFwdEnt>(p, gm, tt_e, i_e);
  double f[kFwdEnt];
  float w1[kFwdEnt], w2[kFwdEnt];
#pragma unroll
  for (int v = 0; v < kFwdEnt; ++v) {
    const bool live = v == 0 || v * kThreads < gm.nent;
    f[v] = live ? p.inv_freq[i_e[v]] : 0.0;
    if constexpr (kPosOnly) {  // the hook has no weights
      w1[v] = w2[v] = 0.f;
    } else {
      w1[v] = live ? tn.w[kIl ? 2 * i_e[v] : i_e[v]] : 0.f;
      w2[v] = live ? tn.w[kIl ? 2 * i_e[v] + 1 : i_e[v] + p.half] : 0.f;
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  TileData<kTPT> d;
  if constexpr (!kPosOnly) tile_loads<false, !kIl, kTPT, kL>(p, gm, d);
  __builtin_amdgcn_sched_barrier(0);
  const SeqCursor sc = seq_cursor(p, last_start_at_or_before((cu_ptr)p.cu, p.nseq, gm.t0));
  tile_table<kDtype, kIl, false, kL, kPosOnly>(p, gm, tt_e, i_e, f, w1, w2, sc, s_pos, s_cs, pos_out);
  if constexpr (!kPosOnly) tile_compute<kDtype, kIl, false, kTPT, kL>(p, gm, d, s_pos, s_cs, nullptr, nullptr);
}

// LDS of the norm kernels after the table (the forward's one, the backward's
// two): weights [2 D] floats, then (backward) the workgroup's weight-gradient
// sums [2 D], the per-wave sums of one flush [4][D] and the frequencies
// [D / 2], doubles.
__device__ __forceinline__ float* lds_weights(double2* s_cs, const NormParams& p, int ntables) {
  return reinterpret_cast<float*>(reinterpret_cast<char*>(s_cs) + ntables * p.table_bytes);
}

// Both tensors' weights into LDS (a tensor without heads may have none).
__device__ __forceinline__ void load_weights(const NormParams& p, float* s_w) {
  for (int i = threadIdx.x; i < p.D / 2; i += kThreads) {  // float4s of the 2 D weights
    const bool of_k = i * 4 >= p.D;
    const float* base = p.ten[of_k ? 1 : 0].w;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (base != nullptr) v = *reinterpret_cast<const float4*>(base + (of_k ? i * 4 - p.D : i * 4));
    reinterpret_cast<float4*>(s_w)[i] = v;
  }
}

// Forward: one tile per workgroup.
template <int kDtype, bool kIl, int kTPT, int kL>
__global__ __launch_bounds__(kThreads) void rope_qk_norm_fwd_kernel(const NormParams p) {
  __shared__ int32_t s_pos[kMaxTileTokens];
  extern __shared__ double2 s_cs[];
  const uint32_t tile = blockIdx.y * gridDim.x + blockIdx.x;
  if (tile >= p.ntiles) return;
  fwd_tile<kDtype, kIl, kTPT, kL>(p, tile, s_pos, s_cs);
}

// The positions hook of the forward: one tile per workgroup through the
// forward tile's own geometry, sequence search and position code.
__global__ __launch_bounds__(kThreads) void rope_qk_norm_fwd_positions_kernel(const NormParams p) {
  __shared__ int32_t s_pos[kMaxTileTokens];
  const uint32_t tile = blockIdx.y * gridDim.x + blockIdx.x;
  if (tile >= p.ntiles) return;
  fwd_tile<ROPE_QK_BF16, false, kFwdTasks, 8, true>(p, tile, s_pos, nullptr,
                                                    p.pos_rows + static_cast<int64_t>(tile) * p.pos_row_len);
}

// Adds this thread's weight-gradient terms of tensor `sel` into the
// workgroup's sums: across the lanes of a wave that hold the same chunk, then
// across the waves (in a fixed order); ends with a barrier.  kSplit: the
// lane's elements are those of a split row (elem_off).
template <int kVec, int kL, bool kSplit>
__device__ __forceinline__ void flush_dw(const NormParams& p, int sel, const double* acc, double* s_wave,
                                         double* s_acc) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int L = kL, D = kL * kVec;
  const int c = tid & (L - 1);
  double v[kVec];
#pragma unroll
  for (int j = 0; j < kVec; ++j) v[j] = acc[j];
  for (int m = L; m < 64; m <<= 1) {
    const int addr = (lane ^ m) << 2;
#pragma unroll
    for (int j = 0; j < kVec; ++j) v[j] += lane_f64(v[j], addr);
  }
  if (lane < L) {
#pragma unroll
    for (int j = 0; j < kVec; ++j) s_wave[wave * D + c * (kSplit ? kVec / 2 : kVec) + elem_off<kSplit, kVec, kL>(j)] = v[j];
  }
  __syncthreads();
  for (int col = tid; col < D; col += kThreads) {
    double s = s_wave[col];
#pragma unroll
    for (int wv = 1; wv < kWaves; ++wv) s += s_wave[wv * D + col];
    s_acc[sel * D + col] += s;
  }
  __syncthreads();
}

// The loop of the backward kernel over its workgroup's run of tiles, then
// the workgroup's weight-gradient sums.  kFold: the tables carry the weights
// (see rope_qk_norm_bwd_kernel).  Instantiated once per kFold, so that each
// loop gets its own register allocation.
template <int kDtype, bool kIl, int kTPT, int kL, bool kPosOnly, bool kFold>
__device__ __forceinline__ void bwd_runs(const NormParams& p, int32_t (*s_pos)[kMaxTileTokens], double2* s_cs,
                                         float* s_w, double* s_acc, double* s_wave, double* s_freq) {
  constexpr int kVec = kDtype == ROPE_QK_FP32 ? 4 : 8;
  const int tab_len = p.table_bytes / static_cast<int>(sizeof(double2));  // entries per table
  const int tid = threadIdx.x;
  const int D = p.D;
  double acc[kVec];
#pragma unroll
  for (int j = 0; j < kVec; ++j) acc[j] = 0.0;
  int cur = -1;  // the tensor acc belongs to
  int b = 0;     // this tile's table
  // a contiguous run of tiles per workgroup, so that each tile's first
  // sequence is found by stepping on from the previous tile's (usually with
  // no memory read: a search per tile is a chain of dependent reads that the
  // tile's table, and so its barrier, would wait for)
  const uint32_t per = p.ntiles / gridDim.x, extra = p.ntiles % gridDim.x;
  const uint32_t first = blockIdx.x * per + min(blockIdx.x, extra);
  const uint32_t end = first + per + (blockIdx.x < extra ? 1u : 0u);
  SeqCursor sc = {-1, INT64_MIN, INT64_MAX};
  for (uint32_t tile = first; tile < end; ++tile) {
    const TileGeom gm = tile_geom(p, tile);
    const bool fresh = gm.sel != cur;
    if (fresh) {
      if constexpr (!kPosOnly) {
        if (cur >= 0) flush_dw<kVec, kL, !kIl>(p, cur, acc, s_wave, s_acc);
#pragma unroll
        for (int j = 0; j < kVec; ++j) acc[j] = 0.0;
      }
      cur = gm.sel;
    }
    TileData<kTPT> d;
    if constexpr (!kPosOnly) tile_loads<true, !kIl, kTPT, kL>(p, gm, d);
    __builtin_amdgcn_sched_barrier(0);
    if (fresh)
      sc = seq_cursor(p, last_start_at_or_before((cu_ptr)p.cu, p.nseq, gm.t0));
    else
      seq_advance(p, sc, gm.t0);
    int tt_e[kBwdEnt], i_e[kBwdEnt];
    double f[kBwdEnt];
    float w1[kBwdEnt], w2[kBwdEnt];
    tile_entries<kBwdEnt>(p, gm, tt_e, i_e);
#pragma unroll
    for (int v = 0; v < kBwdEnt; ++v) {
      f[v] = kPosOnly ? 0.0 : s_freq[i_e[v]];
      const float* wt = s_w + gm.sel * D;
      w1[v] = kFold ? wt[kIl ? 2 * i_e[v] : i_e[v]] : 1.f;
      w2[v] = kFold ? wt[kIl ? 2 * i_e[v] + 1 : i_e[v] + p.half] : 1.f;
    }
    if constexpr (kPosOnly) {
      tile_table<kDtype, kIl, true, kL, true>(p, gm, tt_e, i_e, f, w1, w2, sc, s_pos[b], nullptr,
                                              p.pos_rows + static_cast<int64_t>(tile) * p.pos_row_len);
    } else {
      tile_table<kDtype, kIl, true, kL>(p, gm, tt_e, i_e, f, w1, w2, sc, s_pos[b], s_cs + b * tab_len);
      tile_compute<kDtype, kIl, true, kTPT, kL, kFold>(p, gm, d, s_pos[b], s_cs + b * tab_len, s_w, acc);
    }
    b ^= 1;
  }
  if constexpr (!kPosOnly) {
    if (cur >= 0) flush_dw<kVec, kL, !kIl>(p, cur, acc, s_wave, s_acc);
    double* dst = p.partial + static_cast<int64_t>(blockIdx.x) * 2 * D;
    for (int i = tid; i < 2 * D; i += kThreads) {
      double sum = s_acc[i];
      if (kFold && p.ten[i < D ? 0 : 1].H > 0) sum /= static_cast<double>(s_w[i]);  // sums of w dn x r
      dst[i] = sum;
    }
  }
}

// Backward: gridDim.x workgroups, each taking a contiguous run of tiles; the
// weights and frequencies sit in LDS for all of a workgroup's tiles.
// Consecutive tiles alternate between two tables, so one barrier per tile
// (after its table) suffices: a wave that writes table b for tile i has passed
// tile i - 1's barrier, which every wave reaches only after its tile i - 2
// work, the last reader of table b.  The weight-gradient terms stay in
// registers while the tiles are of one tensor (q's tiles come first, so that
// changes at most once) and are summed across the workgroup only then and at
// the end.
// kPosOnly (the positions test hook): the same runs of tiles and the same
// sequence cursor, writing each tile's first token and positions to row
// `tile` of p.pos_rows; nothing is loaded, computed or stored.
template <int kDtype, bool kIl, int kTPT, int kL, bool kPosOnly = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kBwdWaves16)))
void rope_qk_norm_bwd_kernel(const NormParams p) {
  __shared__ int32_t s_pos[2][kMaxTileTokens];
  extern __shared__ double2 s_cs[];
  float* s_w = lds_weights(s_cs, p, 2);
  double* s_acc = reinterpret_cast<double*>(s_w + 2 * p.D);  // [2 D]
  double* s_wave = s_acc + 2 * p.D;                          // [kWaves][D]
  double* s_freq = s_wave + kWaves * p.D;                    // [D / 2]
  const int tid = threadIdx.x;
  const int D = p.D;
  if constexpr (!kPosOnly) {
    load_weights(p, s_w);
    for (int i = tid; i < 2 * D; i += kThreads) s_acc[i] = 0.0;
    for (int i = tid; i < p.half; i += kThreads) s_freq[i] = p.inv_freq[i];
    __syncthreads();
  }
  // Fold the weights into the tables when every weight of a tensor with
  // heads is finite and nonzero (the usual case): the rotation then yields
  // g = w dn directly, and the weight-gradient sums of w dn x r are divided
  // by w at the end.  Otherwise dn is rotated with unit weights and
  // multiplied by w.  Every wave reads all weights itself (wave-uniform, no
  // barrier).
  bool fold = false;
  if constexpr (!kPosOnly) {
    bool bad = false;
    for (int i = tid & 63; i < 2 * D; i += 64) {
      const float w = s_w[i];
      bad |= p.ten[i < D ? 0 : 1].H > 0 && !(w != 0.f && fabsf(w) < __builtin_inff());
    }
    fold = __ballot(bad) == 0;
  }
  if constexpr (kPosOnly)
    bwd_runs<kDtype, kIl, kTPT, kL, true, false>(p, s_pos, s_cs, s_w, s_acc, s_wave, s_freq);
  else if (fold)
    bwd_runs<kDtype, kIl, kTPT, kL, false, true>(p, s_pos, s_cs, s_w, s_acc, s_wave, s_freq);
  else
    bwd_runs<kDtype, kIl, kTPT, kL, false, false>(p, s_pos, s_cs, s_w, s_acc, s_wave, s_freq);
}

// The weight gradients: one column of the workgroups' sums per workgroup,
// added in a fixed tree order, rounded once to float32.  Workgroups go to
// the 8 XCDs in turn (blockIdx.x % 8), each XCD with its own L2, so XCD x
// takes a contiguous range of columns: the columns that share a 128-byte
// line of a row are summed on one XCD, and each line comes from HBM once
// rather than once per XCD.  (The order only places work; the sums are the
// same whatever XCD runs them.)
constexpr int kXcds = 8;

__global__ __launch_bounds__(kThreads) void dw_reduce_kernel(const double* __restrict__ partial, uint32_t ngroups,
                                                            int32_t D, float* __restrict__ dwq,
                                                            float* __restrict__ dwk) {
  __shared__ double s[kThreads];
  const int per_xcd = gridDim.x / kXcds;  // the grid is kXcds * ceil(2 D / kXcds) workgroups
  const int col = static_cast<int>(blockIdx.x % kXcds) * per_xcd + static_cast<int>(blockIdx.x / kXcds);
  if (col >= 2 * D) return;
  const int tid = threadIdx.x;
  double acc = 0.0;
  for (uint32_t i = tid; i < ngroups; i += kThreads) acc += partial[static_cast<int64_t>(i) * 2 * D + col];
  s[tid] = acc;
  __syncthreads();
  for (int width = kThreads / 2; width > 0; width >>= 1) {
    if (tid < width) s[tid] += s[tid + width];
    __syncthreads();
  }
  if (tid == 0) {
    const float v = static_cast<float>(s[0]);
    if (col < D) {
      if (dwq != nullptr) dwq[col] = v;
    } else if (dwk != nullptr) {
      dwk[col - D] = v;
    }
  }
}

struct Tensor {
  const void* base;
  int64_t st, sh;  // element strides
};

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) % 16) == 0; }

// Geometry shared by the forward, the backward and the workspace query.
struct NormGeometry {
  int64_t L = 0;
  int64_t tile_rows[2] = {0, 0};
  int64_t ntiles[2] = {0, 0};
  int64_t span = 0;    // most tokens one tile touches
  int64_t table_bytes = 0;
  int64_t groups = 0;  // backward workgroups
};

int norm_geometry(int64_t T, int64_t Hq, int64_t Hkv, int64_t D, int dtype, bool s_bwd, NormGeometry* g) {
  const int64_t esz = dtype == ROPE_QK_FP32 ? 4 : 2;
  const int64_t L = D * esz / 16;
  if ((D * esz) % 16 || L < 2 || L > 64 || (L & (L - 1))) return ROPE_QK_ERR_SHAPE;
  if (Hq > kMaxHeads || Hkv > kMaxHeads) return ROPE_QK_ERR_SHAPE;
  // table bytes per token: one (cos, sin) entry per element, scaled by weights
  const int64_t per_token = D * 16;
  int64_t cap_tokens = (s_bwd ? kMaxTableBytes : kFwdTableBytes) / per_token;
  if (cap_tokens > kMaxTileTokens) cap_tokens = kMaxTileTokens;
  g->L = L;
  g->span = 0;
  const int64_t Hs[2] = {Hq, Hkv};
  for (int s = 0; s < 2; ++s) {
    const int64_t H = Hs[s];
    int64_t rows = int64_t(s_bwd ? kBwdTasks : kFwdTasks) * (kThreads / L);
    if (H > 0 && rows > (cap_tokens - 1) * H) rows = (cap_tokens - 1) * H;
    g->tile_rows[s] = rows;
    g->ntiles[s] = H > 0 ? (T * H + rows - 1) / rows : 0;
    if (H > 0) {
      const int64_t span = rows % H == 0 ? rows / H : (H + rows - 2) / H + 1;  // tokens one tile touches
      if (span > g->span) g->span = span;
    }
  }
  g->table_bytes = g->span * per_token;
  const int64_t total = g->ntiles[0] + g->ntiles[1];
  if (total > INT32_MAX) return ROPE_QK_ERR_SHAPE;
  // runs of at least ~8 tiles (but no fewer than 768 workgroups, three per
  // compute unit): with shorter runs each workgroup's own work (weights into
  // LDS, its weight-gradient sums, the reduction's share of them) outweighs
  // its tiles (the Qwen2.5-0.5B-shaped backward took 47.7 us with 3072
  // workgroups of under 3 tiles each, 35.3 us with 1024 of 8)
  const int64_t most = dtype == ROPE_QK_FP32 ? kBwdGroups32 : kBwdGroups16;
  int64_t groups = total / kBwdTilesPerRun;
  if (groups < kBwdMinGroups) groups = kBwdMinGroups;
  if (groups > most) groups = most;
  g->groups = total < groups ? total : groups;
  return ROPE_QK_OK;
}

int64_t workspace_bytes(const NormGeometry& g, int64_t D) {
  return g.groups * 2 * D * static_cast<int64_t>(sizeof(double));
}

// Everything both passes check: the shared call checks, the norm's own limits
// (eps, full rotary dim, row shape) and each tensor's alignment and layout.
int check_norm_call(int dtype, int64_t nseq, int64_t T, int64_t Hq, int64_t Hkv, int64_t D, double theta,
                    const rope_qk_options& o, double eps, const float* wq, const float* wk, const Tensor* ts,
                    int nts, bool bwd, NormGeometry* g) {
  int status = check_call(dtype, nseq, T, Hq, Hkv, D, theta, o);
  if (status != ROPE_QK_OK) return status;
  if (!(eps > 0.0) || !isfinite(eps) || (o.rotary_dim != 0 && o.rotary_dim != D)) return ROPE_QK_ERR_OPTION;
  status = norm_geometry(T, Hq, Hkv, D, dtype, bwd, g);
  if (status != ROPE_QK_OK) return status;
  if (T == 0 || Hq + Hkv == 0) return ROPE_QK_OK;
  if ((Hq > 0 && wq == nullptr) || (Hkv > 0 && wk == nullptr)) return ROPE_QK_ERR_NULL;
  const int64_t esz = dtype == ROPE_QK_FP32 ? 4 : 2;
  for (int i = 0; i < nts; ++i) {
    const int64_t H = (i % 2 == 0) ? Hq : Hkv;  // tensors alternate q, k
    if (H == 0) continue;
    if (ts[i].base == nullptr) return ROPE_QK_ERR_NULL;
    if (!aligned16(ts[i].base) || (ts[i].st * esz) % 16 || (ts[i].sh * esz) % 16) return ROPE_QK_ERR_ALIGN;
    if (ts[i].st < 0 || ts[i].sh < 0 || rows_overlap(T, H, D, ts[i].st, ts[i].sh)) return ROPE_QK_ERR_LAYOUT;
  }
  // the last two tensors are written (q's, then k's): each must be exactly
  // its own input (in place: ts[i - first_out]) or share no byte with any
  // other tensor of the call
  const int first_out = nts - 2;
  for (int i = first_out; i < nts; ++i) {
    const int64_t Hi = (i % 2 == 0) ? Hq : Hkv;
    for (int j = 0; j < nts; ++j) {
      const int64_t Hj = (j % 2 == 0) ? Hq : Hkv;
      if (j == i || Hi == 0 || Hj == 0) continue;
      const Tensor& a = ts[i];
      const Tensor& b = ts[j];
      if (j == i - first_out && a.base == b.base && a.st == b.st && a.sh == b.sh) continue;
      if (!rows_disjoint(a.base, Hi, a.st * esz, a.sh * esz, b.base, Hj, b.st * esz, b.sh * esz, T, D * esz))
        return ROPE_QK_ERR_LAYOUT;
    }
  }
  if ((Hq > 0 && !aligned16(wq)) || (Hkv > 0 && !aligned16(wk))) return ROPE_QK_ERR_ALIGN;
  return ROPE_QK_OK;
}

void fill_params(NormParams* p, const NormGeometry& g, const int32_t* cu, int64_t nseq, int64_t T, int64_t Hq,
                 int64_t Hkv, int64_t D, double theta, double eps, const rope_qk_options& o, const float* wq,
                 const float* wk, double sign) {
  const int64_t Hs[2] = {Hq, Hkv};
  const float* ws[2] = {wq, wk};
  for (int s = 0; s < 2; ++s) {
    NormTensor& tn = p->ten[s];
    const int64_t H = Hs[s] > 0 ? Hs[s] : 1;
    tn.w = ws[s];
    tn.magic_heads = ((uint64_t(1) << 40) + H - 1) / H;
    tn.rcp_heads = 1.0 / static_cast<double>(H);
    tn.H = static_cast<int32_t>(Hs[s]);
    tn.tile_rows = static_cast<int32_t>(g.tile_rows[s]);
    tn.ntiles = static_cast<uint32_t>(g.ntiles[s]);
  }
  p->cu = cu;
  p->T = T;
  p->magic_half = ((uint64_t(1) << 32) + D / 2 - 1) / (D / 2);
  p->eps = eps;
  p->inv_d = 1.0 / static_cast<double>(D);
  p->sign = sign;
  p->ntiles = static_cast<uint32_t>(g.ntiles[0] + g.ntiles[1]);
  p->table_bytes = static_cast<int32_t>(g.table_bytes);
  p->nseq = static_cast<int32_t>(nseq);
  p->D = static_cast<int32_t>(D);
  p->half = static_cast<int32_t>(D / 2);
  p->pos_offset = static_cast<int32_t>(o.pos_offset);
  p->freq_fp32 = o.freq_precision == ROPE_QK_FREQ_FP32;
  fill_inv_freq(theta, D, o, p->inv_freq);
  p->pos_rows = nullptr;
  p->pos_row_len = 0;
}

void set_tensor(NormTensor* tn, const void* x, const Tensor& tx, const void* gr, const Tensor* tg, void* o,
                const Tensor& to, int64_t esz) {
  tn->x = static_cast<const char*>(x);
  tn->x_st = tx.st * esz;
  tn->x_sh = tx.sh * esz;
  tn->g = static_cast<const char*>(gr);
  tn->g_st = tg ? tg->st * esz : 0;
  tn->g_sh = tg ? tg->sh * esz : 0;
  tn->o = static_cast<char*>(o);
  tn->o_st = to.st * esz;
  tn->o_sh = to.sh * esz;
  const int64_t H = tn->H;
  // token-major with head strides below 2^32 bytes: the kernels address rows
  // as n * head stride, with 32 x 32 -> 64-bit products
  const int64_t kSh = int64_t(1) << 32;
  tn->lin = tx.st == H * tx.sh && (tg == nullptr || tg->st == H * tg->sh) && to.st == H * to.sh &&
            tn->x_sh < kSh && tn->g_sh < kSh && tn->o_sh < kSh;
}

bool same_tensor(const Tensor& a, const Tensor& b) { return a.base == b.base && a.st == b.st && a.sh == b.sh; }

// The kernel instance for a call: storage type, pairing and row width L (a
// compile-time constant, so that the table offsets of a row's elements are
// immediate offsets of its LDS reads and the lane sums unroll).
template <int kDtype, bool kIl>
const void* fwd_for_width(int64_t L) {
#define ROPE_NF(W) reinterpret_cast<const void*>(&rope_qk_norm_fwd_kernel<kDtype, kIl, kFwdTasks, W>)
  switch (L) {
    case 2: return ROPE_NF(2);
    case 4: return ROPE_NF(4);
    case 8: return ROPE_NF(8);
    case 16: return ROPE_NF(16);
    case 32: return ROPE_NF(32);
    case 64: return ROPE_NF(64);
    default: return nullptr;
  }
#undef ROPE_NF
}

template <int kDtype, bool kIl>
const void* bwd_for_width(int64_t L) {
#define ROPE_NB(W) reinterpret_cast<const void*>(&rope_qk_norm_bwd_kernel<kDtype, kIl, kBwdTasks, W>)
  switch (L) {
    case 2: return ROPE_NB(2);
    case 4: return ROPE_NB(4);
    case 8: return ROPE_NB(8);
    case 16: return ROPE_NB(16);
    case 32: return ROPE_NB(32);
    case 64: return ROPE_NB(64);
    default: return nullptr;
  }
#undef ROPE_NB
}

const void* pick_fwd(int dtype, bool il, int64_t L) {
  if (dtype == ROPE_QK_BF16) return il ? fwd_for_width<ROPE_QK_BF16, true>(L) : fwd_for_width<ROPE_QK_BF16, false>(L);
  if (dtype == ROPE_QK_FP16) return il ? fwd_for_width<ROPE_QK_FP16, true>(L) : fwd_for_width<ROPE_QK_FP16, false>(L);
  return il ? fwd_for_width<ROPE_QK_FP32, true>(L) : fwd_for_width<ROPE_QK_FP32, false>(L);
}

const void* pick_bwd(int dtype, bool il, int64_t L) {
  if (dtype == ROPE_QK_BF16) return il ? bwd_for_width<ROPE_QK_BF16, true>(L) : bwd_for_width<ROPE_QK_BF16, false>(L);
  if (dtype == ROPE_QK_FP16) return il ? bwd_for_width<ROPE_QK_FP16, true>(L) : bwd_for_width<ROPE_QK_FP16, false>(L);
  return il ? bwd_for_width<ROPE_QK_FP32, true>(L) : bwd_for_width<ROPE_QK_FP32, false>(L);
}

// Weight-gradient scratch of rope_qk_norm_bwd_noalloc: one array per GPU the
// library runs on, held until the process ends.  Its size is the largest
// workspace any accepted shape needs (bf16 or fp16 at D = 512: 3072
// workgroups x 2 D float64 sums), so every call the workspace form accepts
// fits.  In host code `scratch` names a host-side stand-in; its device
// address comes from hipGetSymbolAddress, per device.
constexpr int64_t kScratchBytes = kBwdGroups16 * 2 * (2 * kMaxHalf) * static_cast<int64_t>(sizeof(double));
static_assert(kScratchBytes == 24 << 20, "scratch size stated in include/rope_qk.h");
static_assert(kBwdGroups32 * 2 * kMaxHalf * static_cast<int64_t>(sizeof(double)) <= kScratchBytes,
              "float32 rows (D <= 256) fit too");
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on `device`, looked up once per device
// with that device current (each GPU holds its own copy of the array).
int scratch_address(int device, void** out) {
  if (device < 0 || device >= kMaxDevices) return ROPE_QK_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device] == nullptr) {
    int current = -1;
    if (hipGetDevice(&current) != hipSuccess) return ROPE_QK_ERR_LAUNCH;
    if (current != device && hipSetDevice(device) != hipSuccess) return ROPE_QK_ERR_LAUNCH;
    void* ptr = nullptr;
    const hipError_t err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (current != device && hipSetDevice(current) != hipSuccess) return ROPE_QK_ERR_LAUNCH;
    if (err != hipSuccess || ptr == nullptr) return ROPE_QK_ERR_LAUNCH;
    g_scratch_ptr[device] = ptr;
  }
  *out = g_scratch_ptr[device];
  return ROPE_QK_OK;
}

// The backward's checks and launches.  use_scratch: the no-allocation form,
// whose sums go to this device's `scratch` (looked up after every host
// check, so its errors come in the workspace form's order) instead of the
// caller's workspace.
int norm_bwd_impl(const void* dq_out, const void* dk_out, const void* q, const void* k, void* dq, void* dk,
                  const float* q_weight, const float* k_weight, double eps, float* dq_weight, float* dk_weight,
                  void* workspace, int64_t workspace_size, const int32_t* cu_seqlens, int64_t nseq, int64_t T,
                  int64_t Hq, int64_t Hkv, int64_t D, const int64_t* strides, double theta, int dtype,
                  const rope_qk_options* options, void* stream, bool use_scratch) {
  const rope_qk_options o = options ? *options : rope_qk_options{};
  if (strides == nullptr) return ROPE_QK_ERR_NULL;
  const Tensor ts[6] = {{dq_out, strides[0], strides[1]}, {dk_out, strides[2], strides[3]},
                        {q, strides[4], strides[5]},      {k, strides[6], strides[7]},
                        {dq, strides[8], strides[9]},     {dk, strides[10], strides[11]}};
  NormGeometry g;
  const int status = check_norm_call(dtype, nseq, T, Hq, Hkv, D, theta, o, eps, q_weight, k_weight, ts, 6, true, &g);
  if (status != ROPE_QK_OK) return status;
  if ((Hq > 0 && dq_weight == nullptr) || (Hkv > 0 && dk_weight == nullptr)) return ROPE_QK_ERR_NULL;
  const int64_t need = workspace_bytes(g, D);
  if (use_scratch) {
    if (need > kScratchBytes) return ROPE_QK_ERR_SCRATCH;
  } else {
    if (need > 0 && (workspace == nullptr || workspace_size < need)) return ROPE_QK_ERR_WORKSPACE;
    if (workspace != nullptr && !aligned16(workspace)) return ROPE_QK_ERR_ALIGN;
  }
  if (!(dq_weight == nullptr || aligned16(dq_weight)) || !(dk_weight == nullptr || aligned16(dk_weight)))
    return ROPE_QK_ERR_ALIGN;
  if (g.groups > 0 && cu_seqlens == nullptr) return ROPE_QK_ERR_NULL;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (use_scratch) {
    // the device the kernels run on: the stream's, or the current one for the NULL stream
    int device = -1;
    if (s != nullptr ? hipStreamGetDevice(s, &device) != hipSuccess : hipGetDevice(&device) != hipSuccess)
      return ROPE_QK_ERR_LAUNCH;
    const int found = scratch_address(device, &workspace);
    if (found != ROPE_QK_OK) return found;
  }
  const int64_t esz = dtype == ROPE_QK_FP32 ? 4 : 2;
  double* partial = static_cast<double*>(workspace);
  if (g.groups > 0) {
    NormParams p;
    fill_params(&p, g, cu_seqlens, nseq, T, Hq, Hkv, D, theta, eps, o, q_weight, k_weight, -1.0);
    set_tensor(&p.ten[0], q, ts[2], dq_out, &ts[0], dq, ts[4], esz);
    set_tensor(&p.ten[1], k, ts[3], dk_out, &ts[1], dk, ts[5], esz);
    p.ten[0].copy = Hq > 0 && !same_tensor(ts[0], ts[4]);
    p.ten[1].copy = Hkv > 0 && !same_tensor(ts[1], ts[5]);
    p.partial = partial;
    const size_t lds = static_cast<size_t>(2 * p.table_bytes) + static_cast<size_t>(2 * D) * sizeof(float) +
                       static_cast<size_t>((2 + kWaves) * D + D / 2) * sizeof(double);
    void* args[] = {&p};
    const void* kernel = pick_bwd(dtype, o.pairing == ROPE_QK_PAIR_INTERLEAVED, g.L);
    if (kernel == nullptr) return ROPE_QK_ERR_SHAPE;
    const hipError_t err =
        hipLaunchKernel(kernel, dim3(static_cast<uint32_t>(g.groups)), dim3(kThreads), args, lds, s);
    if (err != hipSuccess) return ROPE_QK_ERR_LAUNCH;
  }
  if (dq_weight == nullptr && dk_weight == nullptr) return ROPE_QK_OK;
  uint32_t ng = static_cast<uint32_t>(g.groups);
  int32_t d32 = static_cast<int32_t>(D);
  const double* partial_c = partial;
  void* args[] = {const_cast<double**>(&partial_c), &ng, &d32, &dq_weight, &dk_weight};
  const uint32_t reduce_groups = static_cast<uint32_t>(kXcds * ((2 * D + kXcds - 1) / kXcds));
  const hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(&dw_reduce_kernel), dim3(reduce_groups),
                                         dim3(kThreads), args, 0, s);
  return err == hipSuccess ? ROPE_QK_OK : ROPE_QK_ERR_LAUNCH;
}


}  // namespace

extern "C" {

int rope_qk_norm_fwd(const void* q, const void* k, void* q_out, void* k_out, const float* q_weight,
                     const float* k_weight, double eps, const int32_t* cu_seqlens, int64_t nseq, int64_t T,
                     int64_t Hq, int64_t Hkv, int64_t D, const int64_t* strides, double theta, int dtype,
                     const rope_qk_options* options, void* stream) {
  const rope_qk_options o = options ? *options : rope_qk_options{};
  if (strides == nullptr) return ROPE_QK_ERR_NULL;
  const Tensor ts[4] = {{q, strides[0], strides[1]}, {k, strides[2], strides[3]},
                        {q_out, strides[4], strides[5]}, {k_out, strides[6], strides[7]}};
  NormGeometry g;
  const int status = check_norm_call(dtype, nseq, T, Hq, Hkv, D, theta, o, eps, q_weight, k_weight, ts, 4, false, &g);
  if (status != ROPE_QK_OK) return status;
  if (T == 0 || Hq + Hkv == 0) return ROPE_QK_OK;
  const bool copy_q = Hq > 0 && !same_tensor(ts[0], ts[2]);
  const bool copy_k = Hkv > 0 && !same_tensor(ts[1], ts[3]);
  if (nseq == 0 && !copy_q && !copy_k) return ROPE_QK_OK;  // in place and nothing inside: nothing to do
  if (cu_seqlens == nullptr) return ROPE_QK_ERR_NULL;
  const int64_t esz = dtype == ROPE_QK_FP32 ? 4 : 2;
  NormParams p;
  fill_params(&p, g, cu_seqlens, nseq, T, Hq, Hkv, D, theta, eps, o, q_weight, k_weight, 1.0);
  set_tensor(&p.ten[0], q, ts[0], nullptr, nullptr, q_out, ts[2], esz);
  set_tensor(&p.ten[1], k, ts[1], nullptr, nullptr, k_out, ts[3], esz);
  p.ten[0].copy = copy_q;
  p.ten[1].copy = copy_k;
  p.partial = nullptr;
  const int64_t nt = p.ntiles;
  const int64_t gx = nt < kGridX ? nt : kGridX;
  const dim3 grid(static_cast<uint32_t>(gx), static_cast<uint32_t>((nt + gx - 1) / gx));
  const size_t lds = static_cast<size_t>(p.table_bytes) + static_cast<size_t>(2 * D) * sizeof(float);
  void* args[] = {&p};
  const void* kernel = pick_fwd(dtype, o.pairing == ROPE_QK_PAIR_INTERLEAVED, g.L);
  if (kernel == nullptr) return ROPE_QK_ERR_SHAPE;
  const hipError_t err = hipLaunchKernel(kernel, grid, dim3(kThreads), args, lds, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? ROPE_QK_OK : ROPE_QK_ERR_LAUNCH;
}

int64_t rope_qk_norm_bwd_workspace_bytes(int64_t T, int64_t Hq, int64_t Hkv, int64_t D, int dtype) {
  if (dtype != ROPE_QK_FP32 && dtype != ROPE_QK_BF16 && dtype != ROPE_QK_FP16) return ROPE_QK_ERR_DTYPE;
  if (T < 0 || Hq < 0 || Hkv < 0 || D < 2 || (D & 1) || D > 2 * kMaxHalf || T > INT32_MAX) return ROPE_QK_ERR_SHAPE;
  NormGeometry g;
  const int status = norm_geometry(T, Hq, Hkv, D, dtype, true, &g);
  if (status != ROPE_QK_OK) return status;
  return workspace_bytes(g, D);
}

int rope_qk_norm_tile_positions(const int32_t* cu_seqlens, int64_t nseq, int64_t T, int64_t Hq, int64_t Hkv,
                                int64_t D, int dtype, const rope_qk_options* options, int backward, int32_t* out,
                                int64_t out_len, int64_t* ntiles, int64_t* row_len, void* stream) {
  if (ntiles == nullptr || row_len == nullptr) return ROPE_QK_ERR_NULL;
  *ntiles = 0;
  *row_len = 0;
  const rope_qk_options o = options ? *options : rope_qk_options{};
  int status = check_call(dtype, nseq, T, Hq, Hkv, D, 1.0, o);
  if (status != ROPE_QK_OK) return status;
  if (o.rotary_dim != 0 && o.rotary_dim != D) return ROPE_QK_ERR_OPTION;
  NormGeometry g;
  status = norm_geometry(T, Hq, Hkv, D, dtype, backward != 0, &g);
  if (status != ROPE_QK_OK) return status;
  if (T == 0 || Hq + Hkv == 0) return ROPE_QK_OK;
  *ntiles = g.ntiles[0] + g.ntiles[1];
  *row_len = 1 + g.span;
  if (out == nullptr) return ROPE_QK_OK;  // the geometry only
  if (cu_seqlens == nullptr) return ROPE_QK_ERR_NULL;
  if (out_len < *ntiles * *row_len) return ROPE_QK_ERR_SHAPE;
  NormParams p;
  fill_params(&p, g, cu_seqlens, nseq, T, Hq, Hkv, D, 1.0, 1.0, o, nullptr, nullptr, backward ? -1.0 : 1.0);
  p.partial = nullptr;
  p.pos_rows = out;
  p.pos_row_len = *row_len;
  void* args[] = {&p};
  hipError_t err;
  if (backward) {
    err = hipLaunchKernel(reinterpret_cast<const void*>(&rope_qk_norm_bwd_kernel<ROPE_QK_BF16, false, kBwdTasks, 8, true>),
                          dim3(static_cast<uint32_t>(g.groups)), dim3(kThreads), args, 0,
                          static_cast<hipStream_t>(stream));
  } else {
    const int64_t nt = *ntiles;
    const int64_t gx = nt < kGridX ? nt : kGridX;
    err = hipLaunchKernel(reinterpret_cast<const void*>(&rope_qk_norm_fwd_positions_kernel),
                          dim3(static_cast<uint32_t>(gx), static_cast<uint32_t>((nt + gx - 1) / gx)), dim3(kThreads),
                          args, 0, static_cast<hipStream_t>(stream));
  }
  return err == hipSuccess ? ROPE_QK_OK : ROPE_QK_ERR_LAUNCH;
}

int rope_qk_norm_bwd(const void* dq_out, const void* dk_out, const void* q, const void* k, void* dq, void* dk,
                     const float* q_weight, const float* k_weight, double eps, float* dq_weight, float* dk_weight,
                     void* workspace, int64_t workspace_size, const int32_t* cu_seqlens, int64_t nseq, int64_t T,
                     int64_t Hq, int64_t Hkv, int64_t D, const int64_t* strides, double theta, int dtype,
                     const rope_qk_options* options, void* stream) {
  return norm_bwd_impl(dq_out, dk_out, q, k, dq, dk, q_weight, k_weight, eps, dq_weight, dk_weight, workspace,
                       workspace_size, cu_seqlens, nseq, T, Hq, Hkv, D, strides, theta, dtype, options, stream,
                       false);
}

int rope_qk_norm_bwd_noalloc(const void* dq_out, const void* dk_out, const void* q, const void* k, void* dq,
                             void* dk, const float* q_weight, const float* k_weight, double eps, float* dq_weight,
                             float* dk_weight, const int32_t* cu_seqlens, int64_t nseq, int64_t T, int64_t Hq,
                             int64_t Hkv, int64_t D, const int64_t* strides, double theta, int dtype,
                             const rope_qk_options* options, void* stream) {
  return norm_bwd_impl(dq_out, dk_out, q, k, dq, dk, q_weight, k_weight, eps, dq_weight, dk_weight, nullptr, 0,
                       cu_seqlens, nseq, T, Hq, Hkv, D, strides, theta, dtype, options, stream, true);
}

}  // extern "C"
