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
//  * Row tiles.  A row is one head of one token: D elements in L = D*size/16
//    chunks of 16 bytes, L a power of two from 2 to 64.  Lane l of a
//    workgroup holds chunk l % L of row u * (256 / L) + l / L of the tile, for
//    u < kTPT, so the chunks of a row sit on L consecutive lanes of one wave
//    and each wave-wide load or store covers whole rows.  A tile is a run of
//    whole rows in (token, head of q then k) order that may begin and end
//    inside a token.
//  * Per row: the sum of squares in float64, summed over the row's lanes by
//    a xor butterfly (ds_bpermute; every lane ends with the same bits),
//    r = 1/sqrt(mean + eps) from v_rsq_f64 and three Newton steps, then the
//    rotation exactly as in the rotation kernels: the rotate_half partner
//    chunk comes from lane l ^ L/2 (negated in the first half), interleaved
//    pairs sit inside a chunk; the cos/sin table is built once per tile.
//  * Backward: the rotation by -angle (the table holds -sin), then the RMSNorm
//    gradient with a second row sum (sum_j g_j x_j); the weight gradient is
//    summed per lane over its rows, then across the lanes of a wave that hold
//    the same chunk, then across the 4 waves in LDS, into one float64 partial
//    per tile and column, which two small kernels sum in a fixed order: the
//    result is deterministic.
//  * Everything is evaluated in float64 and rounded once to the storage type.

#include "rope_common.h"

namespace {

constexpr int kNormTasks = 4;        // rows per lane per tile
constexpr int64_t kMaxHeads = 65535;  // row -> (token, head) division limit
constexpr uint32_t kReduceSlices = 256;
constexpr int kWaves = kThreads / 64;

struct NormParams {
  const char* xq;          // forward: q; backward: the forward's input q
  const char* xk;
  const char* gq;          // backward: incoming gradient of the forward's output q
  const char* gk;
  char* oq;                // forward: output q; backward: gradient of the input q
  char* ok;
  const float* wq;         // [D] weights of q and of k
  const float* wk;
  double* partial;         // backward: [ntiles][2 D] weight-gradient partials
  const int32_t* cu;
  int64_t T;
  int64_t xq_st, xq_sh, xk_st, xk_sh;  // byte strides
  int64_t gq_st, gq_sh, gk_st, gk_sh;
  int64_t oq_st, oq_sh, ok_st, ok_sh;
  uint64_t magic_heads;    // ceil(2^40 / H): exact n / H for n < 2^24
  uint64_t magic_half;     // ceil(2^32 / half)
  double rcp_heads;        // 1 / H, rounded
  double eps;
  double inv_d;            // 1 / D (exact: D is a power of two)
  double sign;             // +1 forward, -1 backward
  uint32_t ntiles;
  int32_t tile_rows;
  int32_t nseq;
  int32_t Hq;
  int32_t H;               // Hq + Hkv
  int32_t D;
  int32_t half;            // D / 2
  int32_t L;               // chunks per row
  int32_t lshift;          // log2(L)
  int32_t pos_offset;
  int32_t freq_fp32;
  int32_t copy_q;          // 1: tokens outside every sequence are copied to the output of q
  int32_t copy_k;
  double inv_freq[kMaxHalf];
};

// The float64 value lane (addr / 4) holds (ds_bpermute, two dwords).
__device__ __forceinline__ double lane_f64(double v, int addr) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(addr, static_cast<int>(b)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(addr, static_cast<int>(b >> 32)));
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

// Sum over the L consecutive lanes of a row (xor butterfly; a + b and b + a
// are the same float64, so every lane of the row ends with the same bits).
__device__ __forceinline__ double row_sum(double v, int L, int lane) {
  for (int m = 1; m < L; m <<= 1) v += lane_f64(v, (lane ^ m) << 2);
  return v;
}

// 1 / sqrt(a) for finite a > 0: the hardware estimate refined by three
// Newton steps y <- y + y (1 - a y^2) / 2 (each roughly squares the
// relative error), which leaves an error of about one float64 ulp.
__device__ __forceinline__ double rsqrt_f64(double a) {
  double y = __builtin_amdgcn_rsq(a);
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const double e = fma(-(a * y), y, 1.0);
    y = fma(0.5 * y, e, y);
  }
  return y;
}

// kVec storage elements of a 16-byte chunk as float64.
template <int kDtype>
__device__ __forceinline__ void unpack_chunk(const u32x4& w, double* x) {
  if constexpr (kDtype == ROPE_QK_FP32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = static_cast<double>(__uint_as_float(w[j]));
  } else {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const f64x2 v = unpack16<kDtype>(w[d]);
      x[2 * d] = v.x;
      x[2 * d + 1] = v.y;
    }
  }
}

// One rounding of kVec float64 values to the storage type (16-bit: fast path,
// redone exactly when a value is hard; see pack16_fast).
template <int kDtype>
__device__ __forceinline__ u32x4 pack_chunk(const double* y) {
  u32x4 out;
  if constexpr (kDtype == ROPE_QK_FP32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = __float_as_uint(static_cast<float>(y[j]));
  } else {
    bool tie = false;
#pragma unroll
    for (int d = 0; d < 4; ++d) out[d] = pack16_fast<kDtype>(y[2 * d], y[2 * d + 1], tie);
    if (tie) {
#pragma unroll
      for (int d = 0; d < 4; ++d) out[d] = pack16_exact<kDtype>(y[2 * d], y[2 * d + 1]);
    }
  }
  return out;
}

// The 16-byte chunk lane (addr / 4) holds, with the sign of every element
// flipped when `neg` (the rotate_half partner of a first-half chunk).
template <int kDtype>
__device__ __forceinline__ u32x4 partner_chunk(const u32x4& v, int addr, bool neg) {
  const uint32_t flip = neg ? (kDtype == ROPE_QK_FP32 ? 0x80000000u : 0x80008000u) : 0u;
  u32x4 out;
#pragma unroll
  for (int d = 0; d < 4; ++d) out[d] = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(addr, static_cast<int>(v[d]))) ^ flip;
  return out;
}

// The rotation of one chunk of normalised values n (own) with the partner's p
// (rotate_half; p already negated in the first half) or of the pairs inside
// the chunk (interleaved); cs points at the chunk's first table entry, stride
// `step` entries apart.
template <bool kIl, int kVec>
__device__ __forceinline__ void rotate_chunk(const double* n, const double* p, const double2* cs, int step, double* y) {
  if constexpr (kIl) {
#pragma unroll
    for (int jj = 0; jj < kVec / 2; ++jj) {
      const double2 c = cs[jj * step];
      const double a = n[2 * jj], b = n[2 * jj + 1];
      y[2 * jj] = fma(a, c.x, -(b * c.y));
      y[2 * jj + 1] = fma(b, c.x, a * c.y);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      const double2 c = cs[j * step];
      y[j] = fma(n[j], c.x, p[j] * c.y);
    }
  }
}

template <int kDtype, bool kIl, bool kBwd, int kTPT>
__device__ __forceinline__ void norm_tile(const NormParams& p, uint32_t tile, int32_t* s_pos, double2* s_cs,
                                          float* s_w, double* s_dw) {
  constexpr int kVec = kDtype == ROPE_QK_FP32 ? 4 : 8;  // elements per chunk
  constexpr int kPPC = kIl ? kVec / 2 : kVec;          // table pairs per chunk
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int L = p.L;
  const int c = tid & (L - 1);  // the chunk of its rows this lane holds
  const int hl = L >> 1;        // chunks per half row
  const cu_ptr cu = (cu_ptr)p.cu;
  const int32_t nseq = p.nseq;
  const int32_t H = p.H;

  // first row n0 = t0 * H + r0 (n0 < 2^47 is exact in float64; the rounded quotient is off by at most one)
  const int64_t n0 = static_cast<int64_t>(tile) * p.tile_rows;
  int32_t t0i = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(static_cast<double>(n0) * p.rcp_heads));
  int64_t r0l = n0 - static_cast<int64_t>(t0i) * H;
  if (r0l < 0) { t0i -= 1; r0l += H; }
  if (r0l >= H) { t0i += 1; r0l -= H; }
  const int64_t t0 = t0i;
  const uint32_t r0 = static_cast<uint32_t>(r0l);
  const int64_t n_end = min(n0 + p.tile_rows, p.T * H);
  const int ntok = static_cast<int>(div_tok(static_cast<uint32_t>(n_end - n0) + r0 - 1, p.magic_heads)) + 1;
  const int64_t t_end = t0 + ntok;
  const int nent = ntok * p.half;

  // 1. inv_freq of this thread's table entries and the weights, before the data
  double f[kEnt];
  int tt_e[kEnt], i_e[kEnt];
#pragma unroll
  for (int v = 0; v < kEnt; ++v) {
    const int e = tid + v * kThreads;
    const int tt = e < nent ? static_cast<int>(div_small(static_cast<uint32_t>(e), p.magic_half)) : 0;
    tt_e[v] = tt;
    i_e[v] = e < nent ? e - tt * p.half : 0;
    f[v] = (v == 0 || v * kThreads < nent) ? p.inv_freq[i_e[v]] : 0.0;
  }
  const int nw4 = p.D >> 1;  // float4s of the two weight vectors
  float4 wv = make_float4(0.f, 0.f, 0.f, 0.f);
  if (tid < nw4) {
    const bool of_k = tid * 4 >= p.D;
    const float* base = of_k ? p.wk : p.wq;  // NULL for a tensor without heads
    if (base != nullptr) wv = *reinterpret_cast<const float4*>(base + (of_k ? tid * 4 - p.D : tid * 4));
  }
  __builtin_amdgcn_sched_barrier(0);

  // 2. every load of the tile (rows past the tile's end re-read its first row)
  u32x4 a[kTPT], g[kTPT];
  gchar* optr[kTPT];
  int tt_of[kTPT];
  bool act[kTPT], isq[kTPT];
  const int rows_per_step = kThreads >> p.lshift;
#pragma unroll
  for (int u = 0; u < kTPT; ++u) {
    const int lr = u * rows_per_step + (tid >> p.lshift);
    act[u] = n0 + lr < n_end;
    const uint32_t l = act[u] ? r0 + static_cast<uint32_t>(lr) : r0;
    const uint32_t tt = div_tok(l, p.magic_heads);
    const uint32_t h = l - tt * static_cast<uint32_t>(H);
    const int64_t t = t0 + tt;
    const bool is_q = static_cast<int32_t>(h) < p.Hq;
    const int64_t hh = is_q ? static_cast<int64_t>(h) : static_cast<int64_t>(h) - p.Hq;
    const int64_t off = static_cast<int64_t>(c) * 16;
    const gchar* xrow = is_q ? (const gchar*)p.xq + t * p.xq_st + hh * p.xq_sh
                             : (const gchar*)p.xk + t * p.xk_st + hh * p.xk_sh;
    a[u] = __builtin_nontemporal_load(reinterpret_cast<const gu32x4*>(xrow + off));
    if constexpr (kBwd) {
      const gchar* grow = is_q ? (const gchar*)p.gq + t * p.gq_st + hh * p.gq_sh
                               : (const gchar*)p.gk + t * p.gk_st + hh * p.gk_sh;
      g[u] = __builtin_nontemporal_load(reinterpret_cast<const gu32x4*>(grow + off));
    }
    optr[u] = (is_q ? (gchar*)p.oq + t * p.oq_st + hh * p.oq_sh : (gchar*)p.ok + t * p.ok_st + hh * p.ok_sh) + off;
    tt_of[u] = static_cast<int>(tt);
    isq[u] = is_q;
  }
  __builtin_amdgcn_sched_barrier(0);

  // 3. positions and the cos/sin table; the weights into LDS
  if (tid < nw4) reinterpret_cast<float4*>(s_w)[tid] = wv;
  const int32_t s0 = last_start_at_or_before(cu, nseq, t0);
  const int64_t cu_last = cu[nseq];
  const int64_t cu_first_end = nseq >= 1 ? static_cast<int64_t>(cu[1]) : INT64_MIN;  // cu[1] exists only then
  int64_t start[kEnt];
#pragma unroll
  for (int v = 0; v < kEnt; ++v) start[v] = s0 >= 0 ? static_cast<int64_t>(cu[s0]) : INT64_MIN;
  for (int32_t j = s0 + 1; j <= nseq; ++j) {
    const int64_t cv = cu[j];
    if (cv >= t_end) break;
#pragma unroll
    for (int v = 0; v < kEnt; ++v) start[v] = cv <= t0 + tt_e[v] ? cv : start[v];
  }
#pragma unroll
  for (int v = 0; v < kEnt; ++v) {
    if (v > 0 && v * kThreads >= nent) break;
    const int e = tid + v * kThreads;
    const int64_t t = t0 + tt_e[v];
    const bool inside = start[v] != INT64_MIN && t < cu_last;
    const int64_t pos64 = inside ? t - start[v] + (t < cu_first_end ? p.pos_offset : 0) : -1;
    const int32_t pos = pos64 <= INT32_MAX ? static_cast<int32_t>(pos64) : -1;
    if (e < nent) {
      if (i_e[v] == 0) s_pos[tt_e[v]] = pos;
      if (pos >= 0) {
        double sn, cs;
        const double ang = p.freq_fp32 ? static_cast<double>(static_cast<float>(pos) * static_cast<float>(f[v]))
                                       : static_cast<double>(pos) * f[v];
        rope_sincos(ang, &sn, &cs);
        s_cs[cs_slot(tt_e[v], i_e[v], kPPC, kIl ? L : hl)] = make_double2(cs, p.sign * sn);
      }
    }
  }
  __syncthreads();

  // 4. normalise and rotate every row (forward), or undo the rotation and take
  //    the norm's gradient (backward); then store
  const int paddr = (lane ^ hl) << 2;  // rotate_half partner lane
  const bool first = c < hl;
  const int cw = c * kVec;                      // this lane's first element
  const int pw = (kIl ? c : (c ^ hl)) * kVec;  // the partner chunk's first element
  double acc_q[kVec], acc_k[kVec];
#pragma unroll
  for (int j = 0; j < kVec; ++j) acc_q[j] = acc_k[j] = 0.0;
  bool st[kTPT];
  u32x4 out[kTPT];
#pragma unroll
  for (int u = 0; u < kTPT; ++u) {
    const int tt = tt_of[u];
    const bool inside = s_pos[tt] >= 0;
    st[u] = act[u] && (inside || (isq[u] ? p.copy_q : p.copy_k));
    const float* w = s_w + (isq[u] ? 0 : p.D);
    const double2* cs = kIl ? s_cs + tt * kPPC * L + c : s_cs + tt * kPPC * hl + (c & (hl - 1));
    const int step = kIl ? L : hl;
    double x[kVec];
    unpack_chunk<kDtype>(a[u], x);
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < kVec; ++j) ss = fma(x[j], x[j], ss);
    ss = row_sum(ss, L, lane);
    const double r = rsqrt_f64(fma(ss, p.inv_d, p.eps));
    double y[kVec];
    if constexpr (!kBwd) {
      double n[kVec], pn[kVec];
#pragma unroll
      for (int j = 0; j < kVec; ++j) n[j] = (x[j] * r) * static_cast<double>(w[cw + j]);
      if constexpr (!kIl) {
        const u32x4 pr = partner_chunk<kDtype>(a[u], paddr, first);
        double px[kVec];
        unpack_chunk<kDtype>(pr, px);
#pragma unroll
        for (int j = 0; j < kVec; ++j) pn[j] = (px[j] * r) * static_cast<double>(w[pw + j]);
      }
      rotate_chunk<kIl, kVec>(n, pn, cs, step, y);
      out[u] = inside ? pack_chunk<kDtype>(y) : a[u];
    } else {
      double dy[kVec], pdy[kVec], dn[kVec];
      unpack_chunk<kDtype>(g[u], dy);
      if constexpr (!kIl) {
        const u32x4 pr = partner_chunk<kDtype>(g[u], paddr, first);
        unpack_chunk<kDtype>(pr, pdy);
      }
      rotate_chunk<kIl, kVec>(dy, pdy, cs, step, dn);  // rotation by -angle: the table holds -sin
      double gx = 0.0;
      double gw[kVec];
#pragma unroll
      for (int j = 0; j < kVec; ++j) {
        gw[j] = dn[j] * static_cast<double>(w[cw + j]);
        gx = fma(gw[j], x[j], gx);
      }
      gx = row_sum(gx, L, lane);
      const double coef = (r * r) * (gx * p.inv_d);
      const bool use = act[u] && inside;
#pragma unroll
      for (int j = 0; j < kVec; ++j) {
        y[j] = r * (gw[j] - x[j] * coef);
        const double dw = use ? dn[j] * x[j] * r : 0.0;
        if (isq[u]) acc_q[j] += dw; else acc_k[j] += dw;
      }
      out[u] = inside ? pack_chunk<kDtype>(y) : g[u];
    }
  }
#pragma unroll
  for (int u = 0; u < kTPT; ++u) {
    if (!st[u]) continue;
    __builtin_nontemporal_store(out[u], reinterpret_cast<gu32x4*>(optr[u]));
  }

  if constexpr (kBwd) {
    // weight-gradient partial of the tile: lanes holding the same chunk, then the waves
    for (int m = L; m < 64; m <<= 1) {
      const int addr = (lane ^ m) << 2;
#pragma unroll
      for (int j = 0; j < kVec; ++j) {
        acc_q[j] += lane_f64(acc_q[j], addr);
        acc_k[j] += lane_f64(acc_k[j], addr);
      }
    }
    const int wave = tid >> 6;
    const int width = 2 * p.D;
    if (lane < L) {
#pragma unroll
      for (int j = 0; j < kVec; ++j) {
        s_dw[wave * width + cw + j] = acc_q[j];
        s_dw[wave * width + p.D + cw + j] = acc_k[j];
      }
    }
    __syncthreads();
    double* dst = p.partial + static_cast<int64_t>(tile) * width;
    for (int col = tid; col < width; col += kThreads) {
      double s = s_dw[col];
#pragma unroll
      for (int wv2 = 1; wv2 < kWaves; ++wv2) s += s_dw[wv2 * width + col];
      dst[col] = s;
    }
  }
}

template <int kDtype, bool kIl, bool kBwd, int kTPT>
__global__ __launch_bounds__(kThreads) void rope_qk_norm_kernel(const NormParams p) {
  __shared__ int32_t s_pos[kMaxTileTokens];
  extern __shared__ double2 s_dyn[];  // [table][weights 2D floats][backward: wave partials 4 x 2D doubles]
  const uint32_t tile = blockIdx.y * gridDim.x + blockIdx.x;
  if (tile >= p.ntiles) return;
  const int table_entries = kMaxTableBytes / 16;
  double2* s_cs = s_dyn;
  float* s_w = reinterpret_cast<float*>(s_dyn + table_entries);
  double* s_dw = reinterpret_cast<double*>(s_dyn + table_entries) + p.D;  // after 2D floats = D doubles
  norm_tile<kDtype, kIl, kBwd, kTPT>(p, tile, s_pos, s_cs, s_w, s_dw);
}

// Stage 1 of the weight-gradient sum: column col of the tiles of slice
// blockIdx.y, in tile order.
__global__ __launch_bounds__(kThreads) void dw_slices_kernel(const double* __restrict__ partial, uint32_t ntiles,
                                                            int32_t width, uint32_t slice,
                                                            double* __restrict__ sums) {
  const int col = blockIdx.x * kThreads + threadIdx.x;
  if (col >= width) return;
  const uint32_t a = blockIdx.y * slice;
  const uint32_t b = min(a + slice, ntiles);
  double acc = 0.0;
  for (uint32_t t = a; t < b; ++t) acc += partial[static_cast<int64_t>(t) * width + col];
  sums[static_cast<int64_t>(blockIdx.y) * width + col] = acc;
}

// Stage 2: the slices in order, rounded once to float32.
__global__ __launch_bounds__(kThreads) void dw_final_kernel(const double* __restrict__ sums, uint32_t nslices,
                                                           int32_t D, float* __restrict__ dwq,
                                                           float* __restrict__ dwk) {
  const int col = blockIdx.x * kThreads + threadIdx.x;
  if (col >= 2 * D) return;
  double acc = 0.0;
  for (uint32_t s = 0; s < nslices; ++s) acc += sums[static_cast<int64_t>(s) * 2 * D + col];
  const float v = static_cast<float>(acc);
  if (col < D) {
    if (dwq != nullptr) dwq[col] = v;
  } else if (dwk != nullptr) {
    dwk[col - D] = v;
  }
}

struct Tensor {
  const void* base;
  int64_t st, sh;  // element strides
};

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) % 16) == 0; }

// Geometry shared by the forward, the backward and the workspace query.
struct NormGeometry {
  int64_t L = 0, tile_rows = 0, ntiles = 0, nslices = 0, span = 0;
};

int norm_geometry(int64_t T, int64_t Hq, int64_t Hkv, int64_t D, int dtype, NormGeometry* g) {
  const int64_t esz = dtype == ROPE_QK_FP32 ? 4 : 2;
  const int64_t L = D * esz / 16;
  if ((D * esz) % 16 || L < 2 || L > 64 || (L & (L - 1))) return ROPE_QK_ERR_SHAPE;
  const int64_t H = Hq + Hkv;
  if (H > kMaxHeads) return ROPE_QK_ERR_SHAPE;
  const int64_t half = D / 2;
  int64_t cap_tokens = kMaxTableBytes / (half * 16);
  if (cap_tokens > kMaxTileTokens) cap_tokens = kMaxTileTokens;
  int64_t tile_rows = int64_t(kNormTasks) * (kThreads / L);
  if (H > 0 && tile_rows > (cap_tokens - 1) * H) tile_rows = (cap_tokens - 1) * H;
  g->L = L;
  g->tile_rows = tile_rows;
  g->ntiles = H > 0 ? (T * H + tile_rows - 1) / tile_rows : 0;
  if (g->ntiles > INT32_MAX) return ROPE_QK_ERR_SHAPE;
  g->nslices = g->ntiles < kReduceSlices ? g->ntiles : kReduceSlices;
  g->span = H > 0 ? (tile_rows % H == 0 ? tile_rows / H : (H + tile_rows - 2) / H + 1) : 0;
  return ROPE_QK_OK;
}

int64_t workspace_bytes(const NormGeometry& g, int64_t D) {
  return (g.ntiles + g.nslices) * 2 * D * static_cast<int64_t>(sizeof(double));
}

// Everything both passes check: the shared call checks, the norm's own limits
// (eps, full rotary dim, row shape) and each tensor's alignment and layout.
int check_norm_call(int dtype, int64_t nseq, int64_t T, int64_t Hq, int64_t Hkv, int64_t D, double theta,
                    const rope_qk_options& o, double eps, const float* wq, const float* wk, const Tensor* ts,
                    int nts, NormGeometry* g) {
  int status = check_call(dtype, nseq, T, Hq, Hkv, D, theta, o);
  if (status != ROPE_QK_OK) return status;
  if (!(eps > 0.0) || !isfinite(eps) || (o.rotary_dim != 0 && o.rotary_dim != D)) return ROPE_QK_ERR_OPTION;
  status = norm_geometry(T, Hq, Hkv, D, dtype, g);
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
  if ((Hq > 0 && !aligned16(wq)) || (Hkv > 0 && !aligned16(wk))) return ROPE_QK_ERR_ALIGN;
  return ROPE_QK_OK;
}

void fill_params(NormParams* p, const NormGeometry& g, const int32_t* cu, int64_t nseq, int64_t T, int64_t Hq,
                 int64_t Hkv, int64_t D, double theta, double eps, int dtype, const rope_qk_options& o,
                 const float* wq, const float* wk, double sign) {
  const int64_t H = Hq + Hkv;
  p->wq = wq;
  p->wk = wk;
  p->cu = cu;
  p->T = T;
  p->magic_heads = ((uint64_t(1) << 40) + H - 1) / H;
  p->magic_half = ((uint64_t(1) << 32) + D / 2 - 1) / (D / 2);
  p->rcp_heads = 1.0 / static_cast<double>(H);
  p->eps = eps;
  p->inv_d = 1.0 / static_cast<double>(D);
  p->sign = sign;
  p->ntiles = static_cast<uint32_t>(g.ntiles);
  p->tile_rows = static_cast<int32_t>(g.tile_rows);
  p->nseq = static_cast<int32_t>(nseq);
  p->Hq = static_cast<int32_t>(Hq);
  p->H = static_cast<int32_t>(H);
  p->D = static_cast<int32_t>(D);
  p->half = static_cast<int32_t>(D / 2);
  p->L = static_cast<int32_t>(g.L);
  int s = 0;
  while ((int64_t(1) << s) < g.L) ++s;
  p->lshift = s;
  p->pos_offset = static_cast<int32_t>(o.pos_offset);
  p->freq_fp32 = o.freq_precision == ROPE_QK_FREQ_FP32;
  fill_inv_freq(theta, D, o, p->inv_freq);
}

bool same_tensor(const Tensor& a, const Tensor& b) { return a.base == b.base && a.st == b.st && a.sh == b.sh; }

size_t norm_lds(int64_t D, bool bwd) {
  return static_cast<size_t>(kMaxTableBytes) + static_cast<size_t>(2 * D) * sizeof(float) +
         (bwd ? static_cast<size_t>(kWaves * 2 * D) * sizeof(double) : 0);
}

const void* pick_norm_kernel(int dtype, bool interleaved, bool bwd) {
#define ROPE_NK(DT, IL, BW) reinterpret_cast<const void*>(&rope_qk_norm_kernel<DT, IL, BW, kNormTasks>)
#define ROPE_NK_DT(DT) \
  (interleaved ? (bwd ? ROPE_NK(DT, true, true) : ROPE_NK(DT, true, false)) \
               : (bwd ? ROPE_NK(DT, false, true) : ROPE_NK(DT, false, false)))
  return dtype == ROPE_QK_BF16 ? ROPE_NK_DT(ROPE_QK_BF16)
         : dtype == ROPE_QK_FP16 ? ROPE_NK_DT(ROPE_QK_FP16)
                                 : ROPE_NK_DT(ROPE_QK_FP32);
#undef ROPE_NK_DT
#undef ROPE_NK
}

int launch_norm(const NormParams& p, const NormGeometry& g, int64_t D, int dtype, bool interleaved, bool bwd,
                hipStream_t stream) {
  if (g.ntiles == 0) return ROPE_QK_OK;
  const int64_t gx = g.ntiles < kGridX ? g.ntiles : kGridX;
  const dim3 grid(static_cast<uint32_t>(gx), static_cast<uint32_t>((g.ntiles + gx - 1) / gx));
  NormParams pc = p;
  void* args[] = {&pc};
  const hipError_t err = hipLaunchKernel(pick_norm_kernel(dtype, interleaved, bwd), grid, dim3(kThreads), args,
                                         norm_lds(D, bwd), stream);
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
  const int status = check_norm_call(dtype, nseq, T, Hq, Hkv, D, theta, o, eps, q_weight, k_weight, ts, 4, &g);
  if (status != ROPE_QK_OK) return status;
  if (T == 0 || Hq + Hkv == 0) return ROPE_QK_OK;
  const bool copy_q = Hq > 0 && !same_tensor(ts[0], ts[2]);
  const bool copy_k = Hkv > 0 && !same_tensor(ts[1], ts[3]);
  if (nseq == 0 && !copy_q && !copy_k) return ROPE_QK_OK;  // in place and nothing inside: nothing to do
  if (cu_seqlens == nullptr) return ROPE_QK_ERR_NULL;
  const int64_t esz = dtype == ROPE_QK_FP32 ? 4 : 2;
  NormParams p;
  fill_params(&p, g, cu_seqlens, nseq, T, Hq, Hkv, D, theta, eps, dtype, o, q_weight, k_weight, 1.0);
  p.xq = static_cast<const char*>(q);
  p.xk = static_cast<const char*>(k);
  p.gq = p.gk = nullptr;
  p.oq = static_cast<char*>(q_out);
  p.ok = static_cast<char*>(k_out);
  p.partial = nullptr;
  p.xq_st = strides[0] * esz, p.xq_sh = strides[1] * esz, p.xk_st = strides[2] * esz, p.xk_sh = strides[3] * esz;
  p.gq_st = p.gq_sh = p.gk_st = p.gk_sh = 0;
  p.oq_st = strides[4] * esz, p.oq_sh = strides[5] * esz, p.ok_st = strides[6] * esz, p.ok_sh = strides[7] * esz;
  p.copy_q = copy_q;
  p.copy_k = copy_k;
  return launch_norm(p, g, D, dtype, o.pairing == ROPE_QK_PAIR_INTERLEAVED, false, static_cast<hipStream_t>(stream));
}

int64_t rope_qk_norm_bwd_workspace_bytes(int64_t T, int64_t Hq, int64_t Hkv, int64_t D, int dtype) {
  if (dtype != ROPE_QK_FP32 && dtype != ROPE_QK_BF16 && dtype != ROPE_QK_FP16) return ROPE_QK_ERR_DTYPE;
  if (T < 0 || Hq < 0 || Hkv < 0 || D < 2 || (D & 1) || D > 2 * kMaxHalf || T > INT32_MAX) return ROPE_QK_ERR_SHAPE;
  NormGeometry g;
  const int status = norm_geometry(T, Hq, Hkv, D, dtype, &g);
  if (status != ROPE_QK_OK) return status;
  return workspace_bytes(g, D);
}

int rope_qk_norm_bwd(const void* dq_out, const void* dk_out, const void* q, const void* k, void* dq, void* dk,
                     const float* q_weight, const float* k_weight, double eps, float* dq_weight, float* dk_weight,
                     void* workspace, int64_t workspace_size, const int32_t* cu_seqlens, int64_t nseq, int64_t T,
                     int64_t Hq, int64_t Hkv, int64_t D, const int64_t* strides, double theta, int dtype,
                     const rope_qk_options* options, void* stream) {
  const rope_qk_options o = options ? *options : rope_qk_options{};
  if (strides == nullptr) return ROPE_QK_ERR_NULL;
  const Tensor ts[6] = {{dq_out, strides[0], strides[1]}, {dk_out, strides[2], strides[3]},
                        {q, strides[4], strides[5]},      {k, strides[6], strides[7]},
                        {dq, strides[8], strides[9]},     {dk, strides[10], strides[11]}};
  NormGeometry g;
  const int status = check_norm_call(dtype, nseq, T, Hq, Hkv, D, theta, o, eps, q_weight, k_weight, ts, 6, &g);
  if (status != ROPE_QK_OK) return status;
  if ((Hq > 0 && dq_weight == nullptr) || (Hkv > 0 && dk_weight == nullptr)) return ROPE_QK_ERR_NULL;
  const int64_t need = workspace_bytes(g, D);
  if (need > 0 && (workspace == nullptr || workspace_size < need)) return ROPE_QK_ERR_WORKSPACE;
  if (workspace != nullptr && !aligned16(workspace)) return ROPE_QK_ERR_ALIGN;
  if (!(dq_weight == nullptr || aligned16(dq_weight)) || !(dk_weight == nullptr || aligned16(dk_weight)))
    return ROPE_QK_ERR_ALIGN;
  if (g.ntiles > 0 && cu_seqlens == nullptr) return ROPE_QK_ERR_NULL;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t esz = dtype == ROPE_QK_FP32 ? 4 : 2;
  double* partial = static_cast<double*>(workspace);
  double* sums = partial + g.ntiles * 2 * D;
  if (g.ntiles > 0) {
    NormParams p;
    fill_params(&p, g, cu_seqlens, nseq, T, Hq, Hkv, D, theta, eps, dtype, o, q_weight, k_weight, -1.0);
    p.xq = static_cast<const char*>(q);
    p.xk = static_cast<const char*>(k);
    p.gq = static_cast<const char*>(dq_out);
    p.gk = static_cast<const char*>(dk_out);
    p.oq = static_cast<char*>(dq);
    p.ok = static_cast<char*>(dk);
    p.partial = partial;
    p.gq_st = strides[0] * esz, p.gq_sh = strides[1] * esz, p.gk_st = strides[2] * esz, p.gk_sh = strides[3] * esz;
    p.xq_st = strides[4] * esz, p.xq_sh = strides[5] * esz, p.xk_st = strides[6] * esz, p.xk_sh = strides[7] * esz;
    p.oq_st = strides[8] * esz, p.oq_sh = strides[9] * esz, p.ok_st = strides[10] * esz, p.ok_sh = strides[11] * esz;
    p.copy_q = Hq > 0 && !same_tensor(ts[0], ts[4]);
    p.copy_k = Hkv > 0 && !same_tensor(ts[1], ts[5]);
    const int st = launch_norm(p, g, D, dtype, o.pairing == ROPE_QK_PAIR_INTERLEAVED, true, s);
    if (st != ROPE_QK_OK) return st;
    const uint32_t slice = static_cast<uint32_t>((g.ntiles + g.nslices - 1) / g.nslices);
    const int32_t width = static_cast<int32_t>(2 * D);
    uint32_t nt = static_cast<uint32_t>(g.ntiles);
    void* a1[] = {&partial, &nt, const_cast<int32_t*>(&width), const_cast<uint32_t*>(&slice), &sums};
    hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(&dw_slices_kernel),
                                     dim3(static_cast<uint32_t>((width + kThreads - 1) / kThreads),
                                          static_cast<uint32_t>(g.nslices)),
                                     dim3(kThreads), a1, 0, s);
    if (err != hipSuccess) return ROPE_QK_ERR_LAUNCH;
  }
  if (dq_weight == nullptr && dk_weight == nullptr) return ROPE_QK_OK;
  uint32_t ns = static_cast<uint32_t>(g.nslices);
  int32_t d32 = static_cast<int32_t>(D);
  const double* sums_c = sums;
  void* a2[] = {const_cast<double**>(&sums_c), &ns, &d32, &dq_weight, &dk_weight};
  const hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(&dw_final_kernel),
                                         dim3(static_cast<uint32_t>((2 * D + kThreads - 1) / kThreads)),
                                         dim3(kThreads), a2, 0, s);
  return err == hipSuccess ? ROPE_QK_OK : ROPE_QK_ERR_LAUNCH;
}

}  // extern "C"
