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
//  * The work is a flat list of tasks in (token, head of q then k, chunk)
//    order.  Half rows of 128 bytes or more: a task is a 16-byte chunk of the
//    first half of a head together with the chunk D/2 further on (the
//    rotate_half partner), and one lane holds both.  Shorter half rows (1, 2
//    or 4 chunks): a task is a single 16-byte chunk and consecutive lanes
//    cover whole rows, so every wave-wide load and store covers whole 128-byte
//    lines (partner halves loaded by separate instructions cost ~13% of HBM
//    throughput on MI355X at D = 64).  A lane and the lane kG away hold the
//    two chunks of a row; through ds_swizzle each sends the other half of its
//    chunk's dwords, rotates its half of the pairs whole and sends the
//    other's outputs back, so each element is unpacked once.
//  * A workgroup owns one tile of consecutive tasks (256 lanes x 2 pairs or
//    x 1-8 chunks), which may begin and end inside a token, so every tile but
//    the last is full whatever the head count.  The grid is two-dimensional
//    rather than a grid-stride loop: a loop's second copy of the body would
//    set the register count (and so the occupancy) of every launch.
//  * Each lane first issues the load of its table entry's inv_freq and then
//    all its data loads (non-temporal), and only then finds the tile's token
//    positions -- a wave-uniform binary search of cu_seqlens through the
//    scalar cache, whose loads are not ordered behind the data -- and
//    evaluates cos/sin once per (token, pair) in float64 into LDS, where all
//    heads of q and k read them.  The memory counter completes in order, so
//    waiting for inv_freq does not wait for the data: the table is built
//    while the tile's data is in flight.
//  * Every task is rotated before any store is issued: a store's registers
//    cannot be reused until it completes, so an early store would make the
//    next task wait for a write acknowledgement.
//  * The rotation is done in float64 and rounded once: fp32 output is the
//    correctly rounded fp32; bf16 and fp16 output is the correctly rounded
//    bf16 or fp16 (fast float64->fp32->16-bit path, and an exact re-rounding
//    for the rare values whose fp32 rounding lands exactly on a midpoint of
//    the 16-bit grid, or, for fp16, in its subnormal range).
//  * All offsets are 64-bit; one build covers every tensor size.

#include "rope_common.h"

namespace {

constexpr uint32_t kMaxTasksPerToken = 65535;
constexpr int kPairTasks = 2;                         // chunk pairs per lane (pair tiles)
constexpr int kInterleaved = -1;                      // tile mode of interleaved pairing
constexpr int kUnitTasks = 8;      // chunks per lane: 16-bit chunk tasks in small launches, fp32 interleaved short rows
constexpr int kLongRowTasks = 4;   // chunks per lane: 16-bit chunk tasks in larger launches, fp32 unit tiles, interleaved long rows
constexpr int kPartRowTasks = 1;   // chunks per lane: larger 16-bit launches of rows rotating under a line of a longer head
constexpr int64_t kSmallLaunchTasks = int64_t(1) << 21;  // chunk-task launches of at most this many tasks are small
constexpr int64_t kShortRowChunks = 8;                // interleaved rows of up to this many chunks are short

// Resident workgroups per compute unit for pair tiles, measured on MI355X
// (bf16, D = 128, 0.5-10 GB per launch): with 256 or more tasks per token
// (e.g. 40 or 72 heads) 3 resident tiles stream 2-5% faster than 4-6, with
// fewer (e.g. 16 heads) 4 are best.  fp16, whose rounding test issues about
// a quarter more vector instructions, is best at 5 (1-9% faster than 3 on
// the 40- and 72-head shapes, 2% faster than 4 with 16 heads; 6 is no
// better).  Unit tiles run uncapped (5 per CU at their register count); any
// cap costs them 2-17%.
constexpr int kPairCapWide = 3;
constexpr int kPairCapNarrow = 4;
constexpr int kPairCapFp16 = 5;
constexpr int64_t kWideTasksPerToken = 256;

struct RopeParams {
  char* q;                 // base of q (bytes)
  char* k;                 // base of k (bytes)
  const int32_t* cu;       // cu_seqlens[nseq + 1]
  int64_t T;
  int64_t q_st, q_sh;      // byte strides of q along tokens / heads
  int64_t k_st, k_sh;      // byte strides of k along tokens / heads
  uint64_t magic_tok;      // ceil(2^40 / tasks_per_tok): exact n / tasks_per_tok for n < 2^24
  uint64_t magic_chunk;    // ceil(2^32 / chunks)
  uint64_t magic_half;     // ceil(2^32 / half)
  double rcp_tok;          // 1 / tasks_per_tok, rounded
  uint32_t ntiles;         // ceil(T * tasks_per_tok / tile_tasks) < 2^31
  uint32_t tok_step;       // unit tiles: 256 / tasks_per_tok when that is exact, else 0
  int32_t tile_tasks;      // consecutive tasks per tile
  int32_t nseq;
  int32_t Hq;
  int32_t tasks_per_tok;   // (Hq + Hkv) * chunks per row for unit tiles, per half row for pair tiles
  int32_t chunks;          // 16-byte chunks per half row
  int32_t half;            // D / 2
  int32_t half_bytes;      // (D / 2) * element size
  int32_t pos_offset;      // added to the positions of segment 0
  int32_t freq_fp32;       // 1: angles as float32 tables form them (inv_freq already rounded to float32)
  double sign;             // +1 forward, -1 backward
  double inv_freq[kMaxHalf];
};

// Rotate one task of 16-bit data: a holds x[i .. i+7], b holds x[i+D/2 .. i+D/2+7].
template <int kDtype, bool kExact>
__device__ __forceinline__ bool rotate_pair16(const u32x4& a, const u32x4& b, const double2* __restrict__ cs,
                                              int chunks, u32x4& oa, u32x4& ob) {
  bool tie = false;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const double2 c0 = cs[(2 * j) * chunks];
    const double2 c1 = cs[(2 * j + 1) * chunks];
    const f64x2 x1 = unpack16<kDtype>(a[j]), x2 = unpack16<kDtype>(b[j]);
    const double y1l = fma(x1.x, c0.x, -(x2.x * c0.y));
    const double y2l = fma(x2.x, c0.x, x1.x * c0.y);
    const double y1h = fma(x1.y, c1.x, -(x2.y * c1.y));
    const double y2h = fma(x2.y, c1.x, x1.y * c1.y);
    if (kExact) {
      oa[j] = pack16_exact<kDtype>(y1l, y1h);
      ob[j] = pack16_exact<kDtype>(y2l, y2h);
    } else {
      oa[j] = pack16_fast<kDtype>(y1l, y1h, tie);
      ob[j] = pack16_fast<kDtype>(y2l, y2h, tie);
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

// Partner exchange for unit tiles: lane l receives the dword lane l ^ kG
// passes (that lane holds the 16-byte chunk D/2 further on, or back, in the
// same row; a row's 2*kG chunks sit on 2*kG consecutive lanes).  ds_swizzle
// in bit-mask mode (and-mask 31, xor-mask kG, within each 32-lane half)
// moves it through the LDS crossbar, leaving the vector ALU to the rotation.
template <int kG>
__device__ __forceinline__ uint32_t partner_dword(uint32_t x) {
  static_assert(kG == 1 || kG == 2 || kG == 4, "unit tiles need a half row of 1, 2 or 4 chunks");
  constexpr int kPattern = (kG << 10) | 0x1F;
  return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(x), kPattern));
}

// (mask & x) | (~mask & y) in one bitfield insert.  Written out because a
// select between two elements of one vector register group becomes an
// element extract at a variable index (a compare and a select per element).
__device__ __forceinline__ uint32_t lane_pick(uint32_t mask, uint32_t x, uint32_t y) {
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(mask), "v"(x), "v"(y));
  return r;
}

// Unit tiles: a lane and its partner (the lane kG away) hold the two 16-byte
// chunks of one row (x[m .. m+7] and x[m+D/2 .. m+D/2+7] for 16-bit data).
// Each rotates two dwords' worth of the chunks' pairs whole: m holds two
// dwords of the lane's own chunk, g the same dwords of the partner's chunk,
// and the outputs are its own chunk's (om) and the partner chunk's (op), in
// the float64 operations of the paired form.
template <int kDtype, bool kExact>
__device__ __forceinline__ bool rotate_half16(const uint32_t (&m)[2], const uint32_t (&g)[2],
                                              const double2* __restrict__ cs, int chunks, uint32_t (&om)[2],
                                              uint32_t (&op)[2]) {
  bool tie = false;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const double2 c0 = cs[(2 * j) * chunks];
    const double2 c1 = cs[(2 * j + 1) * chunks];
    const f64x2 x1 = unpack16<kDtype>(m[j]), x2 = unpack16<kDtype>(g[j]);
    const double y1l = fma(x1.x, c0.x, -(x2.x * c0.y));
    const double y2l = fma(x2.x, c0.x, x1.x * c0.y);
    const double y1h = fma(x1.y, c1.x, -(x2.y * c1.y));
    const double y2h = fma(x2.y, c1.x, x1.y * c1.y);
    if (kExact) {
      om[j] = pack16_exact<kDtype>(y1l, y1h);
      op[j] = pack16_exact<kDtype>(y2l, y2h);
    } else {
      om[j] = pack16_fast<kDtype>(y1l, y1h, tie);
      op[j] = pack16_fast<kDtype>(y2l, y2h, tie);
    }
  }
  return tie;
}

__device__ __forceinline__ void rotate_half_f32(const uint32_t (&m)[2], const uint32_t (&g)[2],
                                                const double2* __restrict__ cs, int chunks, uint32_t (&om)[2],
                                                uint32_t (&op)[2]) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const double2 c = cs[j * chunks];
    const double x1 = static_cast<double>(__uint_as_float(m[j]));
    const double x2 = static_cast<double>(__uint_as_float(g[j]));
    om[j] = __float_as_uint(static_cast<float>(fma(x1, c.x, -(x2 * c.y))));
    op[j] = __float_as_uint(static_cast<float>(fma(x2, c.x, x1 * c.y)));
  }
}

// Interleaved pairing (element 2i with 2i + 1): both elements of a pair sit
// in one chunk, so a lane rotates its own chunk with no exchange.  16-bit
// data: each dword holds one pair (x[2i] low, x[2i+1] high).
template <int kDtype, bool kExact>
__device__ __forceinline__ bool rotate_pairs16(const u32x4& own, const double2* __restrict__ cs, int chunks,
                                               u32x4& out) {
  bool tie = false;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const double2 c = cs[j * chunks];
    const f64x2 x = unpack16<kDtype>(own[j]);
    const double y1 = fma(x.x, c.x, -(x.y * c.y));
    const double y2 = fma(x.y, c.x, x.x * c.y);
    out[j] = kExact ? pack16_exact<kDtype>(y1, y2) : pack16_fast<kDtype>(y1, y2, tie);
  }
  return tie;
}

// fp32: dwords (0, 1) and (2, 3) are the two pairs of a chunk.
__device__ __forceinline__ void rotate_pairs_f32(const u32x4& own, const double2* __restrict__ cs, int chunks,
                                                 u32x4& out) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const double2 c = cs[j * chunks];
    const double x1 = static_cast<double>(__uint_as_float(own[2 * j]));
    const double x2 = static_cast<double>(__uint_as_float(own[2 * j + 1]));
    out[2 * j] = __float_as_uint(static_cast<float>(fma(x1, c.x, -(x2 * c.y))));
    out[2 * j + 1] = __float_as_uint(static_cast<float>(fma(x2, c.x, x1 * c.y)));
  }
}

// One tile: tile_tasks consecutive tasks of the flat (token, head, chunk)
// order, which may start and end inside a token.
// kG = 0: a task is a pair of 16-byte chunks D/2 apart (one lane holds both).
// kG = 1, 2, 4 (half rows of fewer than 128 bytes): a task is one 16-byte
// chunk; consecutive lanes cover whole rows, so every load and store of a
// wave covers whole cache lines, and the partner chunk comes from the lane
// kG away.
// kG = kInterleaved: interleaved pairing; a task is one 16-byte chunk of whole
// pairs, consecutive lanes on consecutive chunks.
// kPosOnly (the positions test hook): run the tile's geometry and position
// code only, and write the tile's first token and its tokens' positions to
// pos_out[0 .. ntok] instead of loading, rotating and storing anything.
template <int kDtype, int kG, int kTPT, bool kPosOnly = false>
__device__ __forceinline__ void rope_tile(const RopeParams& p, uint32_t tile, int32_t* s_pos, double2* s_cs,
                                          int32_t* pos_out = nullptr) {
  constexpr bool k16 = kDtype != ROPE_QK_FP32;            // bf16 or fp16 storage
  constexpr int kVec = k16 ? 8 : 4;                        // elements per 16 bytes
  constexpr int kPPC = kG == kInterleaved ? kVec / 2 : kVec;  // table pairs per chunk
  const int tid = threadIdx.x;
  const cu_ptr cu = (cu_ptr)p.cu;  // address-space cast (C-style: reinterpret_cast cannot change it)
  const int32_t nseq = p.nseq;
  const int32_t tpt = p.tasks_per_tok;
  {
    // first task n0 = t0 * tasks_per_tok + r0 (n0 < 2^42 is exact in float64;
    // the rounded quotient is off by at most one)
    const int64_t n0 = static_cast<int64_t>(tile) * p.tile_tasks;
    int32_t t0i = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(static_cast<double>(n0) * p.rcp_tok));
    int64_t r0l = n0 - static_cast<int64_t>(t0i) * tpt;
    if (r0l < 0) { t0i -= 1; r0l += tpt; }
    if (r0l >= tpt) { t0i += 1; r0l -= tpt; }
    const int64_t t0 = t0i;
    const uint32_t r0 = static_cast<uint32_t>(r0l);
    const int64_t n_end = min(n0 + p.tile_tasks, p.T * tpt);          // one past the tile's last task
    const int ntok = static_cast<int>(div_tok(static_cast<uint32_t>(n_end - n0) + r0 - 1, p.magic_tok)) + 1;
    const int64_t t_end = t0 + ntok;  // one past the tile's last token
    const int nent = ntok * p.half;
    // unit tiles: where the table's second copy (sine negated) starts; the 4
    // entries past a multiple of 16 keep a wave's reads of the two copies on
    // different LDS banks
    const int alt = ((nent + 15) & ~15) + 4;

    // 1. inv_freq of this thread's table entries.  Issued before the tile's
    //    data: the memory counter completes in order, so the table can be
    //    built while the data loads are still in flight.
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
    __builtin_amdgcn_sched_barrier(0);

    // 2. every load of the tile (lanes past the last token re-read the tile's first task)
    u32x4 a[kTPT], b[kTPT];
    gchar* ptr[kTPT];
    int tt_of[kTPT], c_of[kTPT];
    bool act[kTPT];
    if constexpr (!kPosOnly) {
    // Unit tiles whose token task count divides 256 (e.g. 16 heads at D = 64):
    // a lane's tasks are tok_step tokens apart at the same head and chunk, so
    // only the first address needs the general computation.
    const bool stepped = kG != 0 && p.tok_step != 0;  // wave-uniform
    bool is_q0 = false;
#pragma unroll
    for (int u = 0; u < kTPT; ++u) {
      act[u] = n0 + static_cast<int64_t>(tid + u * kThreads) < n_end;
      if (stepped && u > 0) {
        const int64_t step = static_cast<int64_t>(u * p.tok_step) * (is_q0 ? p.q_st : p.k_st);
        ptr[u] = ptr[0] + (act[u] ? step : int64_t(0));  // offset select keeps the global address space
        tt_of[u] = act[u] ? tt_of[0] + u * static_cast<int>(p.tok_step) : tt_of[0];
        c_of[u] = c_of[0];
      } else {
        const uint32_t l_raw = r0 + static_cast<uint32_t>(tid + u * kThreads);  // task index from the tile's first token
        const uint32_t l = act[u] ? l_raw : r0;
        const uint32_t tt = div_tok(l, p.magic_tok);
        const uint32_t r = l - tt * static_cast<uint32_t>(tpt);
        uint32_t h, c, cc;  // head, chunk within the row, chunk within the half row
        if constexpr (kG == 0 || kG == kInterleaved) {
          h = div_small(r, p.magic_chunk);
          c = r - h * static_cast<uint32_t>(p.chunks);
          cc = c;
        } else {
          h = r / (2 * kG);
          c = r % (2 * kG);
          cc = c % kG;
        }
        const int64_t t = t0 + tt;
        const bool is_q = static_cast<int32_t>(h) < p.Hq;
        if (u == 0) is_q0 = is_q;
        gchar* row = is_q ? (gchar*)p.q + t * p.q_st + static_cast<int64_t>(h) * p.q_sh
                          : (gchar*)p.k + t * p.k_st + static_cast<int64_t>(h - p.Hq) * p.k_sh;
        ptr[u] = row + static_cast<int64_t>(c) * 16;
        tt_of[u] = static_cast<int>(tt);
        c_of[u] = static_cast<int>(cc);
      }
      // streamed once: non-temporal, so they do not displace other data in the caches
      a[u] = __builtin_nontemporal_load(reinterpret_cast<const gu32x4*>(ptr[u]));
      if constexpr (kG == 0) b[u] = __builtin_nontemporal_load(reinterpret_cast<const gu32x4*>(ptr[u] + p.half_bytes));
    }
    }
    __builtin_amdgcn_sched_barrier(0);

    // 3. positions (scalar loads, not ordered behind the data) and the table
    const int32_t s0 = last_start_at_or_before(cu, nseq, t0);
    const int64_t cu_last = cu[nseq];
    const int64_t cu_first_end = cu[1];  // segment 0 is [cu[0], cu[1]) (nseq >= 1 here)
    int64_t start[kEnt];
#pragma unroll
    for (int v = 0; v < kEnt; ++v) start[v] = s0 >= 0 ? static_cast<int64_t>(cu[s0]) : INT64_MIN;
    for (int32_t j = s0 + 1; j <= nseq; ++j) {  // boundaries inside the tile (wave-uniform)
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
        if constexpr (kPosOnly) {
          if (i_e[v] == 0) pos_out[1 + tt_e[v]] = pos;
          if (e == 0) pos_out[0] = static_cast<int32_t>(t0);
          continue;
        }
        if (pos >= 0) {
          double sn, cs;
          // float32 convention: float32 position times float32 frequency, one rounding
          const double ang = p.freq_fp32 ? static_cast<double>(static_cast<float>(pos) * static_cast<float>(f[v]))
                                         : static_cast<double>(pos) * f[v];
          rope_sincos(ang, &sn, &cs);
          const int slot = cs_slot(tt_e[v], i_e[v], kPPC, p.chunks);
          s_cs[slot] = make_double2(cs, p.sign * sn);
          if constexpr (kG > 0) s_cs[alt + slot] = make_double2(cs, -p.sign * sn);
        }
      }
    }
    if constexpr (kPosOnly) return;
    __syncthreads();

    // 4. rotate every task, then store them all; tokens outside every
    //    sequence are left untouched
    bool st[kTPT];
    u32x4 oa[kTPT], ob[kTPT];
    // Unit tiles: a tile starts on a row boundary and holds whole rows of
    // 2 kG tasks (its task count is a multiple of 2 kG), so every chunk a lane
    // holds sits at position tid mod 2 kG of its row, always in the same half.
    // A lane in the second half reads the table copy with the sine negated,
    // starting kPPC / 2 entries further on, at the pairs of dwords 2-3 that it
    // rotates (see the rotation below).
    const bool fst = kG <= 0 || (tid & kG) == 0;
    const uint32_t keep = fst ? 0xFFFFFFFFu : 0u;  // bit mask selecting the first operand of lane_pick
    const double2* tab = kG > 0 && !fst ? s_cs + alt + (kPPC / 2) * kG : s_cs;
#pragma unroll
    for (int u = 0; u < kTPT; ++u) {
      st[u] = act[u] && s_pos[tt_of[u]] >= 0;
      const int chunks = kG > 0 ? kG : p.chunks;
      const double2* cs = tab + tt_of[u] * kPPC * chunks + c_of[u];
      if constexpr (kG == kInterleaved) {
        if constexpr (k16) {
          if (rotate_pairs16<kDtype, false>(a[u], cs, chunks, oa[u]))
            rotate_pairs16<kDtype, true>(a[u], cs, chunks, oa[u]);
        } else {
          rotate_pairs_f32(a[u], cs, chunks, oa[u]);
        }
      } else if constexpr (kG == 0) {
        if constexpr (k16) {
          if (rotate_pair16<kDtype, false>(a[u], b[u], cs, chunks, oa[u], ob[u]))
            rotate_pair16<kDtype, true>(a[u], b[u], cs, chunks, oa[u], ob[u]);
        } else {
          rotate_f32(a[u], b[u], cs, chunks, oa[u], ob[u]);
        }
      } else {
        // The lane with the first-half chunk rotates the pairs of dwords 0-1
        // of both chunks, its partner those of dwords 2-3: each sends the
        // dwords of its own chunk that the other needs, rotates, and sends the
        // other's outputs back, so every element is unpacked once and every
        // table entry read once for both elements of its pair.  The partner
        // reads the table copy with the sine negated, which turns the pair
        // rotation (own, received) into (second element's output, first
        // element's output): the paired form's float64 operations, bit for bit.
        uint32_t m[2], g[2], om[2], op[2];
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          m[d] = lane_pick(keep, a[u][d], a[u][d + 2]);
          g[d] = partner_dword<kG>(lane_pick(keep, a[u][d + 2], a[u][d]));
        }
        if constexpr (k16) {
          if (rotate_half16<kDtype, false>(m, g, cs, chunks, om, op))
            rotate_half16<kDtype, true>(m, g, cs, chunks, om, op);
        } else {
          rotate_half_f32(m, g, cs, chunks, om, op);
        }
        uint32_t back[2];
#pragma unroll
        for (int d = 0; d < 2; ++d) back[d] = partner_dword<kG>(op[d]);
        oa[u] = u32x4{lane_pick(keep, om[0], back[0]), lane_pick(keep, om[1], back[1]),
                      lane_pick(keep, back[0], om[0]), lane_pick(keep, back[1], om[1])};
      }
    }
#pragma unroll
    for (int u = 0; u < kTPT; ++u) {
      if (!st[u]) continue;
      __builtin_nontemporal_store(oa[u], reinterpret_cast<gu32x4*>(ptr[u]));
      if constexpr (kG == 0) __builtin_nontemporal_store(ob[u], reinterpret_cast<gu32x4*>(ptr[u] + p.half_bytes));
    }
  }
}

// One tile per workgroup; the grid's rows cover launches of more than kGridX tiles.
template <int kDtype, int kG, int kTPT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
void rope_qk_kernel(const RopeParams p) {
  __shared__ int32_t s_pos[kMaxTileTokens];  // positions of the tile's tokens
  extern __shared__ double2 s_cs[];          // [tokens touched * half] {cos, sign*sin}
  const uint32_t tile = blockIdx.y * gridDim.x + blockIdx.x;
  if (tile < p.ntiles) rope_tile<kDtype, kG, kTPT>(p, tile, s_pos, s_cs);
}

// The positions test hook: one tile per workgroup, in the geometry of the
// call it was prepared for, through the rotation tile's own position code;
// row `tile` of out receives the tile's first token and the positions of the
// tokens it touches.
__global__ __launch_bounds__(kThreads) void rope_tile_positions_kernel(const RopeParams p, int32_t* out,
                                                                       int64_t row_len) {
  __shared__ int32_t s_pos[kMaxTileTokens];
  const uint32_t tile = blockIdx.y * gridDim.x + blockIdx.x;
  if (tile < p.ntiles)
    rope_tile<ROPE_QK_BF16, 0, kPairTasks, true>(p, tile, s_pos, nullptr, out + static_cast<int64_t>(tile) * row_len);
}

// Per-token positions (rope_qk_positions): the same position code on tiles of
// kPositionTileTokens whole tokens (one task per token), each tile writing
// its positions at out[t0 ...] through a staging row in LDS.
constexpr int kPositionTileTokens = kMaxTileTokens;

__global__ __launch_bounds__(kThreads) void rope_token_positions_kernel(const RopeParams p, int32_t* out) {
  __shared__ int32_t s_pos[kMaxTileTokens];
  __shared__ int32_t s_row[1 + kPositionTileTokens];
  const uint32_t tile = blockIdx.y * gridDim.x + blockIdx.x;
  if (tile >= p.ntiles) return;
  const int64_t t0 = static_cast<int64_t>(tile) * kPositionTileTokens;  // tiles of whole tokens
  const int64_t t = t0 + threadIdx.x;
  if (p.nseq == 0) {  // no sequence: every token is outside
    if (threadIdx.x < kPositionTileTokens && t < p.T) out[t] = -1;
    return;
  }
  rope_tile<ROPE_QK_BF16, 0, kPairTasks, true>(p, tile, s_pos, nullptr, s_row);
  __syncthreads();
  if (threadIdx.x < kPositionTileTokens && t < p.T) out[t] = s_row[1 + threadIdx.x];
}

// A rotation call after its checks: the kernel parameters, the kernel and its
// launch shape (fn == nullptr: nothing to launch), and the most tokens one
// tile touches.
struct RopeLaunch {
  RopeParams p;
  const void* fn;
  dim3 grid;
  size_t lds;
  int64_t span;
};

// Checks and geometry of a rotation call.  With tensors == false (the
// positions hook) q, k and their strides are not looked at.
int prepare_rope(void* q, void* k, const int32_t* cu, int64_t nseq, int64_t T, int64_t Hq, int64_t Hkv, int64_t D,
                 int64_t q_st, int64_t q_sh, int64_t k_st, int64_t k_sh, double theta, int dtype,
                 const rope_qk_options* options, double sign, bool tensors, RopeLaunch* L) {
  L->fn = nullptr;
  const rope_qk_options o = options ? *options : rope_qk_options{};
  const int status = check_call(dtype, nseq, T, Hq, Hkv, D, theta, o);
  if (status != ROPE_QK_OK) return status;
  const int64_t r = o.rotary_dim == 0 ? D : o.rotary_dim;  // elements of each head that are rotated
  if (T == 0 || nseq == 0 || Hq + Hkv == 0) return ROPE_QK_OK;
  const int64_t esz = dtype == ROPE_QK_FP32 ? 4 : 2;
  if (cu == nullptr) return ROPE_QK_ERR_NULL;
  if (tensors) {
    if ((Hq > 0 && q == nullptr) || (Hkv > 0 && k == nullptr)) return ROPE_QK_ERR_NULL;
    if ((Hq > 0 && (q_st < 0 || q_sh < 0 || rows_overlap(T, Hq, D, q_st, q_sh))) ||
        (Hkv > 0 && (k_st < 0 || k_sh < 0 || rows_overlap(T, Hkv, D, k_st, k_sh))))
      return ROPE_QK_ERR_LAYOUT;
    // q and k are rotated by one launch: they must share no byte (the
    // strides are at most 2^40 bytes here, so the byte strides fit int64)
    if (Hq > 0 && Hkv > 0 &&
        !rows_disjoint(q, Hq, q_st * esz, q_sh * esz, k, Hkv, k_st * esz, k_sh * esz, T, D * esz))
      return ROPE_QK_ERR_LAYOUT;
  }

  const bool interleaved = o.pairing == ROPE_QK_PAIR_INTERLEAVED;
  const int64_t half = r / 2;  // rotated pairs per head
  // 16-byte chunks holding the first elements of pairs: half a rotated row, or all of it when interleaved
  if (((interleaved ? r : half) * esz) % 16) return ROPE_QK_ERR_ALIGN;
  if (tensors) {
    if (Hq > 0 && ((reinterpret_cast<uintptr_t>(q) % 16) || (q_st * esz) % 16 || (q_sh * esz) % 16))
      return ROPE_QK_ERR_ALIGN;
    if (Hkv > 0 && ((reinterpret_cast<uintptr_t>(k) % 16) || (k_st * esz) % 16 || (k_sh * esz) % 16))
      return ROPE_QK_ERR_ALIGN;
  }

  const int64_t chunks = (interleaved ? r : half) * esz / 16;
  // rotate_half with half rows of 1, 2 or 4 chunks: unit tiles (one chunk per
  // task, partner by lane exchange); interleaved: one chunk of whole pairs per task
  const int unit_g = !interleaved && (chunks == 1 || chunks == 2 || chunks == 4) ? static_cast<int>(chunks) : 0;
  const bool chunk_tasks = unit_g != 0 || interleaved;
  const int64_t tasks_per_tok = (Hq + Hkv) * (unit_g ? 2 * chunks : chunks);
  if (tasks_per_tok > kMaxTasksPerToken) return ROPE_QK_ERR_SHAPE;
  // Chunks per lane, measured on MI355X (bf16 and fp16, HIP graphs of
  // forward launches over resident batches):
  //  - 16-bit launches of up to 2^21 tasks (64 MiB of traffic, e.g. 16 heads
  //    of D = 64 over 16,384 tokens, two tiles per compute unit): 8, which
  //    amortises each tile's work best; 2 and 4 are 8-15% slower;
  //  - larger 16-bit launches (0.13-1 GB at D = 64): 4, 2-7% faster than 8;
  //    rotate_half rows that rotate less than one 128-byte line of a longer
  //    head (rotary_dim < D with r / 2 elements under 64 bytes): 1, 14-26%
  //    faster than 8 from 2^21 tasks on (the lines' unrotated rest is fetched
  //    too, so these launches count as large from half the task count);
  //  - interleaved rows of more than 8 chunks (D = 128 bf16): 4, 7% faster
  //    than 8 (register count 128 -> 90, occupancy 4 -> 5);
  //  - fp32: 4 for unit tiles (8 would spill), 8 for short interleaved rows.
  const bool part_row = unit_g != 0 && unit_g < 4 && r < D;
  const bool small_launch = T * tasks_per_tok <= (part_row ? kSmallLaunchTasks / 2 : kSmallLaunchTasks);
  int64_t lane_tasks = kPairTasks;
  if (chunk_tasks) {
    if (interleaved)
      lane_tasks = chunks > kShortRowChunks || (dtype != ROPE_QK_FP32 && !small_launch) ? kLongRowTasks : kUnitTasks;
    else if (dtype == ROPE_QK_FP32)
      lane_tasks = kLongRowTasks;
    else
      lane_tasks = small_launch ? kUnitTasks : part_row ? kPartRowTasks : kLongRowTasks;
  }

  // a tile touches at most cap_tokens tokens, so its table and positions fit in LDS
  int64_t cap_tokens = kMaxTableBytes / (half * 16);
  if (cap_tokens > kMaxTileTokens) cap_tokens = kMaxTileTokens;
  int64_t tile_tasks = int64_t(kThreads) * lane_tasks;
  if (tile_tasks > (cap_tokens - 1) * tasks_per_tok) tile_tasks = (cap_tokens - 1) * tasks_per_tok;
  // tokens one tile touches: exactly tile_tasks / tasks_per_tok when every tile starts on a token
  const int64_t span = tile_tasks % tasks_per_tok == 0 ? tile_tasks / tasks_per_tok
                                                      : (tasks_per_tok + tile_tasks - 2) / tasks_per_tok + 1;
  const int64_t ntiles = (T * tasks_per_tok + tile_tasks - 1) / tile_tasks;
  if (ntiles > INT32_MAX) return ROPE_QK_ERR_SHAPE;

  RopeParams& p = L->p;
  p.q = static_cast<char*>(q);
  p.k = static_cast<char*>(k);
  p.cu = cu;
  p.T = T;
  p.q_st = q_st * esz;
  p.q_sh = q_sh * esz;
  p.k_st = k_st * esz;
  p.k_sh = k_sh * esz;
  p.magic_tok = ((uint64_t(1) << 40) + tasks_per_tok - 1) / tasks_per_tok;
  p.magic_chunk = ((uint64_t(1) << 32) + chunks - 1) / chunks;
  p.magic_half = ((uint64_t(1) << 32) + half - 1) / half;
  p.tok_step = chunk_tasks && kThreads % tasks_per_tok == 0 ? static_cast<uint32_t>(kThreads / tasks_per_tok) : 0u;
  p.rcp_tok = 1.0 / static_cast<double>(tasks_per_tok);
  p.ntiles = static_cast<uint32_t>(ntiles);
  p.tile_tasks = static_cast<int32_t>(tile_tasks);
  p.nseq = static_cast<int32_t>(nseq);
  p.Hq = static_cast<int32_t>(Hq);
  p.tasks_per_tok = static_cast<int32_t>(tasks_per_tok);
  p.chunks = static_cast<int32_t>(chunks);
  p.half = static_cast<int32_t>(half);
  p.half_bytes = static_cast<int32_t>(half * esz);
  p.pos_offset = static_cast<int32_t>(o.pos_offset);
  p.freq_fp32 = o.freq_precision == ROPE_QK_FREQ_FP32;
  p.sign = sign;
  fill_inv_freq(theta, r, o, p.inv_freq);

  // LDS: the table of the tokens one tile touches; for pair tiles, padded so
  // that at most the measured best number of workgroups share a compute unit
  // (unit tiles: two copies, the second with the sine negated, 16-entry aligned plus 4)
  size_t lds = static_cast<size_t>(unit_g ? 2 * span * half + 20 : span * half) * sizeof(double2);
  if (!chunk_tasks) {
    const int64_t cap = dtype == ROPE_QK_FP16                ? kPairCapFp16
                        : tasks_per_tok >= kWideTasksPerToken ? kPairCapWide
                                                              : kPairCapNarrow;
    const size_t pad = static_cast<size_t>(kLdsPerCu / (cap + 1) + 1024 - kMaxTileTokens * sizeof(int32_t));
    if (lds < pad) lds = pad;
  }
  const int64_t gx = ntiles < kGridX ? ntiles : kGridX;
  L->grid = dim3(static_cast<uint32_t>(gx), static_cast<uint32_t>((ntiles + gx - 1) / gx));
  L->lds = lds;
  L->span = span;

#define ROPE_FN(DT, G, TPT) reinterpret_cast<const void*>(&rope_qk_kernel<DT, G, TPT>)
#define ROPE_UNIT(DT, TPT) \
  (unit_g == 1 ? ROPE_FN(DT, 1, TPT) : unit_g == 2 ? ROPE_FN(DT, 2, TPT) : ROPE_FN(DT, 4, TPT))
#define ROPE_PICK(DT, UNIT)                                                                                      \
  (interleaved ? (lane_tasks == kUnitTasks ? ROPE_FN(DT, kInterleaved, kUnitTasks)                                \
                                           : ROPE_FN(DT, kInterleaved, kLongRowTasks))                             \
   : unit_g == 0 ? ROPE_FN(DT, 0, kPairTasks)                                                                     \
                 : UNIT)
#define ROPE_PICK16(DT)                                                                  \
  ROPE_PICK(DT, (lane_tasks == kUnitTasks       ? ROPE_UNIT(DT, kUnitTasks)              \
                 : lane_tasks == kLongRowTasks  ? ROPE_UNIT(DT, kLongRowTasks)           \
                 : unit_g == 1                  ? ROPE_FN(DT, 1, kPartRowTasks)          \
                                                : ROPE_FN(DT, 2, kPartRowTasks)))
  L->fn = dtype == ROPE_QK_BF16   ? ROPE_PICK16(ROPE_QK_BF16)
          : dtype == ROPE_QK_FP16 ? ROPE_PICK16(ROPE_QK_FP16)
                                  : ROPE_PICK(ROPE_QK_FP32, ROPE_UNIT(ROPE_QK_FP32, kLongRowTasks));
#undef ROPE_PICK16
#undef ROPE_PICK
#undef ROPE_UNIT
#undef ROPE_FN
  return ROPE_QK_OK;
}

int launch_rope(void* q, void* k, const int32_t* cu, int64_t nseq, int64_t T, int64_t Hq, int64_t Hkv, int64_t D,
                int64_t q_st, int64_t q_sh, int64_t k_st, int64_t k_sh, double theta, int dtype,
                const rope_qk_options* options, void* stream, double sign) {
  RopeLaunch L;
  const int status = prepare_rope(q, k, cu, nseq, T, Hq, Hkv, D, q_st, q_sh, k_st, k_sh, theta, dtype, options, sign,
                                  true, &L);
  if (status != ROPE_QK_OK || L.fn == nullptr) return status;
  void* args[] = {&L.p};
  const hipError_t err = hipLaunchKernel(L.fn, L.grid, dim3(kThreads), args, L.lds, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? ROPE_QK_OK : ROPE_QK_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int rope_qk_fwd(void* q, void* k, const int32_t* cu_seqlens, int64_t nseq, int64_t T, int64_t Hq, int64_t Hkv,
                int64_t D, int64_t q_stride_t, int64_t q_stride_h, int64_t k_stride_t, int64_t k_stride_h,
                double theta, int dtype, void* stream) {
  return launch_rope(q, k, cu_seqlens, nseq, T, Hq, Hkv, D, q_stride_t, q_stride_h, k_stride_t, k_stride_h, theta,
                     dtype, nullptr, stream, 1.0);
}

int rope_qk_bwd(void* dq, void* dk, const int32_t* cu_seqlens, int64_t nseq, int64_t T, int64_t Hq, int64_t Hkv,
                int64_t D, int64_t q_stride_t, int64_t q_stride_h, int64_t k_stride_t, int64_t k_stride_h,
                double theta, int dtype, void* stream) {
  return launch_rope(dq, dk, cu_seqlens, nseq, T, Hq, Hkv, D, q_stride_t, q_stride_h, k_stride_t, k_stride_h,
                     theta, dtype, nullptr, stream, -1.0);
}

int rope_qk_fwd_opt(void* q, void* k, const int32_t* cu_seqlens, int64_t nseq, int64_t T, int64_t Hq, int64_t Hkv,
                    int64_t D, int64_t q_stride_t, int64_t q_stride_h, int64_t k_stride_t, int64_t k_stride_h,
                    double theta, int dtype, const rope_qk_options* options, void* stream) {
  return launch_rope(q, k, cu_seqlens, nseq, T, Hq, Hkv, D, q_stride_t, q_stride_h, k_stride_t, k_stride_h, theta,
                     dtype, options, stream, 1.0);
}

int rope_qk_bwd_opt(void* dq, void* dk, const int32_t* cu_seqlens, int64_t nseq, int64_t T, int64_t Hq,
                    int64_t Hkv, int64_t D, int64_t q_stride_t, int64_t q_stride_h, int64_t k_stride_t,
                    int64_t k_stride_h, double theta, int dtype, const rope_qk_options* options, void* stream) {
  return launch_rope(dq, dk, cu_seqlens, nseq, T, Hq, Hkv, D, q_stride_t, q_stride_h, k_stride_t, k_stride_h,
                     theta, dtype, options, stream, -1.0);
}

int rope_qk_positions(const int32_t* cu_seqlens, int64_t nseq, int64_t T, int32_t* pos_out, void* stream) {
  if (nseq < 0 || T < 0 || T > INT32_MAX || nseq >= INT32_MAX) return ROPE_QK_ERR_SHAPE;
  if (T == 0) return ROPE_QK_OK;
  if (cu_seqlens == nullptr || pos_out == nullptr) return ROPE_QK_ERR_NULL;
  // one task per token, tiles of kPositionTileTokens whole tokens, no pos_offset
  const int64_t ntiles = (T + kPositionTileTokens - 1) / kPositionTileTokens;
  RopeParams p{};
  p.cu = cu_seqlens;
  p.T = T;
  p.nseq = static_cast<int32_t>(nseq);
  p.tasks_per_tok = 1;
  p.tile_tasks = kPositionTileTokens;
  p.half = 1;
  p.magic_tok = uint64_t(1) << 40;
  p.magic_half = uint64_t(1) << 32;
  p.rcp_tok = 1.0;
  p.ntiles = static_cast<uint32_t>(ntiles);
  const int64_t gx = ntiles < kGridX ? ntiles : kGridX;
  const dim3 grid(static_cast<uint32_t>(gx), static_cast<uint32_t>((ntiles + gx - 1) / gx));
  void* args[] = {&p, &pos_out};
  const hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(&rope_token_positions_kernel), grid,
                                         dim3(kThreads), args, 0, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? ROPE_QK_OK : ROPE_QK_ERR_LAUNCH;
}

int rope_qk_tile_positions(const int32_t* cu_seqlens, int64_t nseq, int64_t T, int64_t Hq, int64_t Hkv, int64_t D,
                           int dtype, const rope_qk_options* options, int32_t* out, int64_t out_len,
                           int64_t* ntiles, int64_t* row_len, void* stream) {
  if (ntiles == nullptr || row_len == nullptr) return ROPE_QK_ERR_NULL;
  *ntiles = 0;
  *row_len = 0;
  RopeLaunch L;
  const int status = prepare_rope(nullptr, nullptr, cu_seqlens, nseq, T, Hq, Hkv, D, 0, 0, 0, 0, 1.0, dtype, options,
                                  1.0, false, &L);
  if (status != ROPE_QK_OK || L.fn == nullptr) return status;
  *ntiles = L.p.ntiles;
  *row_len = 1 + L.span;
  if (out == nullptr) return ROPE_QK_OK;  // the geometry only
  if (out_len < *ntiles * *row_len) return ROPE_QK_ERR_SHAPE;
  int64_t rl = *row_len;
  void* args[] = {&L.p, &out, &rl};
  const hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(&rope_tile_positions_kernel), L.grid,
                                         dim3(kThreads), args, 0, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? ROPE_QK_OK : ROPE_QK_ERR_LAUNCH;
}

const char* rope_qk_strerror(int status) {
  switch (status) {
    case ROPE_QK_OK: return "ok";
    case ROPE_QK_ERR_NULL: return "a required pointer is NULL";
    case ROPE_QK_ERR_SHAPE: return "unsupported shape (negative size, D odd/<2/>512, T >= 2^31, too many heads)";
    case ROPE_QK_ERR_DTYPE: return "unsupported dtype (expected ROPE_QK_FP32, ROPE_QK_BF16 or ROPE_QK_FP16)";
    case ROPE_QK_ERR_ALIGN: return "misaligned: pointers, strides and D/2 must be multiples of 16 bytes";
    case ROPE_QK_ERR_THETA: return "theta must be finite and > 0";
    case ROPE_QK_ERR_LAUNCH: return "HIP kernel launch failed";
    case ROPE_QK_ERR_LAYOUT: return "negative strides, overlapping rows, or tensors that share memory";
    case ROPE_QK_ERR_OPTION:
      return "an option is out of range (pos_offset, rotary_dim, pairing, scaling, freq_precision, reserved or eps)";
    case ROPE_QK_ERR_WORKSPACE: return "workspace missing or smaller than rope_qk_norm_bwd_workspace_bytes";
    case ROPE_QK_ERR_SCRATCH:
      return "the call needs more weight-gradient scratch than rope_qk_norm_bwd_noalloc's static 24 MiB";
    default: return "unknown status";
  }
}

}  // extern "C"
