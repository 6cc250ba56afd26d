/*
 * rope_qk.h -- fused, in-place rotary position embedding of the query and key
 * tensors of a packed variable-length batch, forward and backward, on AMD
 * Instinct MI355X (gfx950).  C ABI: plain pointers and sizes, no framework
 * types.
 *
 * What the operation is
 * ---------------------
 * "Unsloth prétend accélérer 5 fois l'entraînement des LLM avec de nouveaux
 * noyaux Triton et un auto-packing" (seventnews.com), paragraph on the fused
 * QK RoPE kernel: one kernel rotates both q and k (instead of one kernel each),
 * accepts variable-length input, and works fully in place without clones or
 * contiguous transposes.  The same article's auto-packing paragraph: short
 * sequences are concatenated along one token axis and only their length
 * metadata is kept, so that nothing leaks between samples.  "Chronicals: A
 * High-Performance Framework for LLM Fine-Tuning with 3.51x Speedup over
 * Unsloth", abstract, optimisation (1): QK-RoPE is one of the fused kernels
 * that remove memory traffic.  The article's LONG_INDEXING paragraph: 500K-token
 * contexts overflowed 32-bit indexing; here every offset is 64-bit in the one
 * build.
 *
 * The pages print no formula.  The reading implemented is the standard rotary
 * embedding (RoFormer, Su et al. 2021) in the rotate_half layout: for every
 * token t inside a packed sequence, every head of q and of k, and i < D/2,
 *
 *   inv_freq[i] = theta^(-2i/D)            (float64, computed on the host)
 *   a           = pos(t) * inv_freq[i]      (float64)
 *   x1 = x[t,h,i], x2 = x[t,h,i+D/2]
 *   forward:   x1' = x1 cos a - x2 sin a,   x2' = x2 cos a + x1 sin a
 *   backward:  the same with sin a -> -sin a (the transpose), applied to dq, dk
 *
 * pos(t) = t - cu_seqlens[s], where s is the last index with cu_seqlens[s] <= t,
 * so positions restart at 0 at every sequence boundary.  Tokens t < cu_seqlens[0]
 * and t >= cu_seqlens[nseq] are not written (a tile may read them while its
 * positions are still being found).  The rotation is
 * evaluated in float64 and rounded once to the storage type (round to nearest,
 * ties to even): bf16 and fp16 results are the correctly rounded bf16 or fp16
 * of the float64 rotation, fp32 results the correctly rounded fp32.
 *
 * Memory, ownership, ordering
 * ---------------------------
 * All tensor pointers are device memory owned by the caller; the library
 * allocates nothing, and its only state is the static scratch array of
 * rope_qk_norm_bwd_noalloc (part of its code object).  q is [T, Hq, D] and k is [T, Hkv, D] with
 * element strides (stride_t, stride_h) and a unit stride along D; the two
 * tensors must not overlap each other and each must not overlap itself.
 * Both are checked from the pointers and strides (ROPE_QK_ERR_LAYOUT): q and
 * k pass when their byte ranges do not meet, or when they share one token
 * stride, each token's rows fit in it, and k's rows of a token lie in a gap
 * of q's (views into one fused QKV buffer); any other meeting of the two
 * ranges is refused.
 * Calls are asynchronous on `stream` (a hipStream_t; NULL = the legacy default
 * stream of the current device) and never synchronise with the host:
 * cu_seqlens is read only on the device.  cu_seqlens must be int32, with
 * 0 <= cu[0] <= cu[1] <= ... <= cu[nseq] <= T; this is NOT validated (that
 * would need a device read).  Whatever cu_seqlens holds, the kernel only
 * touches tokens t < T and heads < H, so bad metadata changes positions but
 * never causes an out-of-bounds access.  Calls are reentrant.
 *
 * Errors are returned, never thrown or aborted; a launch error is reported as
 * ROPE_QK_ERR_LAUNCH, and a device-side fault surfaces, as usual with HIP, at
 * the caller's next synchronisation.
 */
#ifndef ROPE_QK_H
#define ROPE_QK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* storage types of q and k (both tensors share one type) */
#define ROPE_QK_FP32 0
#define ROPE_QK_BF16 1
#define ROPE_QK_FP16 2  /* IEEE binary16, subnormals included; results past 65504 become inf */

/* status codes */
#define ROPE_QK_OK 0
#define ROPE_QK_ERR_NULL -1      /* a required pointer is NULL */
#define ROPE_QK_ERR_SHAPE -2     /* negative size, D odd or < 2 or > 512, T >= 2^31, too many heads */
#define ROPE_QK_ERR_DTYPE -3     /* dtype not ROPE_QK_FP32 / ROPE_QK_BF16 / ROPE_QK_FP16 */
#define ROPE_QK_ERR_ALIGN -4     /* base, stride*elem or (D/2)*elem not a multiple of 16 bytes */
#define ROPE_QK_ERR_THETA -5     /* theta not finite or <= 0 */
#define ROPE_QK_ERR_LAUNCH -6    /* the HIP launch itself failed */
#define ROPE_QK_ERR_LAYOUT -7    /* negative strides, a tensor whose rows overlap, or tensors that share memory */
#define ROPE_QK_ERR_OPTION -8    /* a field of rope_qk_options out of range (or eps, for the norm calls) */
#define ROPE_QK_ERR_WORKSPACE -9 /* workspace NULL or smaller than rope_qk_norm_bwd_workspace_bytes */
#define ROPE_QK_ERR_SCRATCH -10  /* rope_qk_norm_bwd_noalloc: the call needs more than its static scratch */

/* pairing of the rotated elements of a head (rope_qk_options.pairing) */
#define ROPE_QK_PAIR_HALF 0         /* element i with element i + r/2 ("rotate_half"; the default) */
#define ROPE_QK_PAIR_INTERLEAVED 1  /* element 2i with element 2i + 1 */

/* frequency rescaling (rope_qk_options.scaling) */
#define ROPE_QK_SCALING_NONE 0
#define ROPE_QK_SCALING_LLAMA3 1

/* how angles are formed (rope_qk_options.freq_precision) */
#define ROPE_QK_FREQ_FP64 0  /* float64 frequency times the position, in float64 (the default) */
#define ROPE_QK_FREQ_FP32 1  /* float32 frequency times the float32 position, in float32 */

/*
 * Forward rotation, in place, of q and k in ONE kernel launch.
 *
 *   q            device pointer to q[T, Hq, D] (may be NULL only if Hq == 0)
 *   k            device pointer to k[T, Hkv, D] (may be NULL only if Hkv == 0)
 *   cu_seqlens   device pointer to int32[nseq + 1], cumulative sequence offsets
 *   nseq         number of packed sequences (0: nothing is rotated)
 *   T            number of tokens along the first axis of q and k, < 2^31
 *   Hq, Hkv      heads of q and of k (grouped-query attention: Hkv <= Hq is usual)
 *   D            head dimension, even, 2 <= D <= 512
 *   q_stride_t, q_stride_h, k_stride_t, k_stride_h
 *                element strides of the token and head axes (contiguous:
 *                (Hq*D, D) and (Hkv*D, D)); must be >= 0
 *   theta        rotary base (e.g. 1e6 for Qwen2.5/Qwen3, 5e5 for Llama-3.1)
 *   dtype        ROPE_QK_FP32, ROPE_QK_BF16 or ROPE_QK_FP16
 *   stream       hipStream_t to launch on
 *
 * Alignment (16-byte vector path): q, k, every stride * elem_size and
 * (D/2) * elem_size must be multiples of 16 bytes.
 * Returns ROPE_QK_OK or a negative status; T == 0, nseq == 0 or no heads is a
 * no-op that launches nothing.
 */
int rope_qk_fwd(void* q, void* k, const int32_t* cu_seqlens, int64_t nseq, int64_t T,
                int64_t Hq, int64_t Hkv, int64_t D, int64_t q_stride_t, int64_t q_stride_h,
                int64_t k_stride_t, int64_t k_stride_h, double theta, int dtype, void* stream);

/*
 * Backward rotation, in place, of the incoming gradients dq and dk: the
 * transpose of the forward map, i.e. rotation by the negated angle.  Same
 * arguments, layout, ownership and errors as rope_qk_fwd.
 */
int rope_qk_bwd(void* dq, void* dk, const int32_t* cu_seqlens, int64_t nseq, int64_t T,
                int64_t Hq, int64_t Hkv, int64_t D, int64_t q_stride_t, int64_t q_stride_h,
                int64_t k_stride_t, int64_t k_stride_h, double theta, int dtype, void* stream);

/*
 * Options of rope_qk_fwd_opt / rope_qk_bwd_opt.  Zero-initialise the struct and
 * set what differs: an all-zero struct, or a NULL pointer, gives exactly
 * rope_qk_fwd / rope_qk_bwd.  None of these is on the pages except the model
 * names; each is the usual reading of the variant the named models use.
 *
 *   pos_offset   added to the position of every token of segment 0, i.e. of
 *                [cu_seqlens[0], cu_seqlens[1]): the global position of the
 *                first token of a shard that starts inside a sequence (token
 *                or context-parallel sharding of one long sequence); later
 *                segments still restart at 0.  0 <= pos_offset and
 *                pos_offset + T <= 2^31 - 1.
 *   rotary_dim   r: rotate elements [0, r) of each head and leave [r, D) not
 *                read and not written, with the frequencies of a head of size
 *                r, inv_freq[i] = theta^(-2i/r).  0 means D.  Even,
 *                2 <= r <= D; (r/2)*elem_size (ROPE_QK_PAIR_HALF) or
 *                r*elem_size (ROPE_QK_PAIR_INTERLEAVED) must be a multiple of
 *                16 bytes.
 *   pairing      ROPE_QK_PAIR_HALF: x1 = x[i], x2 = x[i + r/2];
 *                ROPE_QK_PAIR_INTERLEAVED: x1 = x[2i], x2 = x[2i + 1] (RoFormer's
 *                block-diagonal matrix taken literally); same rotation either way.
 *   scaling      ROPE_QK_SCALING_LLAMA3: the Llama 3.1 frequency rescaling (the
 *                pages name Llama 3.1 among the supported models).  With
 *                L = original_max_position and wavelength w = 2 pi / f of each
 *                inv_freq f: w < L / high_freq_factor keeps f; w > L /
 *                low_freq_factor gives f / factor; otherwise, with
 *                s = (L / w - low_freq_factor) / (high_freq_factor - low_freq_factor),
 *                (1 - s) f / factor + s f.  Needs factor > 0, L > 0 and
 *                high_freq_factor > low_freq_factor > 0 (Llama 3.1: 8, 8192, 4, 1).
 *   freq_precision
 *                ROPE_QK_FREQ_FP32: form each angle the way float32 frequency
 *                tables do, for models trained with them: the frequency (after
 *                any scaling) rounded to float32, the position converted to
 *                float32, their float32 product; each step rounds to nearest
 *                even.  At positions near 5e5 this moves angles by up to
 *                ~0.03 rad from the float64 angles.  cos, sin and the rotation
 *                stay float64, rounded once.  The pages fix neither convention.
 *   reserved     must be 0.
 */
typedef struct rope_qk_options {
  int64_t pos_offset;
  int64_t rotary_dim;
  int32_t pairing;
  int32_t scaling;
  double factor;
  double low_freq_factor;
  double high_freq_factor;
  double original_max_position;
  int32_t freq_precision;
  int32_t reserved;
} rope_qk_options;

/*
 * rope_qk_fwd / rope_qk_bwd with options (NULL: none).  Same arguments,
 * layout, ownership and errors, plus ROPE_QK_ERR_OPTION for an option out of
 * range.  The options are read during the call only.
 */
int rope_qk_fwd_opt(void* q, void* k, const int32_t* cu_seqlens, int64_t nseq, int64_t T,
                    int64_t Hq, int64_t Hkv, int64_t D, int64_t q_stride_t, int64_t q_stride_h,
                    int64_t k_stride_t, int64_t k_stride_h, double theta, int dtype,
                    const rope_qk_options* options, void* stream);
int rope_qk_bwd_opt(void* dq, void* dk, const int32_t* cu_seqlens, int64_t nseq, int64_t T,
                    int64_t Hq, int64_t Hkv, int64_t D, int64_t q_stride_t, int64_t q_stride_h,
                    int64_t k_stride_t, int64_t k_stride_h, double theta, int dtype,
                    const rope_qk_options* options, void* stream);

/*
 * Per-head RMSNorm followed by the rotation, forward, in ONE kernel launch.
 *
 * "Chronicals: A High-Performance Framework for LLM Fine-Tuning with 3.51x
 * Speedup over Unsloth", abstract, optimisation (1): RMSNorm and QK-RoPE are
 * among its fused kernels.  The pages give no formula; the reading is RMSNorm
 * (Zhang and Sennrich, 2019) of each head of q and of k on its own, placed
 * before the rotation as in Qwen3 (q_norm / k_norm), then the rotation of
 * rope_qk_fwd_opt.  For every token inside a sequence and every head, with
 * w = q_weight for q and k_weight for k:
 *
 *   r = 1 / sqrt(mean_j x_j^2 + eps),   n_j = x_j * r * w_j,   y = rope(n)
 *
 * evaluated in float64 and rounded once to the storage type.  Tokens outside
 * [cu_seqlens[0], cu_seqlens[nseq]) are copied unchanged from the input to a
 * separate output, and not written when the output is the input.
 *
 *   q, k           inputs [T, Hq, D], [T, Hkv, D] (device; NULL only without heads)
 *   q_out, k_out   outputs of the same shapes; each may be exactly its input
 *                  (same pointer and strides: in place) or must share no
 *                  memory with any other tensor of the call (checked like q
 *                  against k in rope_qk_fwd: ROPE_QK_ERR_LAYOUT)
 *   q_weight, k_weight
 *                  device float32 [D], 16-byte aligned (NULL only without heads)
 *   eps            finite, > 0 (else ROPE_QK_ERR_OPTION; Qwen3 uses 1e-6)
 *   strides        host int64[8], element strides: q (t, h), k (t, h),
 *                  q_out (t, h), k_out (t, h); unit stride along D
 *   options        as for rope_qk_fwd_opt, except that rotary_dim must be 0 or
 *                  D (the norm covers the whole head)
 *   D              D * element size must be 32, 64, ..., 1024 bytes (a whole
 *                  head is a power-of-two number of 16-byte chunks, at most
 *                  64); Hq <= 65535 and Hkv <= 65535; else ROPE_QK_ERR_SHAPE
 *
 * Other arguments, alignment, errors and stream semantics as rope_qk_fwd.
 * T == 0 or no heads is a no-op; so is nseq == 0 when both outputs are their
 * inputs.
 */
int rope_qk_norm_fwd(const void* q, const void* k, void* q_out, void* k_out, const float* q_weight,
                     const float* k_weight, double eps, const int32_t* cu_seqlens, int64_t nseq, int64_t T,
                     int64_t Hq, int64_t Hkv, int64_t D, const int64_t* strides, double theta, int dtype,
                     const rope_qk_options* options, void* stream);

/*
 * Bytes of device workspace rope_qk_norm_bwd needs for these sizes (>= 0), or
 * a negative status (ROPE_QK_ERR_DTYPE, ROPE_QK_ERR_SHAPE): 16 * D bytes for
 * each of the backward's workgroups, of which there are at most 3072 for
 * bf16 and fp16 and 4096 for fp32 (6 MiB at D = 128 in bf16; at most 24 MiB,
 * at D = 512 in bf16 or fp16).
 */
int64_t rope_qk_norm_bwd_workspace_bytes(int64_t T, int64_t Hq, int64_t Hkv, int64_t D, int dtype);

/*
 * Backward of rope_qk_norm_fwd.  Inputs: dq_out, dk_out (the gradients of the
 * forward's outputs) and q, k (the forward's INPUTS, which the caller keeps);
 * outputs: dq, dk (gradients of the inputs; each may be exactly its dq_out /
 * dk_out, i.e. in place, or must share no memory with any other tensor of
 * the call, ROPE_QK_ERR_LAYOUT otherwise) and dq_weight,
 * dk_weight (device float32 [D], 16-byte aligned, overwritten with the
 * gradient of q_weight / k_weight summed over every normalised head; NULL
 * only without heads).  With n, r as in the forward and dn = rope^T(dy) (the
 * rotation by -angle), g_j = dn_j w_j:
 *
 *   dx_j = r * (g_j - x_j * r^2 * (sum_k g_k x_k) / D),   dw_j = sum dn_j x_j r
 *
 * in float64, dx rounded once to the storage type, dw once to float32; the
 * sum over heads runs in a fixed order, so repeated calls give identical
 * bits.  Tokens outside every sequence pass dq_out / dk_out through to a
 * separate dq / dk (as the forward's identity there) and add nothing to the
 * weight gradients.
 *
 *   workspace, workspace_size
 *                  device memory of at least rope_qk_norm_bwd_workspace_bytes
 *                  bytes, 16-byte aligned, owned by the caller; its contents
 *                  on entry do not matter, and it must not be used by another
 *                  call until this one has completed on `stream`
 *                  (else ROPE_QK_ERR_WORKSPACE / ROPE_QK_ERR_ALIGN)
 *   strides        host int64[12], element strides: dq_out, dk_out, q, k, dq,
 *                  dk, each (t, h)
 *
 * Everything else as rope_qk_norm_fwd (same eps, weights, options, theta).
 * Two launches on `stream` (the rows, then the weight-gradient sums); with
 * T == 0 or no heads only the second, which writes zero weight gradients.
 */
int rope_qk_norm_bwd(const void* dq_out, const void* dk_out, const void* q, const void* k, void* dq, void* dk,
                     const float* q_weight, const float* k_weight, double eps, float* dq_weight, float* dk_weight,
                     void* workspace, int64_t workspace_size, const int32_t* cu_seqlens, int64_t nseq, int64_t T,
                     int64_t Hq, int64_t Hkv, int64_t D, const int64_t* strides, double theta, int dtype,
                     const rope_qk_options* options, void* stream);

/*
 * rope_qk_norm_bwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and errors as rope_qk_norm_bwd without the
 * workspace: the weight-gradient sums go to a static device array of 24 MiB
 * per GPU (the largest workspace any accepted shape needs, so every call the
 * workspace form accepts fits; ROPE_QK_ERR_SCRATCH would report one that
 * does not).  The array is part of the library's code object: each GPU the
 * library runs on holds its own copy until the process ends, and its address
 * is looked up once per device, on the first call for that device (the
 * device of `stream`, or the current device for the NULL stream).  The call
 * makes no hipMalloc, hipFree or other allocation.  Every call on one GPU
 * shares that GPU's array: calls that may overlap on one GPU (different
 * streams, host threads or processes sharing the code object) race and must
 * be ordered by the caller, e.g. by one stream.  Nothing in the array needs
 * to start at any value: each call writes every sum it reads.
 */
int rope_qk_norm_bwd_noalloc(const void* dq_out, const void* dk_out, const void* q, const void* k, void* dq,
                             void* dk, const float* q_weight, const float* k_weight, double eps, float* dq_weight,
                             float* dk_weight, const int32_t* cu_seqlens, int64_t nseq, int64_t T, int64_t Hq,
                             int64_t Hkv, int64_t D, const int64_t* strides, double theta, int dtype,
                             const rope_qk_options* options, void* stream);

/*
 * Per-token positions, for inspection: writes, for every t < T, pos(t) as
 * defined above, or -1 for tokens outside [cu_seqlens[0], cu_seqlens[nseq])
 * (no pos_offset).  Computed by the rotation kernels' own tile code (the
 * search of cu_seqlens for a tile's first token and the scan of the sequence
 * starts inside it), on tiles of 64 whole tokens.  pos_out: device
 * int32[T], caller-owned.  Asynchronous on `stream`.  Returns ROPE_QK_OK,
 * ROPE_QK_ERR_NULL, ROPE_QK_ERR_SHAPE or ROPE_QK_ERR_LAUNCH.
 */
int rope_qk_positions(const int32_t* cu_seqlens, int64_t nseq, int64_t T, int32_t* pos_out,
                      void* stream);

/*
 * Test hook: the positions each tile of a rotation call computes, in that
 * call's own tile decomposition and through the rotation kernels' own
 * geometry and position code (the auto-packing paragraph of the Unsloth
 * article: length metadata keeps packed samples apart).  The call is
 * described by cu_seqlens, nseq, T, Hq, Hkv, D, dtype and options as for
 * rope_qk_fwd_opt (q, k, their strides and theta play no part in it).
 *
 *   out       device int32[out_len], caller-owned, or NULL to ask only for
 *             the geometry; row i (row_len entries from out + i * row_len)
 *             receives tile i's first token, then the position of each token
 *             the tile touches, in order (-1: a token in no sequence); the
 *             rest of the row is not written
 *   ntiles, row_len
 *             host int64 outputs: the call's tile count, and 1 + the most
 *             tokens one tile touches (0 and 0 when the call launches nothing)
 *
 * Errors as rope_qk_fwd_opt (shape, dtype, options, ROPE_QK_ERR_NULL for a
 * NULL cu_seqlens, ntiles or row_len), and ROPE_QK_ERR_SHAPE when out_len <
 * ntiles * row_len.  One launch on `stream` when out is not NULL.
 */
int rope_qk_tile_positions(const int32_t* cu_seqlens, int64_t nseq, int64_t T, int64_t Hq, int64_t Hkv,
                           int64_t D, int dtype, const rope_qk_options* options, int32_t* out,
                           int64_t out_len, int64_t* ntiles, int64_t* row_len, void* stream);

/*
 * The same hook for the fused RMSNorm + rotation: backward == 0 runs the
 * forward's tiles (one per workgroup, each searching cu_seqlens), backward
 * != 0 the backward's runs of tiles with the sequence cursor each workgroup
 * carries from tile to tile.  Arguments, output rows and errors as
 * rope_qk_tile_positions, with the norm's shape limits; nseq == 0 is
 * allowed (every position -1).
 */
int rope_qk_norm_tile_positions(const int32_t* cu_seqlens, int64_t nseq, int64_t T, int64_t Hq, int64_t Hkv,
                                int64_t D, int dtype, const rope_qk_options* options, int backward,
                                int32_t* out, int64_t out_len, int64_t* ntiles, int64_t* row_len,
                                void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* rope_qk_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* ROPE_QK_H */
