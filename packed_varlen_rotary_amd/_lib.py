"""ctypes binding to librope_qk.so: argument marshalling only.

Every step of the rotation runs in the HIP kernels of the library; this module
turns torch tensors into pointers, element strides, a dtype code and the
current HIP stream, and raises on a non-zero status.  There is no fallback:
if the library is missing, every call raises.
"""

from __future__ import annotations

import copy
import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librope_qk.so")

ROPE_QK_FP32 = 0
ROPE_QK_BF16 = 1
ROPE_QK_FP16 = 2
ROPE_QK_PAIR_HALF = 0
ROPE_QK_PAIR_INTERLEAVED = 1
ROPE_QK_SCALING_NONE = 0
ROPE_QK_SCALING_LLAMA3 = 1
ROPE_QK_FREQ_FP64 = 0
ROPE_QK_FREQ_FP32 = 1

# names exported by include/rope_qk.h
EXPORTS = ("rope_qk_fwd", "rope_qk_bwd", "rope_qk_fwd_opt", "rope_qk_bwd_opt", "rope_qk_norm_fwd",
           "rope_qk_norm_bwd", "rope_qk_norm_bwd_workspace_bytes", "rope_qk_norm_bwd_noalloc", "rope_qk_positions",
           "rope_qk_tile_positions", "rope_qk_norm_tile_positions", "rope_qk_strerror",
           "rope_pack_bfd", "rope_pack_cu_seqlens", "rope_pack_cache_create", "rope_pack_cache_get",
           "rope_pack_cache_stats", "rope_pack_cache_destroy")


class RopeQKOptions(ctypes.Structure):
    """Mirror of ``rope_qk_options`` (include/rope_qk.h); all-zero means no options."""

    _fields_ = [
        ("pos_offset", ctypes.c_int64),
        ("rotary_dim", ctypes.c_int64),
        ("pairing", ctypes.c_int32),
        ("scaling", ctypes.c_int32),
        ("factor", ctypes.c_double),
        ("low_freq_factor", ctypes.c_double),
        ("high_freq_factor", ctypes.c_double),
        ("original_max_position", ctypes.c_double),
        ("freq_precision", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


def make_options(pos_offset: int = 0, rotary_dim: int = 0, interleaved: bool = False, llama3=None,
                 freq_fp32: bool = False) -> RopeQKOptions:
    """Options struct from keyword values; llama3 is None or a dict with factor,
    low_freq_factor, high_freq_factor and original_max_position; freq_fp32
    selects ROPE_QK_FREQ_FP32 angles."""
    o = RopeQKOptions()
    o.freq_precision = ROPE_QK_FREQ_FP32 if freq_fp32 else ROPE_QK_FREQ_FP64
    o.pos_offset = int(pos_offset)
    o.rotary_dim = int(rotary_dim or 0)
    o.pairing = ROPE_QK_PAIR_INTERLEAVED if interleaved else ROPE_QK_PAIR_HALF
    if llama3 is not None:
        o.scaling = ROPE_QK_SCALING_LLAMA3
        o.factor = float(llama3["factor"])
        o.low_freq_factor = float(llama3["low_freq_factor"])
        o.high_freq_factor = float(llama3["high_freq_factor"])
        o.original_max_position = float(llama3["original_max_position"])
    return o

class PackPlanStruct(ctypes.Structure):
    """Mirror of ``rope_pack_plan`` (include/rope_pack.h)."""

    _fields_ = [
        ("cu_seqlens_device", ctypes.c_void_p),
        ("cu_seqlens_host", ctypes.c_void_p),
        ("bin_of", ctypes.c_void_p),
        ("offset_of", ctypes.c_void_p),
        ("n", ctypes.c_int64),
        ("nseg", ctypes.c_int64),
        ("nbins", ctypes.c_int64),
        ("T", ctypes.c_int64),
        ("max_seqlen", ctypes.c_int32),
        ("hit", ctypes.c_int32),
    ]


_lock = threading.Lock()
_lib = None


class RopeQKError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"rope_qk status {status}: {msg}")
        self.status = status


def load():
    """Load the shared library (once).  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        # torch wheels bundle their own libamdhip64.so.7; importing torch first makes
        # the library bind to that same HIP runtime instance (streams and device
        # pointers from torch are only valid there) instead of /opt/rocm's copy.
        import torch  # noqa: F401

        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m packed_varlen_rotary_amd.build` "
                "(or __graft_entry__.build()); there is no fallback path"
            )
        lib = ctypes.CDLL(LIB_PATH)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        rot = [vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, i64, ctypes.c_double, ctypes.c_int, vp]
        for name in ("rope_qk_fwd", "rope_qk_bwd"):
            fn = getattr(lib, name)
            fn.argtypes = rot
            fn.restype = ctypes.c_int
        for name in ("rope_qk_fwd_opt", "rope_qk_bwd_opt"):
            fn = getattr(lib, name)
            fn.argtypes = rot[:-1] + [ctypes.POINTER(RopeQKOptions), vp]
            fn.restype = ctypes.c_int
        dbl = ctypes.c_double
        i64p = ctypes.POINTER(ctypes.c_int64)
        optp = ctypes.POINTER(RopeQKOptions)
        lib.rope_qk_norm_fwd.argtypes = [vp, vp, vp, vp, vp, vp, dbl, vp, i64, i64, i64, i64, i64, i64p, dbl,
                                         ctypes.c_int, optp, vp]
        lib.rope_qk_norm_fwd.restype = ctypes.c_int
        lib.rope_qk_norm_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, dbl, vp, vp, vp, i64, vp, i64, i64, i64,
                                         i64, i64, i64p, dbl, ctypes.c_int, optp, vp]
        lib.rope_qk_norm_bwd.restype = ctypes.c_int
        lib.rope_qk_norm_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, dbl, vp, vp, vp, i64, i64, i64,
                                                 i64, i64, i64p, dbl, ctypes.c_int, optp, vp]
        lib.rope_qk_norm_bwd_noalloc.restype = ctypes.c_int
        lib.rope_qk_norm_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64, ctypes.c_int]
        lib.rope_qk_norm_bwd_workspace_bytes.restype = ctypes.c_int64
        lib.rope_pack_bfd.argtypes = [vp, i64, i64, vp, vp, ctypes.POINTER(i64)]
        lib.rope_pack_bfd.restype = ctypes.c_int
        lib.rope_pack_cu_seqlens.argtypes = [vp, vp, vp, i64, i64, i64, vp, ctypes.POINTER(i64)]
        lib.rope_pack_cu_seqlens.restype = ctypes.c_int
        lib.rope_pack_cache_create.argtypes = [i64, ctypes.c_int, ctypes.POINTER(vp)]
        lib.rope_pack_cache_create.restype = ctypes.c_int
        lib.rope_pack_cache_get.argtypes = [vp, vp, i64, i64, vp, ctypes.POINTER(PackPlanStruct)]
        lib.rope_pack_cache_get.restype = ctypes.c_int
        lib.rope_pack_cache_stats.argtypes = [vp, ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(i64)]
        lib.rope_pack_cache_stats.restype = ctypes.c_int
        lib.rope_pack_cache_destroy.argtypes = [vp]
        lib.rope_pack_cache_destroy.restype = None
        lib.rope_qk_positions.argtypes = [vp, i64, i64, vp, vp]
        lib.rope_qk_positions.restype = ctypes.c_int
        lib.rope_qk_tile_positions.argtypes = [vp, i64, i64, i64, i64, i64, ctypes.c_int, optp, vp, i64,
                                               ctypes.POINTER(i64), ctypes.POINTER(i64), vp]
        lib.rope_qk_tile_positions.restype = ctypes.c_int
        lib.rope_qk_norm_tile_positions.argtypes = [vp, i64, i64, i64, i64, i64, ctypes.c_int, optp, ctypes.c_int,
                                                    vp, i64, ctypes.POINTER(i64), ctypes.POINTER(i64), vp]
        lib.rope_qk_norm_tile_positions.restype = ctypes.c_int
        lib.rope_qk_strerror.argtypes = [ctypes.c_int]
        lib.rope_qk_strerror.restype = ctypes.c_char_p
        _lib = lib
        return lib


def rope_qk_strerror(status: int) -> str:
    return load().rope_qk_strerror(int(status)).decode()


def _check(status: int):
    if status != 0:
        raise RopeQKError(status, rope_qk_strerror(status))


def _stream_ptr(device, stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    import torch

    if t.dtype == torch.bfloat16:
        return ROPE_QK_BF16
    if t.dtype == torch.float16:
        return ROPE_QK_FP16
    if t.dtype == torch.float32:
        return ROPE_QK_FP32
    raise TypeError(f"unsupported dtype {t.dtype}: expected torch.float32, torch.bfloat16 or torch.float16")


def _rotate(entry: str, q, k, cu_seqlens, theta: float, stream=None, options=None):
    import torch

    lib = load()
    for name, t in (("q", q), ("k", k)):
        if t.dim() != 3:
            raise ValueError(f"{name} must be [T, H, D], got shape {tuple(t.shape)}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.shape[2] > 1 and t.stride(2) != 1:
            raise ValueError(f"{name} must be unit-stride along D")
    if q.shape[0] != k.shape[0] or q.shape[2] != k.shape[2]:
        raise ValueError("q and k must share T and D")
    if q.dtype != k.dtype:
        raise TypeError("q and k must share one dtype")
    if q.device != k.device or cu_seqlens.device != q.device:
        raise ValueError("q, k and cu_seqlens must be on one device")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous 1-D int32 tensor")
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    args = [
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
        ctypes.c_void_p(cu_seqlens.data_ptr()), cu_seqlens.numel() - 1, T, Hq, Hkv, D,
        q.stride(0), q.stride(1), k.stride(0), k.stride(1),
        float(theta), _dtype_code(q),
    ]
    if entry.endswith("_opt"):
        args.append(ctypes.byref(options) if options is not None else None)
    with torch.cuda.device(q.device):
        status = getattr(lib, entry)(*args, _stream_ptr(q.device, stream))
    _check(status)


def _options_or_none(pos_offset, rotary_dim, interleaved, llama3, freq_fp32):
    if not pos_offset and not rotary_dim and not interleaved and llama3 is None and not freq_fp32:
        return None
    return make_options(pos_offset, rotary_dim, interleaved, llama3, freq_fp32)


def rope_qk_fwd(q, k, cu_seqlens, theta: float, stream=None, *, pos_offset: int = 0, rotary_dim: int = 0,
                interleaved: bool = False, llama3=None, freq_fp32: bool = False):
    """Rotate q [T, Hq, D] and k [T, Hkv, D] in place (one kernel launch).

    cu_seqlens: int32 [nseq + 1] device tensor of packed-sequence offsets.
    stream: a torch.cuda.Stream (default: the current stream of q's device).
    Keyword options (see rope_qk_options in include/rope_qk.h): pos_offset for
    segment 0, rotary_dim, interleaved pairing, llama3 frequency rescaling,
    freq_fp32 for float32-convention angles.
    """
    opts = _options_or_none(pos_offset, rotary_dim, interleaved, llama3, freq_fp32)
    if opts is None:
        _rotate("rope_qk_fwd", q, k, cu_seqlens, theta, stream)
    else:
        _rotate("rope_qk_fwd_opt", q, k, cu_seqlens, theta, stream, opts)


def rope_qk_bwd(dq, dk, cu_seqlens, theta: float, stream=None, *, pos_offset: int = 0, rotary_dim: int = 0,
                interleaved: bool = False, llama3=None, freq_fp32: bool = False):
    """Backward of rope_qk_fwd, in place on the incoming gradients dq and dk."""
    opts = _options_or_none(pos_offset, rotary_dim, interleaved, llama3, freq_fp32)
    if opts is None:
        _rotate("rope_qk_bwd", dq, dk, cu_seqlens, theta, stream)
    else:
        _rotate("rope_qk_bwd_opt", dq, dk, cu_seqlens, theta, stream, opts)


def rope_qk_fwd_opt(q, k, cu_seqlens, theta: float, options=None, stream=None):
    """rope_qk_fwd with a RopeQKOptions struct (None: no options)."""
    _rotate("rope_qk_fwd_opt", q, k, cu_seqlens, theta, stream, options)


def rope_qk_bwd_opt(dq, dk, cu_seqlens, theta: float, options=None, stream=None):
    """rope_qk_bwd with a RopeQKOptions struct (None: no options)."""
    _rotate("rope_qk_bwd_opt", dq, dk, cu_seqlens, theta, stream, options)


def rope_qk_positions(cu_seqlens, T: int, out=None, stream=None):
    """Per-token positions (int32 [T], -1 outside every sequence), computed by
    the rotation kernels' own tile code on tiles of 64 whole tokens."""
    import torch

    lib = load()
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous 1-D int32 tensor")
    if out is None:
        out = torch.empty(T, dtype=torch.int32, device=cu_seqlens.device)
    if out.dtype != torch.int32 or out.numel() != T or not out.is_contiguous():
        raise ValueError("out must be a contiguous int32 tensor of T elements")
    with torch.cuda.device(cu_seqlens.device):
        status = lib.rope_qk_positions(
            ctypes.c_void_p(cu_seqlens.data_ptr()), cu_seqlens.numel() - 1, int(T),
            ctypes.c_void_p(out.data_ptr()), _stream_ptr(cu_seqlens.device, stream),
        )
    _check(status)
    return out


TILE_ROW_UNWRITTEN = -(2 ** 31)  # what the hooks' output rows hold where a tile wrote nothing


def _tile_positions(entry, cu_seqlens, T, Hq, Hkv, D, dtype_code, options, stream, extra=()):
    import torch

    lib = load()
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous 1-D int32 tensor")
    nt, rl = ctypes.c_int64(0), ctypes.c_int64(0)
    opts = ctypes.byref(options) if options is not None else None
    head = [ctypes.c_void_p(cu_seqlens.data_ptr()), cu_seqlens.numel() - 1, int(T), int(Hq), int(Hkv), int(D),
            int(dtype_code), opts, *extra]
    _check(getattr(lib, entry)(*head, None, 0, ctypes.byref(nt), ctypes.byref(rl), None))
    out = torch.full((max(nt.value, 0), max(rl.value, 0)), TILE_ROW_UNWRITTEN, dtype=torch.int32,
                     device=cu_seqlens.device)
    if out.numel():
        with torch.cuda.device(cu_seqlens.device):
            _check(getattr(lib, entry)(*head, ctypes.c_void_p(out.data_ptr()), out.numel(), ctypes.byref(nt),
                                       ctypes.byref(rl), _stream_ptr(cu_seqlens.device, stream)))
    return out


def rope_qk_tile_positions(cu_seqlens, T: int, Hq: int, Hkv: int, D: int, dtype_code: int, options=None,
                           stream=None):
    """Test hook: [ntiles, row_len] int32 device tensor; row i = tile i's first
    token, then the positions of the tokens it touches (TILE_ROW_UNWRITTEN
    after them), computed by the rotation kernels' own tile code for a call
    of these sizes and options (a RopeQKOptions or None)."""
    return _tile_positions("rope_qk_tile_positions", cu_seqlens, T, Hq, Hkv, D, dtype_code, options, stream)


def rope_qk_norm_tile_positions(cu_seqlens, T: int, Hq: int, Hkv: int, D: int, dtype_code: int, backward: bool,
                                options=None, stream=None):
    """The same hook for the fused RMSNorm + rotation's forward or backward tiles."""
    return _tile_positions("rope_qk_norm_tile_positions", cu_seqlens, T, Hq, Hkv, D, dtype_code, options, stream,
                           extra=(1 if backward else 0,))


# ---------------------------------------------------------------------------
# per-head RMSNorm + rotation
# ---------------------------------------------------------------------------

def _check_rows(name, t, ref):
    if t.dim() != 3 or not t.is_cuda or (t.shape[2] > 1 and t.stride(2) != 1):
        raise ValueError(f"{name} must be a [T, H, D] GPU tensor, unit-stride along D")
    if t.dtype != ref.dtype or t.device != ref.device or t.shape[0] != ref.shape[0] or t.shape[2] != ref.shape[2]:
        raise ValueError(f"{name} must match q's dtype, device, T and D")


def _check_weight(name, w, D, device):
    import torch

    if w is None:
        return None
    if w.dtype != torch.float32 or w.dim() != 1 or w.numel() != D or not w.is_contiguous() or w.device != device:
        raise ValueError(f"{name} must be a contiguous float32 [D] tensor on q's device")
    return ctypes.c_void_p(w.data_ptr())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _strides(*ts):
    vals = []
    for t in ts:
        vals += [t.stride(0), t.stride(1)]
    return (ctypes.c_int64 * len(vals))(*vals)


def rope_qk_norm_fwd(q, k, q_weight, k_weight, eps: float, cu_seqlens, theta: float, q_out=None, k_out=None,
                     stream=None, *, pos_offset: int = 0, interleaved: bool = False, llama3=None,
                     freq_fp32: bool = False):
    """Per-head RMSNorm of q [T, Hq, D] and k [T, Hkv, D] followed by the rotation, one launch.

    q_weight, k_weight: float32 [D].  q_out / k_out: output tensors of the
    same shapes (default: q and k themselves, i.e. in place).  Returns
    (q_out, k_out).  Options as rope_qk_fwd (no rotary_dim: the norm covers
    the whole head).
    """
    import torch

    lib = load()
    q_out = q if q_out is None else q_out
    k_out = k if k_out is None else k_out
    for name, t in (("k", k), ("q_out", q_out), ("k_out", k_out)):
        _check_rows(name, t, q)
    _check_rows("q", q, q)
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous 1-D int32 tensor")
    T, Hq, D = q.shape
    opts = make_options(pos_offset, 0, interleaved, llama3, freq_fp32)
    with torch.cuda.device(q.device):
        status = lib.rope_qk_norm_fwd(
            _ptr(q), _ptr(k), _ptr(q_out), _ptr(k_out),
            _check_weight("q_weight", q_weight, D, q.device), _check_weight("k_weight", k_weight, D, q.device),
            float(eps), _ptr(cu_seqlens), cu_seqlens.numel() - 1, T, Hq, k.shape[1], D,
            _strides(q, k, q_out, k_out), float(theta), _dtype_code(q), ctypes.byref(opts),
            _stream_ptr(q.device, stream))
    _check(status)
    return q_out, k_out


def rope_qk_norm_bwd_workspace_bytes(T: int, Hq: int, Hkv: int, D: int, dtype_code: int) -> int:
    n = load().rope_qk_norm_bwd_workspace_bytes(int(T), int(Hq), int(Hkv), int(D), int(dtype_code))
    if n < 0:
        _check(int(n))
    return int(n)


def rope_qk_norm_bwd_noalloc(dq_out, dk_out, q, k, q_weight, k_weight, eps: float, cu_seqlens, theta: float,
                             dq, dk, dq_weight, dk_weight, stream=None, *, pos_offset: int = 0,
                             interleaved: bool = False, llama3=None, freq_fp32: bool = False):
    """rope_qk_norm_bwd without a workspace: the library's static per-GPU
    scratch holds the weight-gradient sums, so the call allocates nothing
    (every output is the caller's; pass dq is dq_out for in place).  Calls
    that may overlap on one GPU share that scratch and must be ordered."""
    import torch

    lib = load()
    for name, t in (("dk_out", dk_out), ("k", k), ("dq", dq), ("dk", dk), ("dq_out", dq_out)):
        _check_rows(name, t, q)
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous 1-D int32 tensor")
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    opts = make_options(pos_offset, 0, interleaved, llama3, freq_fp32)
    with torch.cuda.device(q.device):
        status = lib.rope_qk_norm_bwd_noalloc(
            _ptr(dq_out), _ptr(dk_out), _ptr(q), _ptr(k), _ptr(dq), _ptr(dk),
            _check_weight("q_weight", q_weight, D, q.device), _check_weight("k_weight", k_weight, D, q.device),
            float(eps), _check_weight("dq_weight", dq_weight, D, q.device),
            _check_weight("dk_weight", dk_weight, D, q.device), _ptr(cu_seqlens), cu_seqlens.numel() - 1, T, Hq,
            Hkv, D, _strides(dq_out, dk_out, q, k, dq, dk), float(theta), _dtype_code(q), ctypes.byref(opts),
            _stream_ptr(q.device, stream))
    _check(status)
    return dq, dk, dq_weight, dk_weight


def rope_qk_norm_bwd(dq_out, dk_out, q, k, q_weight, k_weight, eps: float, cu_seqlens, theta: float, dq=None,
                     dk=None, dq_weight=None, dk_weight=None, workspace=None, stream=None, *, pos_offset: int = 0,
                     interleaved: bool = False, llama3=None, freq_fp32: bool = False):
    """Backward of rope_qk_norm_fwd: returns (dq, dk, dq_weight, dk_weight).

    q, k are the forward's INPUTS.  dq / dk default to dq_out / dk_out (in
    place); dq_weight / dk_weight default to new float32 [D] tensors; the
    workspace (uint8 device tensor) is allocated when not given.
    """
    import torch

    lib = load()
    dq = dq_out if dq is None else dq
    dk = dk_out if dk is None else dk
    for name, t in (("dk_out", dk_out), ("k", k), ("dq", dq), ("dk", dk), ("dq_out", dq_out)):
        _check_rows(name, t, q)
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous 1-D int32 tensor")
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    code = _dtype_code(q)
    if dq_weight is None:
        dq_weight = torch.empty(D, dtype=torch.float32, device=q.device)
    if dk_weight is None:
        dk_weight = torch.empty(D, dtype=torch.float32, device=q.device)
    need = rope_qk_norm_bwd_workspace_bytes(T, Hq, Hkv, D, code)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    opts = make_options(pos_offset, 0, interleaved, llama3, freq_fp32)
    with torch.cuda.device(q.device):
        status = lib.rope_qk_norm_bwd(
            _ptr(dq_out), _ptr(dk_out), _ptr(q), _ptr(k), _ptr(dq), _ptr(dk),
            _check_weight("q_weight", q_weight, D, q.device), _check_weight("k_weight", k_weight, D, q.device),
            float(eps), _check_weight("dq_weight", dq_weight, D, q.device),
            _check_weight("dk_weight", dk_weight, D, q.device), _ptr(workspace), workspace.numel(),
            _ptr(cu_seqlens), cu_seqlens.numel() - 1, T, Hq, Hkv, D, _strides(dq_out, dk_out, q, k, dq, dk),
            float(theta), code, ctypes.byref(opts), _stream_ptr(q.device, stream))
    _check(status)
    return dq, dk, dq_weight, dk_weight


# ---------------------------------------------------------------------------
# Best-Fit-Decreasing packing and the packed-metadata cache (include/rope_pack.h)
# ---------------------------------------------------------------------------

def _lengths_i32(lengths):
    import numpy as np

    a = np.ascontiguousarray(np.asarray(lengths, dtype=np.int64))
    if a.ndim != 1:
        raise ValueError("lengths must be 1-D")
    if a.size and (a.min() < -2 ** 31 or a.max() >= 2 ** 31):
        raise ValueError("lengths must fit in int32")
    return np.ascontiguousarray(a.astype(np.int32))


def _host_ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a.size else None


def pack_bfd(lengths, capacity: int):
    """Best-Fit-Decreasing packing (native): (bin_of, offset_of, nbins), int32 numpy arrays."""
    import numpy as np

    lib = load()
    L = _lengths_i32(lengths)
    bin_of = np.empty(L.size, dtype=np.int32)
    offset_of = np.empty(L.size, dtype=np.int32)
    nbins = ctypes.c_int64(0)
    _check(lib.rope_pack_bfd(_host_ptr(L), L.size, int(capacity), _host_ptr(bin_of), _host_ptr(offset_of),
                             ctypes.byref(nbins)))
    return bin_of, offset_of, int(nbins.value)


def packed_cu_seqlens(lengths, bin_of, offset_of, nbins: int, capacity: int):
    """cu_seqlens (int32 numpy) of the packed batch over nbins * capacity tokens."""
    import numpy as np

    lib = load()
    L = _lengths_i32(lengths)
    b = np.ascontiguousarray(np.asarray(bin_of, dtype=np.int32))
    o = np.ascontiguousarray(np.asarray(offset_of, dtype=np.int32))
    if b.shape != L.shape or o.shape != L.shape:
        raise ValueError("bin_of and offset_of must match lengths")
    cu = np.empty(L.size + int(nbins) + 1, dtype=np.int32)
    nseg = ctypes.c_int64(0)
    _check(lib.rope_pack_cu_seqlens(_host_ptr(L), _host_ptr(b), _host_ptr(o), L.size, int(nbins), int(capacity),
                                    _host_ptr(cu), ctypes.byref(nseg)))
    return cu[: nseg.value + 1].copy()


class _DeviceInt32:
    """A device int32 vector owned by the native cache, shown to torch through
    the CUDA array interface (zero copy) so that it can be copied once."""

    def __init__(self, ptr: int, n: int):
        self.__cuda_array_interface__ = {"shape": (n,), "typestr": "<i4", "data": (ptr, False), "version": 2,
                                         "strides": None}


class PackPlan:
    """One packed batch from PackCache.get.  cu_seqlens: device int32 tensor
    owned by torch (None for a host-only cache), copied once from the cache's
    upload when the batch is first packed, on the caller's stream, and shared
    by every later hit; it stays valid while referenced, whatever the cache
    evicts or closes.  The rest are host copies."""

    def __init__(self, s: PackPlanStruct, device, stream=None):
        import numpy as np

        nseg, n = int(s.nseg), int(s.n)
        host = (ctypes.c_int32 * (nseg + 1)).from_address(s.cu_seqlens_host)
        self.cu_seqlens_host = np.frombuffer(host, dtype=np.int32).copy()
        self.bin_of = np.frombuffer((ctypes.c_int32 * n).from_address(s.bin_of), dtype=np.int32).copy() if n else \
            np.empty(0, dtype=np.int32)
        self.offset_of = np.frombuffer((ctypes.c_int32 * n).from_address(s.offset_of), dtype=np.int32).copy() \
            if n else np.empty(0, dtype=np.int32)
        self.n, self.nseg, self.nbins, self.T = n, nseg, int(s.nbins), int(s.T)
        self.max_seqlen = int(s.max_seqlen)
        self.hit = bool(s.hit)
        self.cu_seqlens_ptr = int(s.cu_seqlens_device or 0)  # the cache's own buffer (freed on eviction)
        self.cu_seqlens = None
        if self.cu_seqlens_ptr:
            import torch

            # a torch-owned copy, ordered after the cache's upload on the same
            # stream; evicting the plan frees the cache's buffer only after
            # the device is idle (hipFree), so the copy has been made by then
            view = torch.as_tensor(_DeviceInt32(self.cu_seqlens_ptr, nseg + 1), device=device)
            with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream(device)):
                self.cu_seqlens = view.clone()


class PackCache:
    """The native packed-metadata cache (rope_pack_cache_*): pack a batch once,
    upload its cu_seqlens once, answer every later lookup on the host.

    device: a torch device (default: the current CUDA device), or None with
    host_only=True for a cache without device memory.
    """

    def __init__(self, max_entries: int = 64, device=None, host_only: bool = False):
        lib = load()
        self._lib = lib
        self._ptr = None
        self._max_entries = int(max_entries)
        if host_only:
            self.device, code = None, -1
        else:
            import torch

            self.device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
            code = self.device.index if self.device.index is not None else torch.cuda.current_device()
        ptr = ctypes.c_void_p()
        _check(lib.rope_pack_cache_create(int(max_entries), int(code), ctypes.byref(ptr)))
        self._ptr = ptr
        # Python views of the plans held, by their host cu_seqlens buffer: a hit
        # returns the view made on that plan's miss (the native cache only
        # answers a hit for a plan that this wrapper saw being created)
        self._views = {}

    def get(self, lengths, capacity: int, stream=None) -> PackPlan:
        if self._ptr is None:
            raise RuntimeError("the cache is closed")
        L = _lengths_i32(lengths)
        s = PackPlanStruct()
        sp = _stream_ptr(self.device, stream) if self.device is not None else None
        _check(self._lib.rope_pack_cache_get(self._ptr, _host_ptr(L), L.size, int(capacity), sp, ctypes.byref(s)))
        key = int(s.cu_seqlens_host or 0)
        view = self._views.get(key) if s.hit else None
        if view is None:
            view = PackPlan(s, self.device, stream)
            self._views[key] = view
            if len(self._views) > 4 * self._max_entries:  # drop views of plans long evicted
                self._views = {key: view}
        out = copy.copy(view)  # shares the arrays and the device view; its own hit flag
        out.hit = bool(s.hit)
        return out

    def stats(self):
        """(hits, misses, entries)."""
        h, m, e = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int64(0)
        _check(self._lib.rope_pack_cache_stats(self._ptr, ctypes.byref(h), ctypes.byref(m), ctypes.byref(e)))
        return int(h.value), int(m.value), int(e.value)

    def close(self):
        if self._ptr is not None:
            self._lib.rope_pack_cache_destroy(self._ptr)
            self._ptr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
