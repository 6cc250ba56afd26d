"""Fused in-place QK rotary position embedding over packed variable-length
batches, for AMD Instinct MI355X (gfx950).

The work runs in the HIP kernels of ``librope_qk.so`` (C ABI in
``include/rope_qk.h``); this package is a thin ctypes binding with the same
entry-point names.  PyTorch is used only for device memory and streams.
"""

from ._lib import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    ROPE_QK_BF16,
    ROPE_QK_FP16,
    ROPE_QK_FREQ_FP32,
    ROPE_QK_FREQ_FP64,
    ROPE_QK_FP32,
    ROPE_QK_PAIR_HALF,
    ROPE_QK_PAIR_INTERLEAVED,
    ROPE_QK_SCALING_LLAMA3,
    ROPE_QK_SCALING_NONE,
    RopeQKError,
    RopeQKOptions,
    PackCache,
    PackPlan,
    load,
    make_options,
    pack_bfd,
    packed_cu_seqlens,
    rope_qk_bwd,
    rope_qk_bwd_opt,
    rope_qk_fwd,
    rope_qk_fwd_opt,
    rope_qk_norm_bwd,
    rope_qk_norm_bwd_noalloc,
    rope_qk_norm_bwd_workspace_bytes,
    rope_qk_norm_fwd,
    rope_qk_positions,
    rope_qk_strerror,
)

__all__ = [
    "rope_qk_fwd",
    "rope_qk_bwd",
    "rope_qk_fwd_opt",
    "rope_qk_bwd_opt",
    "rope_qk_norm_fwd",
    "rope_qk_norm_bwd",
    "rope_qk_norm_bwd_noalloc",
    "rope_qk_norm_bwd_workspace_bytes",
    "RopeQKOptions",
    "make_options",
    "rope_qk_positions",
    "rope_qk_strerror",
    "pack_bfd",
    "packed_cu_seqlens",
    "PackCache",
    "PackPlan",
    "RopeQKError",
    "load",
    "LIB_PATH",
    "EXPORTS",
    "ROPE_QK_FP32",
    "ROPE_QK_BF16",
    "ROPE_QK_FP16",
]
