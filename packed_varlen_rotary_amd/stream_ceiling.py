"""ctypes binding to libstream_ceiling.so (include/stream_ceiling.h): the plain
in-place 16-byte stream that the benchmark measures the rotation against.
A measurement aid, not part of the rotation path; argument marshalling only."""

from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libstream_ceiling.so")

_lock = threading.Lock()
_lib = None


def load():
    """Load the library (once); raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            import torch  # noqa: F401  (bind to torch's HIP runtime, as the rotation library does)

            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m packed_varlen_rotary_amd.build`")
            lib = ctypes.CDLL(LIB_PATH)
            lib.stream_ceiling_launch.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int64,
                                                  ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
            lib.stream_ceiling_launch.restype = ctypes.c_int
            _lib = lib
        return _lib


def stream_ceiling_launch(buf, chunks_per_lane: int = 4, groups: int = 0, nontemporal: bool = True,
                          groups_per_cu: int = 0, stream=None):
    """One in-place pass over the bytes of the contiguous GPU tensor buf (left unchanged)."""
    import torch

    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    s = torch.cuda.current_stream(buf.device) if stream is None else stream
    with torch.cuda.device(buf.device):
        status = load().stream_ceiling_launch(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                                              int(chunks_per_lane), int(groups), 1 if nontemporal else 0,
                                              int(groups_per_cu), ctypes.c_void_p(s.cuda_stream))
    if status != 0:
        raise RuntimeError(f"stream_ceiling_launch status {status}")
