"""Build librope_qk.so (the HIP kernels and their C ABI) and libstream_ceiling.so
(the plain stream the bench measures against) in-tree for gfx950.

    python -m packed_varlen_rotary_amd.build

Always recompiles.  hipcc cross-compiles for gfx950 without a GPU present.
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", n) for n in ("rope_qk.hip", "rope_qk_norm.hip", "rope_pack.cpp")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "librope_qk.so")
# the plain in-place stream that the bench measures the rotation against
# (include/stream_ceiling.h): a measurement aid in a library of its own
CEILING_SRCS = [os.path.join(PKG, "csrc", "stream_ceiling.hip")]
CEILING_LIB = os.path.join(PKG, "libstream_ceiling.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the SLP vectorizer packs the per-element rounding-tie flags of a chunk
    # into a bit vector and reduces it with 16-bit vector ops; without it they
    # stay lane masks OR-ed on the scalar unit (8% fewer vector instructions
    # in the default workload's kernel, which runs ~5% faster)
    "-fno-slp-vectorize",
]


def build(verbose: bool = False, extra_flags=(), out: str = LIB, srcs=None) -> str:
    cmd = [HIPCC, *FLAGS, *extra_flags, "-I", INCLUDE, "-o", out + ".tmp", *(SRCS if srcs is None else srcs)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(out + ".tmp", out)
    return out


def build_all(verbose: bool = False) -> list:
    """Both libraries: the rotation library and the stream-ceiling probe."""
    return [build(verbose), build(verbose, out=CEILING_LIB, srcs=CEILING_SRCS)]


if __name__ == "__main__":
    print("\n".join(build_all(verbose=True)))
    sys.exit(0)
