"""The plain in-place stream the benchmark measures against (libstream_ceiling.so).

CPU: the library exports what include/stream_ceiling.h declares and rejects
bad arguments before any HIP call.  GPU: every variant the benchmark times
leaves the buffer unchanged, at sizes that end inside a tile.
"""

import ctypes
import os
import re
import subprocess

import pytest

from packed_varlen_rotary_amd import stream_ceiling as SC

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "stream_ceiling.h")


def consts():
    return {m.group(1): int(m.group(2))
            for m in re.finditer(r"#define\s+(STREAM_CEILING_\w+)\s+(-?\d+)", open(HEADER).read())}


def test_exports_match_header():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    declared = set(re.findall(r"\b(stream_ceiling_\w+)\s*\(", text))
    out = subprocess.run(["nm", "-D", "--defined-only", SC.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    assert set(re.findall(r"\sT\s(stream_ceiling_\w+)$", out, flags=re.M)) == declared == {"stream_ceiling_launch"}


def test_argument_errors_before_any_launch():
    C = consts()
    f = SC.load().stream_ceiling_launch
    buf = ctypes.c_void_p(0x10000)  # never dereferenced: every call below is rejected or a no-op
    assert f(buf, 24, 4, 0, 1, 0, None) == C["STREAM_CEILING_ERR_SIZE"]
    assert f(buf, -16, 4, 0, 1, 0, None) == C["STREAM_CEILING_ERR_SIZE"]
    assert f(buf, (1 << 35) + 16, 4, 0, 1, 0, None) == C["STREAM_CEILING_ERR_SIZE"]
    assert f(buf, 1024, 3, 0, 1, 0, None) == C["STREAM_CEILING_ERR_SHAPE"]
    assert f(buf, 1024, 4, -1, 1, 0, None) == C["STREAM_CEILING_ERR_SHAPE"]
    assert f(buf, 1024, 4, 0, 1, 33, None) == C["STREAM_CEILING_ERR_SHAPE"]
    assert f(buf, 1024, 4, 0, 1, -1, None) == C["STREAM_CEILING_ERR_SHAPE"]
    assert f(None, 1024, 4, 0, 1, 0, None) == C["STREAM_CEILING_ERR_NULL"]
    assert f(ctypes.c_void_p(0x10008), 1024, 4, 0, 1, 0, None) == C["STREAM_CEILING_ERR_ALIGN"]
    assert f(None, 0, 4, 0, 1, 0, None) == C["STREAM_CEILING_OK"]


@pytest.mark.gpu
def test_every_bench_variant_leaves_the_buffer_unchanged():
    import torch

    import bench

    for nbytes in (16, 4096 * 16 + 48, (1 << 22) + 16 * 777):
        g = torch.Generator(device="cuda")
        g.manual_seed(nbytes)
        buf = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
        ref = buf.clone()
        for tpl, groups, nt, cap in bench.CEILING_VARIANTS:
            SC.stream_ceiling_launch(buf, tpl, groups, bool(nt), cap)
        torch.cuda.synchronize()
        assert torch.equal(buf, ref), nbytes
