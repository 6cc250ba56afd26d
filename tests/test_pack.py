"""The native Best-Fit-Decreasing packer and the packed-metadata cache (CPU):
bit-exact against the oracle, argument checks, and the cache's bookkeeping in
host-only mode (no device memory)."""

import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
import packed_varlen_rotary_amd as P
from tests import pack_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ERR_NULL, ERR_SHAPE = -1, -2


def check_against_oracle(lengths, cap):
    b, o, nb = P.pack_bfd(lengths, cap)
    rb, ro, rnb = oracle.bfd_pack(lengths, cap)
    assert nb == rnb and np.array_equal(b, rb) and np.array_equal(o, ro), (cap, list(lengths)[:20])
    cu = P.packed_cu_seqlens(lengths, b, o, nb, cap)
    assert np.array_equal(cu, oracle.packed_cu_seqlens(lengths, rb, ro, rnb, cap))
    return b, o, nb, cu


@pytest.mark.parametrize("case", range(len(pack_pins.HAND_CASES)))
def test_hand_cases(case):
    cap, lengths, b, o, nb, cu = pack_pins.HAND_CASES[case]
    gb, go, gnb, gcu = check_against_oracle(lengths, cap)
    assert list(gb) == b and list(go) == o and gnb == nb and list(gcu) == cu


def test_random_batches_match_the_oracle():
    rng = np.random.default_rng(5)
    for trial in range(80):
        cap = int(rng.integers(1, 5000))
        n = int(rng.integers(0, 400))
        lengths = rng.integers(0, cap + 1, size=n)
        if trial % 4 == 0:
            lengths = rng.integers(0, max(2, cap // 8), size=n)  # many items per bin
        if trial % 7 == 0:
            lengths = np.full(n, int(rng.integers(0, cap + 1)))  # all equal: ties everywhere
        check_against_oracle(lengths, cap)


def test_short_long_mixture_at_scale():
    """3,000 lengths of the 80% short / 20% long mixture into 16,384-token bins."""
    rng = np.random.default_rng(11)
    n = 3000
    short = rng.integers(32, 513, size=n)
    long_ = rng.integers(2048, 8193, size=n)
    lengths = np.where(rng.random(n) < 0.8, short, long_)
    b, o, nb, cu = check_against_oracle(lengths, 16384)
    assert nb * 16384 < 1.05 * lengths.sum() + 16384  # little padding


def test_argument_checks():
    lib = P.load()
    L = np.array([3, 4], dtype=np.int32)
    out = np.zeros(2, dtype=np.int32)
    nb = ctypes.c_int64()
    f = lambda lengths=L, n=2, cap=10, bo=out, oo=out, nbp=ctypes.byref(nb): lib.rope_pack_bfd(  # noqa: E731
        ctypes.c_void_p(lengths.ctypes.data) if lengths is not None else None, n, cap,
        ctypes.c_void_p(bo.ctypes.data) if bo is not None else None,
        ctypes.c_void_p(oo.ctypes.data) if oo is not None else None, nbp)
    assert f() == 0
    assert f(cap=3) == ERR_SHAPE  # a length above capacity
    assert f(lengths=np.array([3, -1], dtype=np.int32)) == ERR_SHAPE
    assert f(cap=0) == ERR_SHAPE
    assert f(n=-1) == ERR_SHAPE
    assert f(cap=2 ** 31) == ERR_SHAPE
    assert f(lengths=None) == ERR_NULL
    assert f(bo=None) == ERR_NULL
    assert f(nbp=None) == ERR_NULL
    assert f(lengths=None, n=0) == 0  # nothing to pack
    with pytest.raises(P.RopeQKError):
        P.pack_bfd([5, 11], 10)
    # a placement whose bin does not start at token 0
    with pytest.raises(P.RopeQKError):
        P.packed_cu_seqlens([3], [0], [1], 1, 10)
    # more tokens than int32 cu_seqlens can hold
    with pytest.raises(P.RopeQKError):
        P.packed_cu_seqlens([2 ** 30, 2 ** 30, 2 ** 30], [0, 1, 2], [0, 0, 0], 3, 2 ** 30)


def test_plan_struct_layout_matches_header(tmp_path):
    src = tmp_path / "layout.c"
    names = [n for n, _ in P._lib.PackPlanStruct._fields_]
    body = "".join(f'  printf("%zu\\n", offsetof(rope_pack_plan, {n}));\n' for n in names)
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "rope_pack.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(rope_pack_plan));\n' + body + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    S = P._lib.PackPlanStruct
    assert got == [ctypes.sizeof(S)] + [getattr(S, n).offset for n in names]


def test_host_only_cache_hits_misses_and_eviction():
    cache = P.PackCache(max_entries=2, host_only=True)
    a = [300, 5000, 12, 16000, 700]
    b = [1, 2, 3]
    c = [9000, 9000]
    p1 = cache.get(a, 16384)
    assert not p1.hit and p1.cu_seqlens is None
    rb, ro, rnb = oracle.bfd_pack(a, 16384)
    assert np.array_equal(p1.bin_of, rb) and np.array_equal(p1.offset_of, ro) and p1.nbins == rnb
    assert np.array_equal(p1.cu_seqlens_host, oracle.packed_cu_seqlens(a, rb, ro, rnb, 16384))
    assert p1.T == rnb * 16384 and p1.nseg == len(p1.cu_seqlens_host) - 1
    assert p1.max_seqlen == int(np.max(np.diff(p1.cu_seqlens_host)))
    assert cache.get(a, 16384).hit
    assert not cache.get(a, 8192 * 2 + 1).hit  # another capacity: another plan (now 2 entries)
    assert cache.stats() == (1, 2, 2)
    assert not cache.get(b, 16384).hit  # third distinct batch: the least recently used (a, 16384) goes
    assert cache.stats()[2] == 2
    assert not cache.get(a, 16384).hit
    assert cache.get(b, 16384).hit
    assert not cache.get(c, 10000).hit
    empty = cache.get([], 16)
    assert empty.nbins == 0 and list(empty.cu_seqlens_host) == [0] and empty.T == 0
    cache.close()
    with pytest.raises(RuntimeError):
        cache.get(a, 16384)


def test_cache_argument_checks():
    lib = P.load()
    ptr = ctypes.c_void_p()
    assert lib.rope_pack_cache_create(0, -1, ctypes.byref(ptr)) == ERR_SHAPE
    assert lib.rope_pack_cache_create(4, -2, ctypes.byref(ptr)) == ERR_SHAPE
    assert lib.rope_pack_cache_create(4, -1, None) == ERR_NULL
    assert lib.rope_pack_cache_create(4, -1, ctypes.byref(ptr)) == 0
    plan = P._lib.PackPlanStruct()
    L = np.array([5, 20], dtype=np.int32)
    assert lib.rope_pack_cache_get(ptr, ctypes.c_void_p(L.ctypes.data), 2, 10, None, ctypes.byref(plan)) == ERR_SHAPE
    assert lib.rope_pack_cache_get(None, ctypes.c_void_p(L.ctypes.data), 2, 30, None, ctypes.byref(plan)) == ERR_NULL
    assert lib.rope_pack_cache_get(ptr, ctypes.c_void_p(L.ctypes.data), 2, 30, None, None) == ERR_NULL
    assert lib.rope_pack_cache_stats(None, None, None, None) == ERR_NULL
    lib.rope_pack_cache_destroy(ptr)
    lib.rope_pack_cache_destroy(None)
