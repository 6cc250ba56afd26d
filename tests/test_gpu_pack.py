"""The packed-metadata cache on the device (needs an MI355X): the uploaded
cu_seqlens, hits answered without device work, and the rotation driven by
the cached metadata."""

import time

import numpy as np
import pytest
import torch

import oracle
import packed_varlen_rotary_amd as P
import workloads as W
from tests.gpu_util import check_against, f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def mixture(n, seed):
    rng = np.random.default_rng(seed)
    return np.where(rng.random(n) < 0.8, rng.integers(32, 513, size=n), rng.integers(2048, 8193, size=n))


def test_device_plan_and_hits():
    cache = P.PackCache(max_entries=4)
    lengths = mixture(300, 1)
    p = cache.get(lengths, 16384)
    torch.cuda.synchronize()
    assert not p.hit and p.cu_seqlens is not None and p.cu_seqlens.device.type == "cuda"
    assert p.cu_seqlens.dtype == torch.int32 and p.cu_seqlens.numel() == p.nseg + 1
    assert np.array_equal(p.cu_seqlens.cpu().numpy(), p.cu_seqlens_host)
    rb, ro, rnb = oracle.bfd_pack(lengths, 16384)
    assert np.array_equal(p.cu_seqlens_host, oracle.packed_cu_seqlens(lengths, rb, ro, rnb, 16384))
    q = cache.get(lengths, 16384)
    assert q.hit and q.cu_seqlens_ptr == p.cu_seqlens_ptr
    assert q.cu_seqlens.data_ptr() == p.cu_seqlens.data_ptr()  # a hit shares the first copy
    assert cache.stats() == (1, 1, 1)
    cache.close()


def test_rotation_with_cached_metadata():
    """q and k of a BFD-packed batch rotated with the cache's device cu_seqlens:
    identical to the same call with a torch-made cu_seqlens, and to the oracle."""
    cache = P.PackCache(max_entries=2)
    lengths = mixture(40, 2)
    p = cache.get(lengths, 8192)
    Hq, Hkv, D = 6, 2, 64
    q = W.randn((p.T, Hq, D), "bf16", seed=3, device=DEV)
    k = W.randn((p.T, Hkv, D), "bf16", seed=4, device=DEV)
    xq, xk = f64(q), f64(k)
    q2, k2 = q.clone(), k.clone()
    P.rope_qk_fwd(q, k, p.cu_seqlens, 1e6)
    P.rope_qk_fwd(q2, k2, torch.as_tensor(p.cu_seqlens_host, device=DEV), 1e6)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(k, k2)
    check_against(q, oracle.rope(xq, p.cu_seqlens_host, 1e6, 1), "q")
    check_against(k, oracle.rope(xk, p.cu_seqlens_host, 1e6, 1), "k")
    cache.close()


def test_hits_do_not_wait_for_the_device():
    """With ~0.2 s of rotation queued on the stream, 300 lookups of a cached
    batch return while the GPU is still busy: a hit makes no device call."""
    cache = P.PackCache(max_entries=2)
    lengths = mixture(200, 5)
    p = cache.get(lengths, 16384)
    torch.cuda.synchronize()
    w = W.make_workload(3)
    t = W.make_tensors(w, ("q", "k"), device=DEV)
    cu = torch.as_tensor(w.cu_seqlens, device=DEV)
    for _ in range(1000):  # ~0.2 s of kernels queued
        P.rope_qk_fwd(t["q"], t["k"], cu, w.theta)
    busy = torch.cuda.Event()
    busy.record()
    t0 = time.perf_counter()
    for _ in range(300):
        assert cache.get(lengths, 16384).hit
    host_s = time.perf_counter() - t0
    still_busy = not busy.query()
    torch.cuda.synchronize()
    assert still_busy, f"the GPU finished before 300 hits returned ({host_s * 1e3:.1f} ms)"
    assert cache.stats()[0] == 300
    cache.close()
    del t
    torch.cuda.empty_cache()


def test_eviction_keeps_live_plans_correct():
    cache = P.PackCache(max_entries=2)
    batches = [mixture(50, s) for s in (10, 11, 12)]
    plans = [cache.get(b, 8192) for b in batches]  # the third evicts the first
    torch.cuda.synchronize()
    for pl in plans[1:]:
        assert np.array_equal(pl.cu_seqlens.cpu().numpy(), pl.cu_seqlens_host)
    again = cache.get(batches[0], 8192)
    torch.cuda.synchronize()
    assert not again.hit and np.array_equal(again.cu_seqlens.cpu().numpy(), plans[0].cu_seqlens_host)
    cache.close()


def test_plans_outlive_eviction_and_close():
    """A plan's device cu_seqlens is torch-owned: after its cache entry is
    evicted (and its cache buffer freed) and after the cache is closed, it
    still holds the plan and drives the rotation like a fresh upload."""
    cache = P.PackCache(max_entries=1)
    batches = [mixture(60, s) for s in (20, 21, 22)]
    plans = [cache.get(b, 8192) for b in batches]  # each evicts the one before
    torch.cuda.synchronize()
    junk = [torch.full((4096,), -7, dtype=torch.int32, device=DEV) for _ in range(64)]  # reuse freed memory
    cache.close()
    torch.cuda.synchronize()
    for pl in plans:
        assert np.array_equal(pl.cu_seqlens.cpu().numpy(), pl.cu_seqlens_host)
    p0 = plans[0]
    q = W.randn((p0.T, 4, 64), "bf16", seed=8, device=DEV)
    k = W.randn((p0.T, 2, 64), "bf16", seed=9, device=DEV)
    q2, k2 = q.clone(), k.clone()
    P.rope_qk_fwd(q, k, p0.cu_seqlens, 1e6)
    P.rope_qk_fwd(q2, k2, torch.as_tensor(p0.cu_seqlens_host, device=DEV), 1e6)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(k, k2)
    del junk
