"""Benchmark: fused QK-RoPE forward + backward over a packed variable-length batch.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 5] [--table 2,3,4]

One step = the whole hot path over one packed batch: rope_qk_fwd on (q, k)
then rope_qk_bwd on (dq, dk), each one kernel launch through the C ABI.
Inputs are resident in HBM before timing starts; consecutive steps rotate
over enough independent batches (>= 1 GiB in total) that every launch reads
cold HBM rather than the 256 MB Infinity Cache.

The headline workload (default 5: the Llama-3.1-8B-shaped 524,288-token
context, the largest) gives `value` and `roofline`; the other model-shaped
workloads (--table, default 2,3,4) are measured in the same run and listed
under `workloads`, each with its forward and backward launch times and the
plain in-place stream of the same bytes (libstream_ceiling.so) beside them.

Prints ONE JSON line on stdout (progress goes to stderr) with:
  value        tokens/s of the whole step (fwd + bwd), wall clock over K steps
               (replayed as one HIP graph unless --no-graph)
  roofline     the rotation kernel's achieved HBM bandwidth: algorithmic bytes
               per launch (read + write of q and k) / mean launch duration,
               from HIP events bracketing the K steps (2 launches each) on the
               launch stream, against MI355X's 8 TB/s; `traffic` is the
               measured HBM bytes per launch from committed rocprofv3 counters
               when they were taken on the current kernel source, else null
  workloads    per workload: forward and backward us per launch and fraction
               of 8 TB/s, the stream ceiling of the same traffic, traffic
  norm         the fused per-head RMSNorm + rotation on --norm-table's
               workloads: forward and backward us per call and fraction
  cpu_baseline the fp64 numpy oracle on a bounded sample of the headline
               workload, on the host cores (threads used, host cores, CPU)
  parity       a fresh batch's GPU outputs checked against the oracle in the
               same run (the oracle's leg: it runs only with cpu_baseline)
Workloads: 1 tiny fp32, 2 Qwen2.5-0.5B-shaped, 3 Qwen3-8B-shaped,
4 Qwen3-32B-shaped, 5 Llama-3.1-8B-shaped 524,288-token context (default).
"""

from __future__ import annotations

import argparse
import dataclasses
import concurrent.futures as cf
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused QK-RoPE fwd+bwd tokens/s and achieved HBM GB/s (% of MI355X peak)"
HBM_PEAK_GBS = 8000.0
# the rotation kernels' sources and the build script that holds their compile flags
KERNEL_SRCS = [os.path.join(ROOT, "packed_varlen_rotary_amd", "csrc", n)
               for n in ("rope_qk.hip", "rope_common.h", "rope_sincos.h")] + \
              [os.path.join(ROOT, "packed_varlen_rotary_amd", "build.py")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "rope_qk_kernel_traffic.md")
# the machine's CPU share for one GPU: the oracle's thread pool stops there
CPU_SHARE = 16
# a timed graph holds at least this much kernel time, so that the events'
# own overhead (a few microseconds) stays under ~0.2% of the region
MIN_REGION_S = 4e-3
# plain in-place stream variants timed for the ceiling: (chunks per lane,
# persistent workgroups (each with the next two tiles' loads in flight) or 0
# for one tile per workgroup, non-temporal, resident workgroups per compute
# unit or 0 for as many as fit)
CEILING_VARIANTS = [(1, 0, 1, 0), (2, 0, 1, 0), (4, 0, 1, 0), (8, 0, 1, 0), (16, 0, 1, 0), (4, 0, 0, 0),
                    (1, 0, 1, 4), (1, 0, 1, 6), (2, 0, 1, 2), (2, 0, 1, 3), (2, 0, 1, 4), (2, 0, 1, 6),
                    (4, 0, 1, 1), (4, 0, 1, 2), (4, 0, 1, 3), (8, 0, 1, 1), (8, 0, 1, 2),
                    (1, 512, 1, 0), (2, 768, 1, 0), (4, 512, 1, 0), (4, 768, 1, 0)]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sha() -> str:
    """SHA-256 over the rotation kernels' sources and build script, in a fixed order."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload_name: str):
    """HBM bytes per launch from the committed counter summary, if it matches this kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    if not m or m.group(1) != kernel_sha():
        return None
    for line in text.splitlines():
        mm = re.match(r"\|\s*(.+?)\s*\|\s*hbm_bytes_per_launch\s*\|\s*(\d+)\s*\|", line)
        if mm and mm.group(1) == workload_name:
            return int(mm.group(2))
    return None


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a bounded sample
# ---------------------------------------------------------------------------

def oracle_inputs(w, nchunks: int, chunk: int):
    """Seeded inputs for the first `nchunks` token chunks of a workload: each
    chunk's positions and its q and k in float64 (bf16 workloads: rounded to
    bf16), drawn before any clock starts."""
    import numpy as np

    import oracle

    pos_all = oracle.segment_positions(w.cu_seqlens, w.T)
    rng = np.random.default_rng(0)
    chunks = []
    for s in list(range(0, w.T, chunk))[:nchunks]:
        n = min(s + chunk, w.T) - s
        xs = []
        for H in (w.Hq, w.Hkv):
            x = rng.standard_normal((n, H, w.D))
            xs.append(oracle.bf16_rne(x) if w.dtype == "bf16" else x.astype(np.float32).astype(np.float64))
        chunks.append((pos_all[s:s + n], xs))
    return chunks


def oracle_pass(w, pos, xs, directions) -> int:
    """The oracle on one chunk: positions already found, float64 rotation of
    q and k in each direction, rounding to the storage type.  Returns the
    chunk's tokens."""
    import numpy as np

    import oracle

    for x in xs:
        for direction in directions:
            y = oracle.rotate(x, pos, w.theta, direction)
            if w.dtype == "bf16":
                oracle.bf16_bits(oracle.bf16_rne(y))
            else:
                y.astype(np.float32)
    return len(pos)


def oracle_rate(w, chunks, directions, threads: int, budget_s: float):
    """Tokens per second of the oracle over the chunks, for at least budget_s:
    a thread pool over chunks (numpy releases the GIL), or one thread."""
    t0 = time.perf_counter()
    tokens = 0
    if threads > 1:
        with cf.ThreadPoolExecutor(max_workers=threads) as ex:
            while time.perf_counter() - t0 < budget_s:
                tokens += sum(ex.map(lambda c: oracle_pass(w, c[0], c[1], directions), chunks))
    else:
        while time.perf_counter() - t0 < budget_s:
            tokens += oracle_pass(w, chunks[0][0], chunks[0][1], directions)
    dt = time.perf_counter() - t0
    return tokens, dt


def cpu_baseline(w, budget_s: float = 12.0, chunk: int = 1024, single_s: float = 3.0):
    """The oracle on the host cores: positions, float64 rotation of q and k
    forward and backward, rounding to the storage type, on chunks of the
    workload's tokens.  Inputs are drawn before the clock starts, so only the
    oracle is timed; a thread pool over chunks (numpy releases the GIL), and
    the same work on one thread for reference."""
    host_cores = len(os.sched_getaffinity(0))
    threads = min(host_cores, CPU_SHARE)
    chunks = oracle_inputs(w, threads, chunk)
    tokens, dt = oracle_rate(w, chunks, (1, -1), threads, budget_s)
    tokens1, dt1 = oracle_rate(w, chunks, (1, -1), 1, single_s)
    return {
        "value": tokens / dt,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{tokens} tokens of the workload ({chunk}-token chunks, q and k, fwd and bwd, "
                  f"positions+fp64 rotation+bf16 rounding; inputs drawn beforehand) in {dt:.1f} s on {threads} threads",
        "host_cores": host_cores,
        "threads": threads,
        "cpu_model": cpu_model(),
        "thread_cap": f"the pool stops at {CPU_SHARE} threads, the host CPU share one GPU's jobs get",
        "single_thread_value": tokens1 / dt1,
    }


def run_cpu_table(args):
    """The oracle per workload and direction, on one thread and on the pool:
    tokens/s and the effective GB/s of the same algorithmic bytes (read and
    write of q and k).  Host only; one JSON line per workload."""
    import workloads as W

    host_cores = len(os.sched_getaffinity(0))
    threads = min(host_cores, CPU_SHARE)
    log(f"[bench] oracle table: {cpu_model()}, {host_cores} host cores, pool of {threads} threads")
    cfgs = [int(c) for c in args.table.split(",") if c.strip()] if args.table else [1, 2, 3, 4, 5]
    for cfg in cfgs:
        w = W.make_workload(cfg)
        chunks = oracle_inputs(w, threads, 1024)
        bytes_per_token = 2 * (w.Hq + w.Hkv) * w.D * (2 if w.dtype == "bf16" else 4)
        row = {"workload": w.name, "io_dtype": w.dtype, "threads": threads, "host_cores": host_cores,
               "cpu_model": cpu_model()}
        for name, direction in (("fwd", 1), ("bwd", -1)):
            tp, dtp = oracle_rate(w, chunks, (direction,), threads, args.cpu_seconds)
            t1, dt1 = oracle_rate(w, chunks, (direction,), 1, max(1.0, args.cpu_seconds / 3))
            row[name] = {"pool_tokens_per_s": tp / dtp, "pool_gb_per_s": tp / dtp * bytes_per_token / 1e9,
                         "single_tokens_per_s": t1 / dt1, "single_gb_per_s": t1 / dt1 * bytes_per_token / 1e9,
                         "pool_tokens": tp, "pool_seconds": dtp}
            log(f"[bench] oracle {w.name} {name}: {tp / dtp:.0f} tokens/s on {threads} threads, "
                f"{t1 / dt1:.0f} on one")
        print(json.dumps(row), flush=True)


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

def resident_sets(w, names, dev, per_set_bytes, max_sets=64):
    """Enough independent batches (>= 1 GiB together) that each launch reads cold HBM."""
    import workloads as W

    nsets = max(1, min(max_sets, -(-(1 << 30) // per_set_bytes)))
    return [W.make_tensors(w, names, device=dev, salt=s) for s in range(nsets)]


def timed_us(fn, n, graph, warmup=2, warm_s=0.1, region_s=0.02):
    """Mean microseconds per call of fn(i), HIP events on the launch stream
    around R passes of n calls (R passes make up >= region_s), each pass one
    HIP graph replay (or n launches one by one).  Passes totalling >= warm_s
    run untimed first, so that the GPU is at its working clocks whatever ran
    (or did not run) before."""
    import torch

    stream = torch.cuda.current_stream()
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    g = None
    if graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            fn(0)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)

    def one_pass():
        if g is not None:
            g.replay()
        else:
            for i in range(n):
                fn(i)

    start = time.perf_counter()
    one_pass()  # upload and first replay
    torch.cuda.synchronize()
    per_pass = time.perf_counter() - start
    while time.perf_counter() - start < warm_s:
        t = time.perf_counter()
        one_pass()
        torch.cuda.synchronize()
        per_pass = time.perf_counter() - t
    reps = max(1, math.ceil(region_s / max(per_pass, 1e-6)))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        one_pass()
    b.record(stream)
    torch.cuda.synchronize()
    del g
    return a.elapsed_time(b) * 1e3 / (n * reps)


def launches_for(nbytes, steps):
    """Calls per timed region: at least `steps`, and enough for MIN_REGION_S at ~6 TB/s."""
    return max(steps, min(4000, math.ceil(MIN_REGION_S / (nbytes / 6e12))))


def stream_ceiling(nbytes, dev, steps, graph=True, variants=CEILING_VARIANTS):
    """The plain in-place 16-byte stream (libstream_ceiling.so) over buffers of
    nbytes // 2 bytes (read + write = nbytes of traffic), rotating over
    >= 1 GiB, each variant timed like the rotation; returns the fastest."""
    import torch

    from packed_varlen_rotary_amd import stream_ceiling as SC

    half = nbytes // 2
    nb = max(1, min(64, -(-(1 << 30) // half)))
    bufs = [torch.zeros(half, dtype=torch.uint8, device=dev) for _ in range(nb)]
    n = launches_for(nbytes, steps)
    rows = []
    for tpl, groups, nt, cap in variants:
        try:
            us = timed_us(lambda i: SC.stream_ceiling_launch(bufs[i % nb], tpl, groups, nt, cap), n, graph)
        except RuntimeError as e:  # a launch configuration this part does not take
            log(f"[bench] stream {tpl} chunks/lane, groups {groups}, per CU {cap}: {e}")
            torch.cuda.synchronize()
            continue
        gbs = nbytes / (us * 1e-6) / 1e9
        rows.append({"chunks_per_lane": tpl, "groups": groups, "nontemporal": bool(nt), "groups_per_cu": cap,
                     "us": us, "GB/s": gbs, "frac": gbs / HBM_PEAK_GBS})
    del bufs
    torch.cuda.empty_cache()
    best = min(rows, key=lambda r: r["us"])
    keys = ("chunks_per_lane", "groups", "nontemporal", "groups_per_cu")
    return {"us": best["us"], "frac": best["frac"], "variant": {k: best[k] for k in keys}, "launches_timed": n,
            "variants": rows}


def measure_workload(cfg, dev, steps, graph, with_ceiling=True):
    """Forward and backward launch times of one workload (graph-replayed
    launches over resident batches), its stream ceiling and its traffic."""
    import torch

    import packed_varlen_rotary_amd as P
    import workloads as W

    w = W.make_workload(cfg)
    cu = torch.as_tensor(w.cu_seqlens, device=dev)
    sets = resident_sets(w, ("q", "k"), dev, w.bytes_per_pass // 2)
    ns = len(sets)
    n = launches_for(w.bytes_per_pass, steps)
    fwd_us = timed_us(lambda i: P.rope_qk_fwd(sets[i % ns]["q"], sets[i % ns]["k"], cu, w.theta), n, graph)
    bwd_us = timed_us(lambda i: P.rope_qk_bwd(sets[i % ns]["q"], sets[i % ns]["k"], cu, w.theta), n, graph)
    del sets
    torch.cuda.empty_cache()
    gbs = lambda us: w.bytes_per_pass / (us * 1e-6) / 1e9  # noqa: E731
    row = {"workload": w.name, "T": w.T, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "nseq": w.nseq,
           "bytes_per_launch": w.bytes_per_pass, "launches_timed": n, "resident_batches": ns,
           "fwd_us": fwd_us, "bwd_us": bwd_us, "fwd_frac": gbs(fwd_us) / HBM_PEAK_GBS,
           "bwd_frac": gbs(bwd_us) / HBM_PEAK_GBS, "traffic": measured_traffic(w.name)}
    if with_ceiling:
        c = stream_ceiling(w.bytes_per_pass, dev, steps, graph)
        row["stream_ceiling"] = {k: c[k] for k in ("us", "frac", "variant")}
        row["fwd_of_ceiling"] = c["us"] / fwd_us
        row["bwd_of_ceiling"] = c["us"] / bwd_us
    log(f"[bench] {w.name}: fwd {fwd_us:.2f} us ({100 * row['fwd_frac']:.1f}%), bwd {bwd_us:.2f} us "
        f"({100 * row['bwd_frac']:.1f}%)" + (f"; stream ceiling {row['stream_ceiling']['us']:.2f} us "
                                              f"({100 * row['stream_ceiling']['frac']:.1f}%)" if with_ceiling else ""))
    return row


def run_gpu(args):
    import torch

    import packed_varlen_rotary_amd as P
    import workloads as W

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    w = W.make_workload(args.workload)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cu = torch.as_tensor(w.cu_seqlens, device=dev)
    set_bytes = w.bytes_per_pass  # q, k, dq, dk of one batch: (Hq+Hkv)*D*s*T bytes per pair
    sets = resident_sets(w, ("q", "k", "dq", "dk"), dev, set_bytes)
    nsets = len(sets)
    log(f"[bench] {w.name}: {nsets} resident batches of {set_bytes / 2**20:.1f} MiB")

    def step(i):
        b = sets[i % nsets]
        P.rope_qk_fwd(b["q"], b["k"], cu, w.theta)
        P.rope_qk_bwd(b["dq"], b["dk"], cu, w.theta)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    graph = None
    if args.graph:
        # the K timed steps as one HIP graph (the entry points make no host
        # syncs and allocate nothing, so they capture as plain kernel nodes)
        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            step(0)
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                step(i)
        graph.replay()  # upload and first replay: untimed
        torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_start.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    region_ms = t_start.elapsed_time(t_end)
    del graph

    # the forward and the backward on their own (same replay, enough launches
    # for a region of MIN_REGION_S); --no-split leaves them out (counter runs)
    n = launches_for(w.bytes_per_pass, args.steps)
    fwd_us = bwd_us = None
    if args.split:
        fwd_us = timed_us(lambda i: P.rope_qk_fwd(sets[i % nsets]["q"], sets[i % nsets]["k"], cu, w.theta), n,
                          args.graph)
        bwd_us = timed_us(lambda i: P.rope_qk_bwd(sets[i % nsets]["dq"], sets[i % nsets]["dk"], cu, w.theta), n,
                          args.graph)
        log(f"[bench] {w.name}: forward {fwd_us:.2f} us, backward {bwd_us:.2f} us per launch ({n} launches each)")
    del sets
    torch.cuda.empty_cache()

    # a fresh batch's outputs for the oracle leg's parity check, in the same run
    sample = parity_sample(w, cu, dev)
    torch.cuda.empty_cache()

    launch_ms = region_ms / (2 * args.steps)  # HIP events around the K steps, on the launch stream
    ms_per_step = wall * 1e3 / args.steps
    gbs = lambda us: w.bytes_per_pass / (us * 1e-6) / 1e9  # noqa: E731
    row = {"workload": w.name, "T": w.T, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "nseq": w.nseq,
           "bytes_per_launch": w.bytes_per_pass, "launches_timed": n, "resident_batches": nsets,
           "fwd_us": fwd_us, "bwd_us": bwd_us,
           "fwd_frac": gbs(fwd_us) / HBM_PEAK_GBS if fwd_us else None,
           "bwd_frac": gbs(bwd_us) / HBM_PEAK_GBS if bwd_us else None, "traffic": measured_traffic(w.name)}
    if args.ceiling and args.split:
        c = stream_ceiling(w.bytes_per_pass, dev, args.steps, args.graph)
        row["stream_ceiling"] = {k: c[k] for k in ("us", "frac", "variant")}
        row["fwd_of_ceiling"] = c["us"] / fwd_us
        row["bwd_of_ceiling"] = c["us"] / bwd_us
        log(f"[bench] {w.name}: stream ceiling {c['us']:.2f} us ({100 * c['frac']:.1f}%), variant {c['variant']}")
    return w, {
        "ms_per_step": ms_per_step,
        "tokens_per_s": w.T / (ms_per_step * 1e-3),
        "event_ms_per_step": region_ms / args.steps,
        "launch_ms": launch_ms,
        "gbs": w.bytes_per_pass / (launch_ms * 1e-3) / 1e9,
        "traffic": row["traffic"],
        "fwd_us": fwd_us,
        "bwd_us": bwd_us,
        "parity_sample": sample,
        "resident_batches": nsets,
        "device": torch.cuda.get_device_name(dev),
        "row": row,
    }


def parity_sample(w, cu, dev):
    """A fresh batch of the workload through rope_qk_fwd (q, k) and
    rope_qk_bwd (dq, dk): the inputs and outputs of every token (workloads of
    up to 4e7 elements) or of sampled tokens (the first, the last, every
    sequence start and 512 drawn at random), copied to the host.  The oracle
    leg checks them."""
    import numpy as np
    import torch

    import packed_varlen_rotary_amd as P
    import workloads as W

    t = W.make_tensors(w, ("q", "k", "dq", "dk"), device=dev, salt=999)
    if w.T * (w.Hq + w.Hkv) * w.D <= 40_000_000:
        idx = np.arange(w.T)
    else:
        rng = np.random.default_rng(1)
        idx = np.unique(np.concatenate([[0, w.T - 1], w.cu_seqlens[:-1], rng.integers(0, w.T, 512)]))
        idx = idx[(idx >= 0) & (idx < w.T)]  # a sequence may start at T (empty trailing segments)
    idx_d = torch.as_tensor(idx, device=dev)
    x = {n: t[n].index_select(0, idx_d).float().cpu().numpy().astype(np.float64) for n in t}
    P.rope_qk_fwd(t["q"], t["k"], cu, w.theta)
    P.rope_qk_bwd(t["dq"], t["dk"], cu, w.theta)
    torch.cuda.synchronize()
    out = {}
    for n in t:
        o = t[n].index_select(0, idx_d).cpu()
        out[n] = o.numpy().astype(np.float64) if w.dtype == "fp32" else o.view(torch.int16).numpy().view(np.uint16)
    return {"idx": idx, "x": x, "out": out}


def oracle_parity(w, sample):
    """The oracle's outputs for the sampled tokens against the GPU's: bf16 as
    ulp distance on the bf16 grid (with the bit-exact fraction), fp32 as
    the largest absolute difference."""
    import numpy as np

    import oracle

    idx = sample["idx"]
    pos = oracle.segment_positions(w.cu_seqlens, w.T)[idx]
    worst = {"max_ulp": 0, "max_abs": 0.0, "exact_fraction": 1.0, "tokens_checked": int(len(idx))}
    exact_n, total_n = 0, 0
    for n, d in (("q", 1), ("k", 1), ("dq", -1), ("dk", -1)):
        ref = oracle.rotate(sample["x"][n], pos, w.theta, d)
        got = sample["out"][n]
        if w.dtype == "fp32":
            worst["max_abs"] = max(worst["max_abs"], float(np.abs(got - ref).max()))
        else:
            dist = oracle.ulp_distance_bf16(got, oracle.bf16_bits(oracle.bf16_rne(ref)))
            worst["max_ulp"] = max(worst["max_ulp"], int(dist.max()))
            exact_n += int((dist == 0).sum())
            total_n += dist.size
    if total_n:
        worst["exact_fraction"] = exact_n / total_n
    worst["ok"] = bool(worst["max_ulp"] <= 1 and worst["max_abs"] <= 1e-5)
    return worst


def run_copy_calibration(args):
    """A plain device-to-device copy of a known size, for scaling HBM counters."""
    import torch

    n = args.copy_bytes // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copied {n * 2} bytes x {args.steps}")


def run_copy_ceiling(args):
    """Context for the roofline: the runtime's device-to-device copy moving the
    same HBM traffic as one launch of the workload (read + write of
    bytes_per_pass / 2 bytes), replayed from a HIP graph over rotating buffers
    of >= 1 GiB, timed with events around the replay."""
    import torch

    import workloads as W

    w = W.make_workload(args.workload)
    n = w.bytes_per_pass // 2
    nb = max(2, min(64, -(-(1 << 30) // n)))
    src = [torch.ones(n, dtype=torch.uint8, device="cuda") for _ in range(nb)]
    dst = [torch.empty(n, dtype=torch.uint8, device="cuda") for _ in range(nb)]
    for i in range(args.warmup):
        dst[i % nb].copy_(src[i % nb])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(args.steps):
            dst[i % nb].copy_(src[(i + 1) % nb])
    graph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    graph.replay()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / args.steps
    gbs = w.bytes_per_pass / (us * 1e-6) / 1e9
    log(f"[bench] copy of {n} bytes ({w.bytes_per_pass} bytes of traffic): {us:.2f} us, {gbs:.0f} GB/s")
    print(json.dumps({"metric": "device-to-device copy with one launch's HBM traffic", "workload": w.name,
                      "traffic_bytes": w.bytes_per_pass, "us_per_copy": us, "GB/s": gbs, "frac": gbs / HBM_PEAK_GBS}))


def measure_norm(cfg: int, steps: int, warmup: int, graph: bool) -> dict:
    """The fused per-head RMSNorm + rotation (rope_qk_norm_fwd out of place,
    rope_qk_norm_bwd into a separate dx) on a workload's shapes: each pass
    timed on its own as a graph of `steps` calls over resident sets of
    >= 1 GiB (one by one without a graph), HIP events around the replays
    after 0.1 s of warm-up.  Algorithmic bytes: forward read x + write y,
    backward read x and dy + write dx (the weight-gradient workspace is extra
    traffic, reported separately)."""
    import torch

    import packed_varlen_rotary_amd as P
    import workloads as W

    w = W.make_workload(cfg)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cu = torch.as_tensor(w.cu_seqlens, device=dev)
    qk_bytes = w.bytes_per_pass // 2  # q and k once
    nsets = max(1, min(16, -(-(1 << 30) // (4 * qk_bytes))))
    sets = []
    for s in range(nsets):
        b = W.make_tensors(w, ("q", "k", "dq", "dk"), device=dev, salt=s)
        b["yq"], b["yk"] = torch.empty_like(b["q"]), torch.empty_like(b["k"])
        b["xq"], b["xk"] = torch.empty_like(b["q"]), torch.empty_like(b["k"])
        sets.append(b)
    g = torch.Generator(device="cpu")
    g.manual_seed(7)
    wq = (1.0 + 0.25 * torch.randn(w.D, generator=g)).float().to(dev)
    wk = (1.0 + 0.25 * torch.randn(w.D, generator=g)).float().to(dev)
    eps = 1e-6
    code = {"bf16": P.ROPE_QK_BF16, "fp16": P.ROPE_QK_FP16, "fp32": P.ROPE_QK_FP32}[w.dtype]
    ws_bytes = P.rope_qk_norm_bwd_workspace_bytes(w.T, w.Hq, w.Hkv, w.D, code)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    dwq = torch.empty(w.D, dtype=torch.float32, device=dev)
    dwk = torch.empty(w.D, dtype=torch.float32, device=dev)
    log(f"[bench] norm {w.name}: {nsets} resident sets of {4 * qk_bytes / 2**20:.1f} MiB, "
        f"workspace {ws_bytes / 2**20:.2f} MiB")

    def fwd(i):
        b = sets[i % nsets]
        P.rope_qk_norm_fwd(b["q"], b["k"], wq, wk, eps, cu, w.theta, b["yq"], b["yk"])

    def bwd(i):
        b = sets[i % nsets]
        P.rope_qk_norm_bwd(b["dq"], b["dk"], b["q"], b["k"], wq, wk, eps, cu, w.theta, b["xq"], b["xk"],
                           dwq, dwk, ws)

    res = {"workload": w.name, "io_dtype": w.dtype, "resident_sets": nsets, "workspace_bytes": ws_bytes,
           "calls_timed": steps}
    for name, fn, nbytes in (("fwd", fwd, 2 * qk_bytes), ("bwd", bwd, 3 * qk_bytes)):
        us = timed_us(fn, steps, graph, warmup=warmup)
        gbs = nbytes / (us * 1e-6) / 1e9
        res[name] = {"us_per_call": us, "algorithmic_bytes": nbytes, "GB/s": gbs, "frac": gbs / HBM_PEAK_GBS}
        log(f"[bench] norm {name}: {us:.2f} us per call, {gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of peak)")
    del sets, ws
    torch.cuda.empty_cache()
    return res


def run_norm(args):
    """--norm: measure_norm on --workload, as one JSON line."""
    import torch

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    res = measure_norm(args.workload, args.steps, args.warmup, args.graph)
    print(json.dumps({"metric": "fused per-head QK-RMSNorm + RoPE, achieved HBM GB/s per pass", "steps": args.steps,
                      "peak": HBM_PEAK_GBS, **res}))


def run_pack(args):
    """The host packing pipeline: the native Best-Fit-Decreasing packer's
    throughput (the oracle's on a bounded sample beside it), the
    packed-metadata cache's miss and hit latency, and a 24-layer forward loop
    over a BFD-packed batch (Qwen2.5-0.5B-shaped heads) that either looks the
    batch's metadata up in the cache every layer or rebuilds and uploads
    cu_seqlens every layer."""
    import numpy as np
    import torch

    import oracle
    import packed_varlen_rotary_amd as P
    import workloads as W

    rng = np.random.default_rng(0)

    def mixture(n):  # 80% U[32,512] / 20% U[2048,8192], the default workload's length mix
        return np.where(rng.random(n) < 0.8, rng.integers(32, 513, size=n), rng.integers(2048, 8193, size=n))

    cap = 16384
    big = mixture(1_000_000)
    best = min(_timed(lambda: P.pack_bfd(big, cap)) for _ in range(3))
    sample = big[:4000]
    t_or = _timed(lambda: oracle.bfd_pack(sample, cap))
    log(f"[bench] pack: native BFD {big.size / best / 1e6:.2f} M lengths/s (1M lengths), "
        f"oracle {sample.size / t_or / 1e3:.1f} K lengths/s (4000 lengths; quadratic)")
    res = {"native_bfd": {"lengths": int(big.size), "s": best, "lengths_per_s": big.size / best},
           "oracle_bfd": {"lengths": int(sample.size), "s": t_or, "lengths_per_s": sample.size / t_or}}
    if torch.cuda.is_available():
        dev = torch.device("cuda", 0)
        torch.cuda.set_device(dev)
        cache = P.PackCache(max_entries=8, device=dev)
        cache.get(mixture(256), cap)  # the process's first pinned and device allocations: untimed
        torch.cuda.synchronize()
        batch = mixture(256)
        t_miss = _timed(lambda: cache.get(batch, cap))
        hits = 2000
        t_hit = _timed(lambda: [cache.get(batch, cap) for _ in range(hits)]) / hits
        plan = cache.get(batch, cap)
        torch.cuda.synchronize()
        layers, Hq, Hkv, D = 24, 14, 2, 64
        q = W.randn((plan.T, Hq, D), "bf16", seed=1, device=dev)
        k = W.randn((plan.T, Hkv, D), "bf16", seed=2, device=dev)

        def cached_step():
            for _ in range(layers):
                P.rope_qk_fwd(q, k, cache.get(batch, cap).cu_seqlens, 1e6)

        def rebuilt_step():
            for _ in range(layers):
                b, o, nb = P.pack_bfd(batch, cap)
                cu = torch.as_tensor(P.packed_cu_seqlens(batch, b, o, nb, cap), device=dev)
                P.rope_qk_fwd(q, k, cu, 1e6)

        out = {}
        for name, fn in (("cached", cached_step), ("rebuilt", rebuilt_step)):
            fn()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(10):
                fn()
            torch.cuda.synchronize()
            out[name] = (time.perf_counter() - t0) / 10
        log(f"[bench] pack cache: miss {t_miss * 1e6:.0f} us, hit {t_hit * 1e6:.2f} us; {layers}-layer forward loop "
            f"over {plan.T} tokens: {out['cached'] * 1e3:.3f} ms cached vs {out['rebuilt'] * 1e3:.3f} ms rebuilt")
        res["cache"] = {"miss_us": t_miss * 1e6, "hit_us": t_hit * 1e6, "batch_lengths": int(batch.size),
                        "tokens": plan.T, "bins": plan.nbins}
        res["layer_loop"] = {"layers": layers, "ms_cached": out["cached"] * 1e3, "ms_rebuilt": out["rebuilt"] * 1e3}
        cache.close()
    print(json.dumps({"metric": "host packing pipeline: BFD throughput and packed-metadata cache latency", **res}))


def run_eager_baseline(args):
    """Context for the fusion: an unfused rotate_half RoPE written with PyTorch
    eager ops (float32 cos/sin tables gathered by position, q and k rotated
    separately, out of place) on the same workload and GPU, next to the fused
    in-place kernel.  Not a parity path: only its time is reported."""
    import torch

    import packed_varlen_rotary_amd as P
    import workloads as W

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    w = W.make_workload(args.workload)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cu = torch.as_tensor(w.cu_seqlens, device=dev)
    nsets = max(1, min(16, -(-(1 << 30) // w.bytes_per_pass)))
    sets = [W.make_tensors(w, ("q", "k"), device=dev, salt=s) for s in range(nsets)]
    pos = P.rope_qk_positions(cu, w.T).clamp_min(0).long()
    half = w.D // 2
    inv = 1.0 / (w.theta ** (torch.arange(0, half, device=dev, dtype=torch.float32) * 2.0 / w.D))
    max_pos = int(pos.max().item()) + 1
    freqs = torch.outer(torch.arange(max_pos, device=dev, dtype=torch.float32), inv)
    cos_t = torch.cat([freqs.cos(), freqs.cos()], -1).to(sets[0]["q"].dtype)
    sin_t = torch.cat([freqs.sin(), freqs.sin()], -1).to(sets[0]["q"].dtype)

    def rotate_half(x):
        return torch.cat([-x[..., half:], x[..., :half]], -1)

    def eager(i):
        b = sets[i % nsets]
        c = cos_t[pos][:, None, :]
        s = sin_t[pos][:, None, :]
        return b["q"] * c + rotate_half(b["q"]) * s, b["k"] * c + rotate_half(b["k"]) * s

    def fused(i):
        b = sets[i % nsets]
        P.rope_qk_fwd(b["q"], b["k"], cu, w.theta)

    res = {}
    for name, fn in (("eager_unfused", eager), ("fused", fused)):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(args.steps):
            fn(i)
        b_.record()
        torch.cuda.synchronize()
        res[name] = a.elapsed_time(b_) * 1e3 / args.steps
    log(f"[bench] {w.name}: eager unfused RoPE {res['eager_unfused']:.1f} us, fused in place {res['fused']:.1f} us "
        f"per forward ({res['eager_unfused'] / res['fused']:.1f}x)")
    print(json.dumps({"metric": "forward RoPE of q and k: PyTorch eager (unfused) vs the fused kernel", "workload": w.name,
                      "us_eager_unfused": res["eager_unfused"], "us_fused": res["fused"],
                      "speedup": res["eager_unfused"] / res["fused"], "steps": args.steps,
                      "note": "launched one by one (no graph) for both"}))


def run_variants(args):
    """The rotation's options on one workload, forward only: each case timed
    as a graph of K launches over resident batches (HIP events around the
    replay).  Algorithmic bytes: read + write of the rotated elements (all of
    each head, or the leading rotary_dim of it)."""
    import torch

    import packed_varlen_rotary_amd as P
    import workloads as W

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    w = W.make_workload(args.workload)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cu = torch.as_tensor(w.cu_seqlens, device=dev)
    llama3 = dict(factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0, original_max_position=8192.0)
    cases = [
        ("plain", {}, w.dtype),
        ("pos_offset=100000", dict(pos_offset=100000), w.dtype),
        (f"rotary_dim={w.D // 2}", dict(rotary_dim=w.D // 2), w.dtype),
        ("interleaved", dict(interleaved=True), w.dtype),
        ("llama3", dict(llama3=llama3), w.dtype),
        ("freq_fp32", dict(freq_fp32=True), w.dtype),
        ("fp16", {}, "fp16"),
        ("fp32", {}, "fp32"),
        ("interleaved+llama3+freq_fp32+pos_offset", dict(interleaved=True, llama3=llama3, freq_fp32=True,
                                                         pos_offset=77), w.dtype),
    ]
    if args.case:
        want = args.case.split(",")
        unknown = [c for c in want if c not in [n for n, _, _ in cases]]
        if unknown:
            raise SystemExit(f"unknown --case {unknown}; cases: {[n for n, _, _ in cases]}")
        cases = [c for c in cases if c[0] in want]
    res = []
    for name, opts, dt in cases:
        wd = dataclasses.replace(w, dtype=dt)
        nsets = max(1, min(16, -(-(1 << 30) // wd.bytes_per_pass)))
        sets = [W.make_tensors(wd, ("q", "k"), device=dev, salt=s) for s in range(nsets)]

        def fwd(i):
            b = sets[i % nsets]
            P.rope_qk_fwd(b["q"], b["k"], cu, w.theta, **opts)

        for i in range(args.warmup):
            fwd(i)
        torch.cuda.synchronize()
        a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if args.graph:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(args.steps):
                    fwd(i)
            graph.replay()
            torch.cuda.synchronize()
            a.record()
            graph.replay()
            b_.record()
        else:  # one launch at a time (counter runs)
            graph = None
            a.record()
            for i in range(args.steps):
                fwd(i)
            b_.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b_) * 1e3 / args.steps
        r = opts.get("rotary_dim", 0) or w.D
        nbytes = wd.bytes_per_pass * r // w.D
        gbs = nbytes / (us * 1e-6) / 1e9
        log(f"[bench] {w.name} {name} ({dt}): {us:.2f} us, {gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}%)")
        res.append({"case": name, "dtype": dt, "us_per_launch": us, "algorithmic_bytes": nbytes, "GB/s": gbs,
                    "frac": gbs / HBM_PEAK_GBS})
        del sets, graph
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "rope_qk_fwd with each option, per launch", "workload": w.name, "steps": args.steps,
                      "peak": HBM_PEAK_GBS, "cases": res}))


def run_stream_ceiling(args):
    """Every plain in-place stream variant with one launch's HBM traffic of
    --workload (read + write of q and k), timed like the rotation."""
    import torch

    import workloads as W

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    w = W.make_workload(args.workload)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    c = stream_ceiling(w.bytes_per_pass, dev, args.steps, args.graph)
    for v in c["variants"]:
        log(f"[bench] stream {v['chunks_per_lane']} chunks/lane, groups {v['groups']}, nt {v['nontemporal']}, "
            f"per CU {v['groups_per_cu']}: {v['us']:.2f} us ({100 * v['frac']:.1f}%)")
    print(json.dumps({"metric": "plain in-place 16-byte stream with one launch's HBM traffic", "workload": w.name,
                      "traffic_bytes": w.bytes_per_pass, "launches_timed": c["launches_timed"], "best_us": c["us"],
                      "best_frac": c["frac"], "best_variant": c["variant"], "variants": c["variants"]}))


def _timed(fn):
    t0 = time.perf_counter()
    fn()
    return time.perf_counter() - t0


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=5, choices=[1, 2, 3, 4, 5],
                    help="the headline workload (default 5: the 524,288-token Llama-3.1-8B-shaped context)")
    ap.add_argument("--table", default="2,3,4",
                    help="other workloads measured in the same run (comma-separated; empty: none)")
    ap.add_argument("--norm-table", default="3",
                    help="workloads on which the fused RMSNorm + rotation (forward and backward) is also timed in "
                         "the same run (comma-separated; empty: none)")
    ap.add_argument("--no-ceiling", dest="ceiling", action="store_false",
                    help="skip the plain-stream ceiling beside each workload")
    ap.add_argument("--no-split", dest="split", action="store_false",
                    help="skip the forward-only and backward-only timings (few launches, for counter runs)")
    ap.add_argument("--stream-ceiling", action="store_true",
                    help="only time every plain in-place stream variant with one launch's traffic of --workload")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="launch the timed steps one by one on the stream instead of replaying a HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain copy of --copy-bytes (for HBM counter scaling)")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    ap.add_argument("--eager-baseline", action="store_true",
                    help="only time an unfused PyTorch-eager RoPE beside the fused kernel (context)")
    ap.add_argument("--variants", action="store_true",
                    help="only time the rotation's options (forward) on the workload")
    ap.add_argument("--case", default="",
                    help="with --variants: only these cases (comma-separated names, e.g. plain,fp16)")
    ap.add_argument("--pack", action="store_true",
                    help="only time the BFD packer and the packed-metadata cache")
    ap.add_argument("--norm", action="store_true",
                    help="only time the fused RMSNorm + rotation kernels (forward and backward) on --workload")
    ap.add_argument("--copy-ceiling", action="store_true",
                    help="only time the runtime's device copy with one launch's HBM traffic (roofline context)")
    ap.add_argument("--cpu-table", action="store_true",
                    help="only time the oracle per workload (--table, default all) and direction, on the host "
                         "(--cpu-seconds per pool measurement)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the rotation is per token and needs no "
              "exchange, so more GPUs would each run this same one-GPU workload on their own shard.",
              file=sys.stderr)
        sys.exit(2)
    if args.cpu_table:
        if not any(a.startswith("--table") for a in sys.argv[1:]):
            args.table = ""
        run_cpu_table(args)
        return
    if args.copy_calibration:
        run_copy_calibration(args)
        return
    if args.copy_ceiling:
        run_copy_ceiling(args)
        return
    if args.norm:
        run_norm(args)
        return
    if args.pack:
        run_pack(args)
        return
    if args.eager_baseline:
        run_eager_baseline(args)
        return
    if args.variants:
        run_variants(args)
        return
    if args.stream_ceiling:
        run_stream_ceiling(args)
        return

    w, r = run_gpu(args)
    log(f"[bench] gpu done: {r['ms_per_step']:.4f} ms/step, mean launch {r['launch_ms'] * 1e3:.2f} us, "
        f"{r['gbs']:.0f} GB/s")
    import torch

    rows = [r["row"]]
    for cfg in [int(c) for c in args.table.split(",") if c.strip()]:
        if cfg != args.workload:
            rows.append(measure_workload(cfg, torch.device("cuda", 0), args.steps, args.graph, args.ceiling))
    norm_rows = [measure_norm(int(c), max(args.steps, 20), args.warmup, args.graph)
                 for c in args.norm_table.split(",") if c.strip()]
    # the oracle's leg: its outputs against the GPU's on the fresh batch
    # (parity), and its own speed on the host cores (cpu_baseline)
    cpu = None
    parity = {"skipped": "--no-cpu-baseline: the oracle leg did not run"}
    if args.workload and not args.no_cpu_baseline:
        parity = oracle_parity(w, r["parity_sample"])
        log(f"[bench] parity {parity}")
        cpu = cpu_baseline(w, args.cpu_seconds)
        log(f"[bench] cpu oracle: {cpu['value']:.0f} tokens/s on {cpu['cores']} threads")

    achieved = r["gbs"]
    line = {
        "metric": METRIC,
        "value": r["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "T": w.T, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "theta": w.theta,
            "io_dtype": w.dtype, "nseq": w.nseq,
            "step": "rope_qk_fwd(q,k) + rope_qk_bwd(dq,dk), in place",
            "resident_batches": r["resident_batches"],
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": r["traffic"],
        },
        "cpu_baseline": cpu,
        "kernel": {
            "name": "rope_qk_kernel",
            "launches_per_step": 2,
            "algorithmic_bytes_per_launch": w.bytes_per_pass,
            "mean_launch_us": r["launch_ms"] * 1e3,
            "fwd_launch_us": r["fwd_us"],
            "bwd_launch_us": r["bwd_us"],
            "event_ms_per_step": r["event_ms_per_step"],
            "launch": "hip graph of the K steps" if args.graph else "stream launches",
        },
        "workloads": rows,
        "norm": norm_rows,
        "parity": parity,
        "device": r["device"],
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
