"""Seeded synthetic inputs for the packed variable-length QK rotary embedding.

This module only *generates* inputs: sequence lengths, the packed layout
(cumulative sequence offsets), and N(0,1) query/key/gradient tensors.  It holds
none of the rotary arithmetic, so both the fp64 oracle and the HIP path can be
fed from it without sharing any of the method's code.

Packing follows the pages' description of padding-free batches: short
sequences are concatenated into one token axis and only their length metadata
is kept ("Unsloth prétend accélérer 5 fois l'entraînement des LLM ..." on
seventnews.com, the auto-packing paragraph), and Chronicals packs rows with
Best-Fit Decreasing ("Chronicals: A High-Performance Framework for LLM
Fine-Tuning with 3.51x Speedup over Unsloth", abstract, optimisation (4)).

Seeds: lengths come from ``numpy.random.default_rng([cfg, 0, 0])``; tensors
from a ``torch.Generator`` seeded with ``cfg * 1000 + tensor_id`` (q=1, k=2,
dq=3, dk=4) on the device they are made on.
"""

from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

# tensor ids for seeding
TID_Q, TID_K, TID_DQ, TID_DK = 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class Workload:
    """One packed batch: shapes, base theta, dtype name and cu_seqlens."""

    cfg: int
    name: str
    T: int
    Hq: int
    Hkv: int
    D: int
    theta: float
    dtype: str  # "fp32", "bf16" or "fp16"
    cu_seqlens: np.ndarray  # int32 [nseq + 1]

    @property
    def nseq(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)

    @property
    def elem_size(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    @property
    def bytes_per_pass(self) -> int:
        """Read + write of q and k once: the algorithmic HBM bytes of one call."""
        return 2 * (self.Hq + self.Hkv) * self.D * self.elem_size * self.T

    def describe(self) -> dict:
        return {
            "workload": self.name,
            "T": self.T,
            "Hq": self.Hq,
            "Hkv": self.Hkv,
            "D": self.D,
            "theta": self.theta,
            "dtype": self.dtype,
            "nseq": self.nseq,
        }


# ---------------------------------------------------------------------------
# sequence lengths and packing
# ---------------------------------------------------------------------------

def cu_from_lengths(lengths: Sequence[int]) -> np.ndarray:
    """Cumulative offsets [0, l0, l0+l1, ...] as int32."""
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    if len(lengths):
        cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    if cu[-1] > np.iinfo(np.int32).max:
        raise ValueError("packed batch exceeds int32 token offsets")
    return cu.astype(np.int32)


def best_fit_decreasing(lengths: Sequence[int], capacity: int) -> List[List[int]]:
    """Textbook Best-Fit Decreasing bin packing.

    Items are taken longest first (ties keep input order); each goes into the
    open bin with the least remaining room that still fits it (ties: lowest
    bin index); a new bin is opened when none fits.  Returns, per bin, the
    indices into ``lengths`` of its items in placement order.  Items longer
    than ``capacity`` are an error.
    """
    lengths = [int(x) for x in lengths]
    for x in lengths:
        if x <= 0 or x > capacity:
            raise ValueError(f"item length {x} outside (0, {capacity}]")
    order = sorted(range(len(lengths)), key=lambda i: (-lengths[i], i))
    bins: List[List[int]] = []
    room: List[int] = []
    for i in order:
        x = lengths[i]
        best = -1
        for b, r in enumerate(room):
            if r >= x and (best < 0 or r < room[best]):
                best = b
        if best < 0:
            bins.append([i])
            room.append(capacity - x)
        else:
            bins[best].append(i)
            room[best] -= x
    return bins


def _mixture_lengths(rng, n, p_first, lo1, hi1, lo2, hi2) -> np.ndarray:
    """n integer lengths: with probability p_first uniform[lo1,hi1], else uniform[lo2,hi2] (inclusive)."""
    first = rng.random(n) < p_first
    a = rng.integers(lo1, hi1 + 1, size=n)
    b = rng.integers(lo2, hi2 + 1, size=n)
    return np.where(first, a, b).astype(np.int64)


def _concat_truncate(lengths: np.ndarray, T: int) -> List[int]:
    """Concatenate lengths in draw order and cut the last one so the sum is exactly T."""
    out: List[int] = []
    total = 0
    for x in lengths:
        x = int(x)
        if total + x >= T:
            out.append(T - total)
            total = T
            break
        out.append(x)
        total += x
    if total != T:
        raise ValueError("not enough lengths drawn to fill T")
    return out


def qwen25_05b_rows(capacity: int = 16384, n_items: int = 256, min_fill: int = 16320):
    """Rows of the Qwen2.5-0.5B-shaped workload.

    256 lengths from the 80% uniform[32,512] / 20% uniform[2048,8192] mixture
    (the 80/20 short/long split the Unsloth article quotes in its packing
    paragraph), packed with Best-Fit Decreasing into 16,384-token rows.  Every
    row whose fill is at least ``min_fill`` is returned as a length list padded
    to the full capacity by one filler segment; the graded row is the one with
    the most sequences.  Returns (graded_index, rows).
    """
    rng = np.random.default_rng([2, 0, 0])
    lengths = _mixture_lengths(rng, n_items, 0.8, 32, 512, 2048, 8192)
    bins = best_fit_decreasing(lengths, capacity)
    rows = []
    for b in bins:
        row = [int(lengths[i]) for i in b]
        fill = sum(row)
        if fill >= min_fill:
            if fill < capacity:
                row.append(capacity - fill)
            rows.append(row)
    if not rows:
        raise RuntimeError("no full row produced")
    graded = max(range(len(rows)), key=lambda r: (len(rows[r]), -r))
    return graded, rows


def make_workload(cfg: int, row: Optional[int] = None) -> Workload:
    """The five packed-batch workloads (1: tiny fp32 check; 2-5: bf16 model shapes).

    ``row`` selects another full Best-Fit-Decreasing row of workload 2 (parity
    cases); by default the graded row is used.
    """
    if cfg == 1:
        cu = cu_from_lengths([7, 33, 64, 152])
        return Workload(1, "tiny-packed-fp32 T=256 Hq=14 Hkv=2 D=64", 256, 14, 2, 64, 1e6, "fp32", cu)
    if cfg == 2:
        graded, rows = qwen25_05b_rows()
        r = graded if row is None else row
        cu = cu_from_lengths(rows[r])
        name = "qwen2.5-0.5b-shaped T=16384 Hq=14 Hkv=2 D=64"
        if row is not None and row != graded:
            name += f" (bfd row {row})"
        return Workload(2, name, 16384, 14, 2, 64, 1e6, "bf16", cu)
    if cfg == 3:
        rng = np.random.default_rng([3, 0, 0])
        raw = np.rint(rng.lognormal(mean=np.log(256.0), sigma=1.0, size=4096))
        lengths = np.clip(raw, 16, 4096).astype(np.int64)
        cu = cu_from_lengths(_concat_truncate(lengths, 65536))
        return Workload(3, "qwen3-8b-shaped T=65536 Hq=32 Hkv=8 D=128", 65536, 32, 8, 128, 1e6, "bf16", cu)
    if cfg == 4:
        rng = np.random.default_rng([4, 0, 0])
        lengths = _mixture_lengths(rng, 4096, 0.5, 64, 1024, 4096, 16384)
        cu = cu_from_lengths(_concat_truncate(lengths, 131072))
        return Workload(4, "qwen3-32b-shaped T=131072 Hq=64 Hkv=8 D=128", 131072, 64, 8, 128, 1e6, "bf16", cu)
    if cfg == 5:
        cu = cu_from_lengths([524288])
        return Workload(5, "llama-3.1-8b-shaped long context T=524288 Hq=32 Hkv=8 D=128", 524288, 32, 8, 128, 5e5, "bf16", cu)
    raise ValueError(f"unknown workload {cfg}")


def qwen25_05b_row_count() -> int:
    return len(qwen25_05b_rows()[1])


# ---------------------------------------------------------------------------
# tensors
# ---------------------------------------------------------------------------

def torch_dtype(name: str):
    import torch

    return {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[name]


def randn(shape, dtype: str, seed: int, device="cpu"):
    """N(0,1) tensor drawn in fp32 from a seeded torch.Generator on ``device``,
    then rounded (round-to-nearest-even) to ``dtype``."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    x = torch.randn(*shape, generator=gen, dtype=torch.float32, device=device)
    if dtype != "fp32":
        x = x.to(torch_dtype(dtype))
    return x


def make_tensors(w: Workload, which=("q", "k"), device="cpu", salt: int = 0):
    """Seeded q/k (and optionally dq/dk) tensors of the workload's shapes."""
    ids = {"q": TID_Q, "k": TID_K, "dq": TID_DQ, "dk": TID_DK}
    heads = {"q": w.Hq, "k": w.Hkv, "dq": w.Hq, "dk": w.Hkv}
    out = {}
    for name in which:
        seed = w.cfg * 1000 + ids[name] + 100003 * salt
        out[name] = randn((w.T, heads[name], w.D), w.dtype, seed, device)
    return out
