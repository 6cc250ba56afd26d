"""CPU oracle for Best-Fit-Decreasing packing of variable-length sequences and
for the flat cu_seqlens of the packed batch.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it, and it shares nothing with the native packer.

What is computed, and where it comes from
-----------------------------------------
"Chronicals: A High-Performance Framework for LLM Fine-Tuning with 3.51x
Speedup over Unsloth", abstract, optimisation (4): Best-Fit Decreasing
sequence packing recovers most of the compute that padding wastes, with the
usual bin-packing approximation guarantees.  The pages do not spell the
algorithm out; the reading is the textbook one (Johnson, 1973):

* items (sequence lengths) are taken in decreasing order of length, equal
  lengths in increasing order of their index;
* each goes into the open bin whose remaining room is the smallest that
  still holds it, equal rooms to the bin opened first; if no open bin holds
  it, a new bin is opened;
* within a bin, sequences lie one after another in the order they were
  placed, from token 0.

The packed batch: bin b occupies tokens [b * capacity, (b + 1) * capacity) of
one token axis.  Its sequences are segments of cu_seqlens in placement order,
and the unused tail of the bin, when not empty, is one more segment (padding
that the caller masks), so cu_seqlens covers [0, nbins * capacity) and one
launch handles the whole batch.

Plain Python loops over every open bin: quadratic, obviously the definition.
"""

from __future__ import annotations

import numpy as np

__all__ = ["bfd_pack", "packed_cu_seqlens"]


def bfd_pack(lengths, capacity: int):
    """Best-Fit-Decreasing.  Returns (bin_of, offset_of, nbins): for item i its
    bin and its first token inside the bin (numpy int64 arrays)."""
    lengths = [int(x) for x in lengths]
    if capacity < 1:
        raise ValueError("capacity must be >= 1")
    if any(x < 0 or x > capacity for x in lengths):
        raise ValueError("every length must be in [0, capacity]")
    order = sorted(range(len(lengths)), key=lambda i: (-lengths[i], i))
    room = []  # remaining room of each open bin, in opening order
    bin_of = [0] * len(lengths)
    offset_of = [0] * len(lengths)
    for i in order:
        need = lengths[i]
        best = -1
        for b, r in enumerate(room):
            if r >= need and (best < 0 or r < room[best]):
                best = b
        if best < 0:
            room.append(capacity)
            best = len(room) - 1
        bin_of[i] = best
        offset_of[i] = capacity - room[best]
        room[best] -= need
    return np.array(bin_of, dtype=np.int64), np.array(offset_of, dtype=np.int64), len(room)


def packed_cu_seqlens(lengths, bin_of, offset_of, nbins: int, capacity: int) -> np.ndarray:
    """cu_seqlens of the packed batch over nbins * capacity tokens: each bin's
    sequences in token order, then its unused tail as one segment."""
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = [0]
    for b in range(nbins):
        items = sorted((int(offset_of[i]), int(lengths[i])) for i in range(len(lengths)) if bin_of[i] == b)
        pos = b * capacity
        for off, ln in items:
            if b * capacity + off != pos:
                raise ValueError("sequences of a bin must be contiguous from its first token")
            pos += ln
            cu.append(pos)
        if pos < (b + 1) * capacity:
            cu.append((b + 1) * capacity)
    return np.array(cu, dtype=np.int64)
