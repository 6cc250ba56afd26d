"""Pins that tie the Best-Fit-Decreasing oracle (oracle/pack_oracle.py) to the
algorithm's definition by hand-worked cases and properties.

Each ``pin_*`` takes the oracle module (or a copy with a planted mistake) and
raises AssertionError when it disagrees with:

* cases packed by hand (capacity 10), chosen so that best fit, first fit
  and worst fit give different bins, and that ties (equal lengths, equal
  rooms) are visible in the result;
* the packed batch's cu_seqlens for those cases, padding tails included;
* properties on random inputs: every item in one bin, no bin over capacity,
  the items of a bin tile it from token 0 in decreasing length, at least
  ceil(total / capacity) bins, items longer than half a bin never share.
"""

from __future__ import annotations

import numpy as np

# (capacity, lengths, bin_of, offset_of, nbins, cu_seqlens), each worked by hand
HAND_CASES = [
    # 7 -> bin 0 (room 3); 5 -> bin 1 (room 5); 4 -> bin 1 (room 1); the last 1 fits
    # bin 0 (room 3) and bin 1 (room 1): best fit takes bin 1 (first/worst fit: bin 0)
    (10, [5, 7, 4, 1], [1, 0, 1, 1], [0, 0, 5, 9], 2, [0, 7, 10, 15, 19, 20]),
    # 8 -> b0 (2); 5 -> b1 (5); 4 -> b1 (1); 3 -> b2 (7); 1 fits b0 (2), b1 (1), b2 (7):
    # best fit b1, first fit b0, worst fit b2
    (10, [5, 3, 8, 1, 4], [1, 2, 0, 1, 1], [0, 0, 0, 9, 5], 3, [0, 8, 10, 15, 19, 20, 23, 30]),
    # equal lengths go in index order; the first 2 meets two bins of room 2 and takes
    # the one opened first
    (10, [4, 4, 4, 4, 2, 2], [0, 0, 1, 1, 0, 1], [0, 4, 0, 4, 8, 8], 2, [0, 4, 8, 10, 14, 18, 20]),
    # a bin left with room: its tail is one padding segment
    (10, [7, 2], [0, 0], [0, 7], 1, [0, 7, 9, 10]),
    # full-capacity items each fill a bin; zero-length items are empty segments
    (10, [10, 0, 10], [0, 0, 1], [0, 10, 0], 2, [0, 10, 10, 20]),
    # nothing to pack
    (10, [], [], [], 0, [0]),
]


def pin_hand_cases(O):
    for cap, lengths, b, o, nb, cu in HAND_CASES:
        bin_of, offset_of, nbins = O.bfd_pack(lengths, cap)
        assert list(bin_of) == b and list(offset_of) == o and nbins == nb, (lengths, list(bin_of), list(offset_of))
        got = O.packed_cu_seqlens(lengths, bin_of, offset_of, nbins, cap)
        assert list(got) == cu, (lengths, list(got))


def pin_random_properties(O):
    rng = np.random.default_rng(41)
    for trial in range(60):
        cap = int(rng.integers(1, 200))
        n = int(rng.integers(0, 120))
        lengths = rng.integers(0, cap + 1, size=n)
        if trial % 3 == 0:
            lengths = np.minimum(lengths, max(1, cap // 5))  # many small items
        bin_of, offset_of, nbins = O.bfd_pack(lengths, cap)
        assert len(bin_of) == n and len(offset_of) == n
        assert nbins >= -(-int(lengths.sum()) // cap)
        for b in range(nbins):
            idx = [i for i in range(n) if bin_of[i] == b]
            assert idx, "an empty bin"
            idx.sort(key=lambda i: offset_of[i])
            pos = 0
            for i in idx:
                assert offset_of[i] == pos  # contiguous from token 0
                pos += int(lengths[i])
            assert pos <= cap
            lens = [int(lengths[i]) for i in idx]
            assert lens == sorted(lens, reverse=True)  # placed in decreasing length
        big = [i for i in range(n) if 2 * lengths[i] > cap]
        assert len({int(bin_of[i]) for i in big}) == len(big)  # more than half a bin never share
        cu = O.packed_cu_seqlens(lengths, bin_of, offset_of, nbins, cap)
        assert cu[0] == 0 and cu[-1] == nbins * cap and np.all(np.diff(cu) >= 0)


def pin_half_capacity_pairs(O):
    """Items of exactly half a bin pair up: ceil(n / 2) bins."""
    for n in (1, 2, 7, 10):
        _, _, nbins = O.bfd_pack([5] * n, 10)
        assert nbins == -(-n // 2), n


ALL_PACK_PINS = [pin_hand_cases, pin_random_properties, pin_half_capacity_pairs]
