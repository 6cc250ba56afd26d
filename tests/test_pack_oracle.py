"""The Best-Fit-Decreasing oracle against its pins (CPU), and planted mistakes
that the pins must catch."""

import numpy as np
import pytest

import oracle.pack_oracle as K
from tests import pack_pins


@pytest.mark.parametrize("pin", pack_pins.ALL_PACK_PINS, ids=lambda f: f.__name__)
def test_pack_pin(pin):
    pin(K)


def _variant(lengths, capacity, choose, order_key=lambda L, i: (-L[i], i)):
    lengths = [int(x) for x in lengths]
    order = sorted(range(len(lengths)), key=lambda i: order_key(lengths, i))
    room, bin_of, offset_of = [], [0] * len(lengths), [0] * len(lengths)
    for i in order:
        fits = [b for b, r in enumerate(room) if r >= lengths[i]]
        b = choose(fits, room) if fits else None
        if b is None:
            room.append(capacity)
            b = len(room) - 1
        bin_of[i], offset_of[i] = b, capacity - room[b]
        room[b] -= lengths[i]
    return np.array(bin_of), np.array(offset_of), len(room)


_orig_cu = K.packed_cu_seqlens


def _cu_without_tails(lengths, bin_of, offset_of, nbins, capacity):
    cu = list(_orig_cu(lengths, bin_of, offset_of, nbins, capacity))
    ends = {(b + 1) * capacity for b in range(nbins)}
    fills = {(int(bin_of[i]) * capacity + int(offset_of[i]) + int(lengths[i])) for i in range(len(lengths))}
    return np.array([c for c in cu if c == 0 or c in fills or c not in ends])


PACK_MUTANTS = {
    "first_fit": ("bfd_pack", lambda L, c: _variant(L, c, lambda fits, room: fits[0])),
    "worst_fit": ("bfd_pack", lambda L, c: _variant(L, c, lambda fits, room: max(fits, key=lambda b: (room[b], -b)))),
    "ties_to_last_bin": ("bfd_pack", lambda L, c: _variant(L, c, lambda fits, room: min(fits, key=lambda b: (room[b], -b)))),
    "not_sorted": ("bfd_pack", lambda L, c: _variant(L, c, lambda fits, room: min(fits, key=lambda b: (room[b], b)),
                                                     order_key=lambda L_, i: i)),
    "sorted_increasing": ("bfd_pack", lambda L, c: _variant(L, c, lambda fits, room: min(fits, key=lambda b: (room[b], b)),
                                                            order_key=lambda L_, i: (L_[i], i))),
    "equal_lengths_reversed": ("bfd_pack", lambda L, c: _variant(L, c, lambda fits, room: min(fits, key=lambda b: (room[b], b)),
                                                                 order_key=lambda L_, i: (-L_[i], -i))),
    "no_padding_segments": ("packed_cu_seqlens", _cu_without_tails),
}


@pytest.mark.parametrize("name", sorted(PACK_MUTANTS))
def test_pack_pins_catch_mutant(name, monkeypatch):
    attr, fn = PACK_MUTANTS[name]
    monkeypatch.setattr(K, attr, fn)
    caught = []
    for pin in pack_pins.ALL_PACK_PINS:
        try:
            pin(K)
        except Exception:  # any failure of a pin is a detection
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
