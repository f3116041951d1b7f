"""Host-side packing layouts (block_sparse_token_amd/packing.py): validity,
first-fit-decreasing behaviour on hand-worked cases, and its known bound
against the optimum found by brute force on tiny instances."""
import itertools

import numpy as np
import pytest

from block_sparse_token_amd import packing as P


def _optimal_rows(lengths, capacity):
    """Fewest rows by trying every assignment (tiny inputs only)."""
    n = len(lengths)
    for k in range(1, n + 1):
        for assign in itertools.product(range(k), repeat=n):
            load = [0] * k
            for i, r in enumerate(assign):
                load[r] += lengths[i]
            if max(load) <= capacity and len(set(assign)) == k:
                return k
    return n


def test_bin_pack_hand_worked():
    # FFD on [5, 4, 3, 2, 2, 2] into rows of 8: 5+3, 4+2+2, 2
    rows = P.bin_pack_rows([2, 5, 3, 2, 4, 2], 8)
    assert rows == [[1, 2], [4, 0, 3], [5]]
    segs, pad_flags, pad, n = P.bin_packed_segments([2, 5, 3, 2, 4, 2], 8)
    assert segs == [5, 3, 4, 2, 2, 2, 6] and pad_flags == [False] * 6 + [True]
    assert pad == 6 and n == 3


def test_bin_pack_valid_and_within_ffd_bound():
    rng = np.random.default_rng(0)
    for trial in range(60):
        n = int(rng.integers(1, 8))
        cap = int(rng.integers(5, 13))
        lengths = [int(x) for x in rng.integers(1, cap + 1, size=n)]
        rows = P.bin_pack_rows(lengths, cap)
        placed = sorted(i for r in rows for i in r)
        assert placed == list(range(n))
        assert all(sum(lengths[i] for i in r) <= cap for r in rows)
        opt = _optimal_rows(lengths, cap)
        # first-fit decreasing uses at most 11/9 OPT + 6/9 rows
        assert opt <= len(rows) <= (11 * opt + 6) / 9
        segs, flags, pad, nr = P.bin_packed_segments(lengths, cap)
        assert sum(segs) == nr * cap and pad == nr * cap - sum(lengths)
        assert sum(s for s, f in zip(segs, flags) if not f) == sum(lengths)


def test_padded_lengths():
    segs, pad = P.padded_lengths([3, 7, 5])
    assert segs == [7, 7, 7] and pad == 4 + 2


def test_bin_pack_rejects_bad_input():
    with pytest.raises(ValueError):
        P.bin_pack_rows([3, 9], 8)
    with pytest.raises(ValueError):
        P.bin_pack_rows([3], 0)
