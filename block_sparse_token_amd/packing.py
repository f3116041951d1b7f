"""Host-side batch layouts for comparing packing against padding.

Prepacking summary ("Key design", "Technical framework"): prompts of mixed
lengths waste compute when each is padded to the longest one; packing
several prompts into one row (a bin-packing problem) and masking across
them removes most of that padding.  The operator's native layout already
packs every prompt back to back (cu_seqlens), with no padding at all; these
helpers build the two layouts it is compared with:

* ``padded_lengths``: every prompt padded to the longest prompt;
* ``bin_pack_rows``: prompts placed into rows of a fixed capacity by
  first-fit decreasing (largest prompt first, into the first row with room),
  each row then padded to the capacity.

Pure host logic on lengths; nothing here touches the GPU.
"""
from __future__ import annotations


def padded_lengths(lengths):
    """Each prompt padded to the longest: (segment lengths, pad tokens)."""
    L = max(lengths)
    return [L] * len(lengths), sum(L - n for n in lengths)


def bin_pack_rows(lengths, capacity):
    """First-fit decreasing: a list of rows, each a list of prompt indices,
    every row's lengths summing to at most ``capacity``.  Ties in length keep
    the lower index first, so the result is deterministic."""
    if capacity <= 0:
        raise ValueError("capacity must be positive")
    if any(n > capacity or n <= 0 for n in lengths):
        raise ValueError("every prompt needs 1..capacity tokens")
    order = sorted(range(len(lengths)), key=lambda i: (-lengths[i], i))
    rows, free = [], []
    for i in order:
        for r in range(len(rows)):
            if free[r] >= lengths[i]:
                rows[r].append(i)
                free[r] -= lengths[i]
                break
        else:
            rows.append([i])
            free.append(capacity - lengths[i])
    return rows


def bin_packed_segments(lengths, capacity):
    """Segments of the bin-packed layout in row order: each row's prompts,
    then one padding segment filling the row to ``capacity`` (absent when
    the row is full).  Returns (segment lengths, is_padding flags, pad
    tokens, number of rows)."""
    rows = bin_pack_rows(lengths, capacity)
    segs, pad_flags, pad = [], [], 0
    for row in rows:
        used = 0
        for i in row:
            segs.append(lengths[i])
            pad_flags.append(False)
            used += lengths[i]
        if used < capacity:
            segs.append(capacity - used)
            pad_flags.append(True)
            pad += capacity - used
    return segs, pad_flags, pad, len(rows)
