"""CPU work-list of (segment, q-tile) items (oracle; test infrastructure only).

The pages hand ``cu_seqlens`` and ``max_seqlen`` straight to the backends
(tokenspeed page ``mm_encoder_attention.py``, ``_varlen_metadata`` and the
``vision_attn_*`` functions) and show no scheduler.  The library schedules its
attention kernel from a list whose rule is its own, stated here and checked
bit-exactly against the device builder:

1. Segment ``i`` has length ``len_i = cu[i+1] - cu[i]``.
2. Validation (sticky error bits, OR-ed):
   * bit 1 -- ``cu[0] != 0``: the list is empty;
   * bit 2 -- some ``len_i < 0``: that segment is skipped;
   * bit 4 -- some ``len_i > max_seqlen``: that segment is skipped.
3. Segments with ``len_i > 0`` that pass validation are ordered by ``len_i``
   descending, ties by ``i`` ascending (longest first).
4. Each contributes ``(i, j)`` for ``j = 0 .. ceil(len_i / block_m) - 1``,
   ascending.  ``count`` is the number of items.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

ERR_CU0 = 1
ERR_NEGATIVE = 2
ERR_TOO_LONG = 4


def worklist(cu_seqlens, block_m: int,
             max_seqlen: Optional[int] = None) -> Tuple[np.ndarray, int, int]:
    """Return ``(items int32 [count, 2], count, err)``."""
    cu = [int(c) for c in np.asarray(cu_seqlens).reshape(-1)]
    if block_m <= 0:
        raise ValueError("block_m must be positive")
    n = len(cu) - 1
    err = 0
    if n < 0:
        return np.zeros((0, 2), dtype=np.int32), 0, 0
    if cu[0] != 0:
        return np.zeros((0, 2), dtype=np.int32), 0, ERR_CU0
    keep = []
    for i in range(n):
        length = cu[i + 1] - cu[i]
        if length < 0:
            err |= ERR_NEGATIVE
            continue
        if max_seqlen is not None and length > max_seqlen:
            err |= ERR_TOO_LONG
            continue
        if length > 0:
            keep.append((i, length))
    ordered = sorted(keep, key=lambda il: (-il[1], il[0]))
    items = []
    for i, length in ordered:
        ntiles = -(-length // block_m)
        for j in range(ntiles):
            items.append((i, j))
    arr = np.asarray(items, dtype=np.int32).reshape(-1, 2)
    return arr, len(items), err
