"""Padded sparse-attention selection, written out -- TEST INFRASTRUCTURE ONLY.

What the selection holds follows the metrale page "AttnV41" (decode_prep and
decode_prep_role: the window slots first, then the shared index selection, then
-1 up to the fixed launch width of decode_fixed_topk; decode_body: the window
is a ring written at pos % window). Readings where the page is silent (listed
in the design notes):

* the token at 0-based position ``pos`` sees the window positions
  max(0, pos - window + 1) .. pos, oldest first; position p lives in KV row
  ``win_base + p % window``; a negative pos gives an empty window;
* the index selection is the ``k`` candidates 0 .. n_idx-1 with the largest
  scores, ties broken by the lower candidate index, where k = min(k_idx, n_idx,
  topk - window entries) (never negative); scores are ordered by the IEEE 754
  totalOrder predicate (so -0 sorts below +0). The page does not fix the order
  of the rows inside the index selection (it only changes rounding in the
  attention): they are listed in ascending row order;
* every remaining entry is -1.

Plain Python loops and ``sorted``: slow, obviously correct. Pinned by
``tests/test_selection_oracle.py`` (closed forms and numpy's lexsort).
"""

from __future__ import annotations

import numpy as np


def total_order_key(x) -> int:
    """Unsigned integer that orders binary32 values like IEEE 754 totalOrder.

    ``x`` is a binary32 value (a numpy float32 scalar, whose bits are used as
    they are) or its bit pattern as a Python int. totalOrder puts -NaN below
    -inf and +NaN above +inf, orders NaNs of one sign by payload, and puts -0
    below +0: on the bit pattern that is "flip every bit of a negative value,
    set the sign bit of a non-negative one". The bits are never routed through
    binary64, which would quiet a signaling NaN and change its payload."""
    if isinstance(x, (int, np.integer)) and not isinstance(x, bool):
        u = int(x) & 0xFFFFFFFF
    else:
        u = int(np.asarray(x, dtype=np.float32).reshape(()).view(np.uint32))
    return (u ^ 0xFFFFFFFF) if (u & 0x80000000) else (u | 0x80000000)


def build_selection(scores: np.ndarray, pos, n_idx: int, k_idx: int, window: int,
                    win_base: int, topk: int) -> np.ndarray:
    """[B, topk] int32 selection for scores [B, >= n_idx] (float32) and positions [B]."""
    scores = np.asarray(scores, dtype=np.float32)
    bits = scores.view(np.uint32)
    B = scores.shape[0]
    out = np.full((B, topk), -1, dtype=np.int32)
    for b in range(B):
        p = int(pos[b])
        n_win = max(0, min(p + 1, window)) if window > 0 else 0
        n_win = min(n_win, topk)
        row = []
        for j in range(n_win):
            position = p - n_win + 1 + j
            row.append(win_base + position % window)
        k = max(0, min(k_idx, n_idx, topk - n_win))
        keys = [total_order_key(int(bits[b, i])) for i in range(n_idx)]
        ranked = sorted(range(n_idx), key=lambda i: (-keys[i], i))
        row.extend(sorted(ranked[:k]))
        out[b, :len(row)] = row
    return out
