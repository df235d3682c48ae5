"""KV append / window ring write, written out -- TEST INFRASTRUCTURE ONLY.

The decode step writes the current token's key and value rows into the cache
before attending: at the end of the live prefix for a linear cache (the
fuel-dispatch page "DecodeFlashSpec", field k_len: the live length is the cached
length plus the new token), or at ring slot pos % window for a sliding window
(metrale page "AttnV41", decode_body: the window ring write, with the slot read
on the device). Readings (listed in the design notes): with window == 0 the row
is ``pos``; otherwise it is ``win_base + pos % window``; a position that is
negative or lands outside ``[0, capacity)`` writes nothing.

Plain numpy indexing, one row at a time. Pinned by ``tests/test_append_oracle.py``.
"""

from __future__ import annotations

import numpy as np


def append_kv(k_cache: np.ndarray, v_cache: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
              pos, window: int = 0, win_base: int = 0):
    """Return copies of the caches [B, Hkv, capacity, D] with token b's rows
    k_new[b, :, 0, :] / v_new[b, :, 0, :] written at its slot."""
    k = k_cache.copy()
    v = v_cache.copy()
    B, Hkv, cap, D = k.shape
    for b in range(B):
        p = int(pos[b])
        if p < 0:
            continue
        row = p if window == 0 else win_base + p % window
        if row < 0 or row >= cap:
            continue
        for h in range(Hkv):
            k[b, h, row, :] = k_new[b, h, 0, :]
            v[b, h, row, :] = v_new[b, h, 0, :]
    return k, v
