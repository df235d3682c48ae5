"""KV append / window ring write, written out -- TEST INFRASTRUCTURE ONLY.

The decode step writes the current token's key and value rows into the cache
before attending: at the end of the live prefix for a linear cache (the
fuel-dispatch page "DecodeFlashSpec", field k_len: the live length is the cached
length plus the new token), or at ring slot pos % window for a sliding window
(metrale page "AttnV41", decode_body: the window ring write, with the slot read
on the device). Readings (listed in the design notes): with window == 0 the row
is ``pos``; otherwise it is ``win_base + pos % window``; a position that is
negative or lands outside ``[0, capacity)`` writes nothing.

Several new rows per sequence (``append_rows``: the tokens of a pass are the
last positions of the live prefix) and a paged cache written through a block
table (``append_paged``) compose the same single-row write.

``write_slots`` is the slot-addressed form of the metrale page "DflashScratch"
(field slot_mapping_dev: one 64-bit paged-cache slot per token of the pass,
consumed by a reshape-and-cache write): token n's rows go to slot s = page *
page_size + row of the page pools. Readings: a negative slot is a padding
token and writes nothing; a slot at or past num_pages * page_size writes
nothing (a caller error, never written); two tokens naming one slot are a
caller error (the oracle lets the later token win; the GPU writes each 16-byte
piece from one of them).

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


def append_rows(k_cache: np.ndarray, v_cache: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
                k_lens):
    """Several new rows per sequence at the end of its live prefix: the live
    length counts them (DecodeFlashSpec, field k_len), so with k_new
    [B, Hkv, Sq, D] row t of sequence b goes to cache row k_lens[b] - Sq + t (a
    negative row writes nothing). One append_kv per new row."""
    Sq = k_new.shape[2]
    k, v = k_cache, v_cache
    for t in range(Sq):
        pos = [int(n) - Sq + t for n in k_lens]
        k, v = append_kv(k, v, k_new[:, :, t:t + 1], v_new[:, :, t:t + 1], pos)
    return k, v


def append_paged(k_pages: np.ndarray, v_pages: np.ndarray, block_table: np.ndarray,
                 k_new: np.ndarray, v_new: np.ndarray, k_lens):
    """append_rows through a block table: logical row r of sequence b is row
    r % page_size of page block_table[b, r // page_size] of the pools
    [num_pages, Hkv, page_size, D]. A negative row, or a page id outside the
    pool, writes nothing."""
    k = k_pages.copy()
    v = v_pages.copy()
    num_pages, Hkv, page_size, D = k.shape
    B, _, Sq, _ = k_new.shape
    for b in range(B):
        for t in range(Sq):
            r = int(k_lens[b]) - Sq + t
            if r < 0:
                continue
            pg = int(block_table[b, r // page_size])
            if pg < 0 or pg >= num_pages:
                continue
            k[pg, :, r % page_size, :] = k_new[b, :, t, :]
            v[pg, :, r % page_size, :] = v_new[b, :, t, :]
    return k, v


def write_slots(k_pages: np.ndarray, v_pages: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray,
                slots):
    """Return copies of the page pools [num_pages, Hkv, page_size, D] with token
    n's rows k_rows[n] / v_rows[n] ([N, Hkv, D]) written at slot slots[n]: row
    slots[n] % page_size of page slots[n] // page_size, for every kv head. A
    negative slot or one past the pool writes nothing. One row at a time, in
    token order."""
    k = k_pages.copy()
    v = v_pages.copy()
    num_pages, Hkv, page_size, D = k.shape
    for n in range(k_rows.shape[0]):
        s = int(slots[n])
        if s < 0 or s >= num_pages * page_size:
            continue
        page, row = s // page_size, s % page_size
        for h in range(Hkv):
            k[page, h, row, :] = k_rows[n, h, :]
            v[page, h, row, :] = v_rows[n, h, :]
    return k, v
