"""fp64 CPU oracle for single-token decode attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The library path never does, and this
package imports nothing from it.

The arithmetic lives in ``decode_oracle.c`` (plain C, fp64, the definition of
softmax attention written out; see the header of that file for the readings it
takes). This module compiles it with gcc and marshals numpy arrays into it.

The multi-token, ragged and paged forms (``dense_tokens``, ``dense_ragged``,
``dense_paged``) are compositions of ``dense``: one call per token and
sequence over the rows that token sees, pages gathered back into rows first.
They are pinned by ``tests/test_ragged_oracle.py`` and
``tests/test_tokens_oracle.py``.

Pinned by ``tests/test_oracle.py`` against closed forms and invariants (one
key returns its value row; identical keys return the mean of V; a zero scale
returns the mean; two keys follow the logistic closed form; the GQA head map;
permutation invariance; -1 pads change nothing; dense equals sparse over the
full prefix; fp64 attention from torch on the CPU as a library routine).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "decode_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math). Returns the .so path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        lib.oracle_dense.argtypes = [p, p, p, p, i32, i32, i32, i32, i64, i64,
                                     ctypes.c_float, p, i64, ctypes.c_int]
        lib.oracle_dense.restype = ctypes.c_int
        lib.oracle_sparse.argtypes = [p, p, p, p, i32, p, i32, i32, i32, i32, i32, i64, i64,
                                      ctypes.c_float, p, i64, ctypes.c_int]
        lib.oracle_sparse.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _bits(a, ndim):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16 or a.ndim != ndim:
        raise TypeError(f"expected uint16 bfloat16 bits with {ndim} dims, got {a.dtype} {a.shape}")
    return a


def _rows(rows, total):
    if rows is None:
        return None, total
    r = np.ascontiguousarray(rows, dtype=np.int64)
    if r.ndim != 1 or (r.size and (r.min() < 0 or r.max() >= total)):
        raise ValueError("rows must be flattened b*Hq+h indices in range")
    return r, r.size


def dense(q, k, v, scale: float, k_len: int, rows=None, threads: int | None = None):
    """fp64 attention of q [B,Hq,1,D] over k/v [B,Hkv,capacity,D] rows [0,k_len).

    Returns fp64 [B,Hq,1,D], or [len(rows), D] when ``rows`` (flattened
    b*Hq+h) is given.
    """
    q, k, v = _bits(q, 4), _bits(k, 4), _bits(v, 4)
    B, Hq, Sq, D = q.shape
    Bk, Hkv, cap, Dk = k.shape
    if Sq != 1 or Bk != B or Dk != D or v.shape != k.shape:
        raise ValueError("shape mismatch")
    r, n = _rows(rows, B * Hq)
    out = np.empty((n, D), dtype=np.float64)
    rc = _load().oracle_dense(q.ctypes.data, k.ctypes.data, v.ctypes.data, out.ctypes.data,
                              B, Hq, Hkv, D, cap, int(k_len), float(np.float32(scale)),
                              None if r is None else r.ctypes.data, n,
                              threads or default_threads())
    if rc:
        raise ValueError(f"oracle_dense failed with code {rc}")
    return out.reshape(B, Hq, 1, D) if r is None else out


def sparse(q, k, v, sel, scale: float, k_len: int | None = None, rows=None,
           threads: int | None = None):
    """fp64 attention of q [B,Hq,1,D] over the rows named by sel [B,topk].

    k/v are [kv_batch,Hkv,capacity,D] with kv_batch 1 (shared) or B. Negative
    entries are pads. ``k_len`` bounds the usable rows (default: capacity).
    """
    q, k, v = _bits(q, 4), _bits(k, 4), _bits(v, 4)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    B, Hq, Sq, D = q.shape
    kvb, Hkv, cap, Dk = k.shape
    if Sq != 1 or Dk != D or v.shape != k.shape or sel.ndim != 2 or sel.shape[0] != B:
        raise ValueError("shape mismatch")
    topk = sel.shape[1]
    r, n = _rows(rows, B * Hq)
    out = np.empty((n, D), dtype=np.float64)
    rc = _load().oracle_sparse(q.ctypes.data, k.ctypes.data, v.ctypes.data, sel.ctypes.data,
                               topk, out.ctypes.data, B, Hq, Hkv, D, kvb, cap,
                               int(cap if k_len is None else k_len), float(np.float32(scale)),
                               None if r is None else r.ctypes.data, n,
                               threads or default_threads())
    if rc:
        raise ValueError(f"oracle_sparse failed with code {rc}")
    return out.reshape(B, Hq, 1, D) if r is None else out


def visible_keys(k_len: int, seq_q: int, t: int, causal: bool) -> int:
    """Keys visible to query token t of seq_q when the live prefix k_len already
    counts the seq_q new tokens (DecodeFlashSpec, field k_len: cached length plus
    the new tokens). Causal: token t sits at position k_len - seq_q + t and sees
    rows [0, k_len - seq_q + t + 1); otherwise every token sees [0, k_len)."""
    return max(0, k_len - (seq_q - 1 - t)) if causal else max(0, k_len)


def dense_tokens(q, k, v, scale: float, k_len: int, causal: bool = True,
                 threads: int | None = None):
    """q [B,Hq,Sq,D] against k/v [B,Hkv,capacity,D]: token t attends rows
    [0, visible_keys(k_len, Sq, t, causal)); an empty prefix gives zeros. The
    single-token oracle, one token at a time."""
    q = _bits(q, 4)
    B, Hq, Sq, D = q.shape
    out = np.zeros((B, Hq, Sq, D), dtype=np.float64)
    for t in range(Sq):
        n = visible_keys(int(k_len), Sq, t, causal)
        if n > 0:
            out[:, :, t:t + 1] = dense(q[:, :, t:t + 1], k, v, scale, n, threads=threads)
    return out


def dense_ragged(q, k, v, scale: float, k_lens, causal: bool = True,
                 threads: int | None = None):
    """Dense attention where sequence b attends rows [0, k_lens[b]) of its own
    cache (a length of 0 gives zeros; with several query tokens, token t sees
    visible_keys of them). The token oracle, one sequence at a time."""
    q = _bits(q, 4)
    B, Hq, Sq, D = q.shape
    out = np.zeros((B, Hq, Sq, D), dtype=np.float64)
    for b in range(B):
        out[b] = dense_tokens(q[b:b + 1], k[b:b + 1], v[b:b + 1], scale, int(k_lens[b]), causal,
                              threads=threads)[0]
    return out


def unpage(pages, block_table, n_rows: int):
    """Contiguous [B, Hkv, n_rows, D] cache from pages [num_pages, Hkv, page_size, D]
    through block_table [B, max_pages]: logical row j of sequence b is row
    j % page_size of page block_table[b, j // page_size]. Rows whose page entry is
    negative are left as zeros (they lie past the sequence's length)."""
    pages = np.asarray(pages)
    num_pages, Hkv, page_size, D = pages.shape
    B = block_table.shape[0]
    out = np.zeros((B, Hkv, n_rows, D), dtype=pages.dtype)
    for b in range(B):
        for j0 in range(0, n_rows, page_size):
            pg = int(block_table[b, j0 // page_size])
            if pg < 0:
                continue
            n = min(page_size, n_rows - j0)
            out[b, :, j0:j0 + n] = pages[pg, :, :n]
    return out


def dense_paged(q, k_pages, v_pages, block_table, scale: float, k_lens, causal: bool = True,
                threads: int | None = None):
    """Attention over a paged cache: the pages gathered into contiguous rows,
    then the ragged dense oracle."""
    page_size = k_pages.shape[2]
    n_rows = block_table.shape[1] * page_size
    k = unpage(k_pages, block_table, n_rows)
    v = unpage(v_pages, block_table, n_rows)
    return dense_ragged(q, k, v, scale, k_lens, causal, threads=threads)
