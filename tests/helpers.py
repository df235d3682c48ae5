"""Shared helpers for the GPU tests: device transfer, the tolerance contract, caching."""

from __future__ import annotations

import functools
import os
import sys

import numpy as np

import workloads as W

ATOL, RTOL = 2e-2, 1e-2        # |gpu - ref| <= ATOL + RTOL * |ref|, elementwise, bf16 output
REL_L2_MAX = 1e-2              # ||gpu - ref||_2 / ||ref||_2
COS_MIN = 0.999                # per output row


def log(msg: str):
    """Name the case before a GPU step, flushed, so a crash still says which case ran."""
    sys.stderr.write(f"[case] {msg}\n")
    sys.stderr.flush()


def lib_built() -> bool:
    import decode_attention_05_amd as da
    return os.path.exists(da.library_path)


def ensure_built():
    if not lib_built():
        from decode_attention_05_amd import build
        build.build()


# device transfer lives with the input generators (the benchmark uses it too)
to_dev = W.to_dev
to_dev_i32 = W.to_dev_i32
from_dev = W.from_dev


def as_f64(bits: np.ndarray) -> np.ndarray:
    return W.bf16_bits_to_f32(bits).astype(np.float64)


def check_tolerance(got_bits: np.ndarray, ref: np.ndarray, what: str = ""):
    """The tolerance contract: elementwise allclose form, plus relative L2 and per-row cosine."""
    got = as_f64(got_bits).reshape(ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = ATOL + RTOL * np.abs(ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements outside tolerance; "
                           f"max err {err.max():.3e}")
    num = np.linalg.norm((got - ref).ravel())
    den = np.linalg.norm(ref.ravel())
    if den > 0:
        assert num / den <= REL_L2_MAX, f"{what}: relative L2 error {num / den:.3e}"
    g2 = got.reshape(-1, ref.shape[-1])
    r2 = ref.reshape(-1, ref.shape[-1])
    rn = np.linalg.norm(r2, axis=1)
    gn = np.linalg.norm(g2, axis=1)
    nz = rn > 0
    cos = (g2[nz] * r2[nz]).sum(axis=1) / (rn[nz] * np.maximum(gn[nz], 1e-300))
    assert (cos >= COS_MIN).all(), f"{what}: min row cosine {cos.min():.6f}"
    return float(err.max()), float(num / den) if den > 0 else 0.0


@functools.lru_cache(maxsize=2)
def dense_case_inputs(name: str):
    case = W.DENSE_CASES[name]
    return case, W.dense_inputs(case)


@functools.lru_cache(maxsize=2)
def sparse_case_inputs(name: str):
    case = W.SPARSE_CASES[name]
    return case, W.sparse_inputs(case)
