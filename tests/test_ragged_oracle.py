"""Pins for the ragged and paged oracle compositions (CPU only)."""

import numpy as np

import oracle
import workloads as W


def test_ragged_is_per_sequence_dense():
    q, k, v = W.random_case(120, 3, 4, 2, 64, 50)
    lens = [50, 1, 0]
    out = oracle.dense_ragged(q, k, v, 0.2, lens)
    assert np.array_equal(out[0], oracle.dense(q[:1], k[:1], v[:1], 0.2, 50)[0])
    assert np.array_equal(out[1, :, 0], np.repeat(W.bf16_bits_to_f32(v[1:2, :, 0]), 2, axis=1)[0]
                          .astype(np.float64))
    assert not out[2].any()


def test_identity_page_table_equals_contiguous():
    q, k, v = W.random_case(121, 2, 4, 2, 64, 128)
    page = 32
    # pages [num_pages, Hkv, page, D] holding the contiguous rows in order
    kp = k.reshape(2, 2, 4, page, 64).transpose(0, 2, 1, 3, 4).reshape(8, 2, page, 64)
    vp = v.reshape(2, 2, 4, page, 64).transpose(0, 2, 1, 3, 4).reshape(8, 2, page, 64)
    table = np.arange(8, dtype=np.int32).reshape(2, 4)
    lens = [128, 77]
    assert np.array_equal(oracle.dense_paged(q, kp, vp, table, 0.1, lens),
                          oracle.dense_ragged(q, k, v, 0.1, lens))
    # shuffling the pages and the table together changes nothing
    perm = np.random.Generator(np.random.PCG64(5)).permutation(8)
    inv = np.argsort(perm)
    assert np.array_equal(oracle.dense_paged(q, kp[perm], vp[perm], inv[table].astype(np.int32),
                                             0.1, lens),
                          oracle.dense_ragged(q, k, v, 0.1, lens))
