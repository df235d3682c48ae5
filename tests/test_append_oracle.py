"""Pins for the KV append oracle (CPU only)."""

import numpy as np

import workloads as W
from oracle.append import append_kv


def test_linear_and_ring_slots():
    _, k, v = W.random_case(90, 3, 2, 2, 8, 10)
    _, kn, vn = W.random_case(91, 3, 2, 2, 8, 1)
    k2, v2 = append_kv(k, v, kn, vn, [4, 0, 9])
    for b, row in enumerate([4, 0, 9]):
        assert np.array_equal(k2[b, :, row], kn[b, :, 0]) and np.array_equal(v2[b, :, row], vn[b, :, 0])
        mask = np.ones(10, bool)
        mask[row] = False
        assert np.array_equal(k2[b][:, mask], k[b][:, mask])   # nothing else changes
    # ring of 4 slots at rows 6..9: positions 5, 8, 11 -> rows 7, 6, 9
    k3, _ = append_kv(k, v, kn, vn, [5, 8, 11], window=4, win_base=6)
    for b, row in enumerate([7, 6, 9]):
        assert np.array_equal(k3[b, :, row], kn[b, :, 0])


def test_out_of_range_positions_write_nothing():
    _, k, v = W.random_case(92, 2, 2, 2, 8, 6)
    _, kn, vn = W.random_case(93, 2, 2, 2, 8, 1)
    k2, v2 = append_kv(k, v, kn, vn, [-1, 6])
    assert np.array_equal(k2, k) and np.array_equal(v2, v)
