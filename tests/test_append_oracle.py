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


def test_rows_at_the_end_of_each_prefix():
    from oracle.append import append_rows
    _, k, v = W.random_case(94, 3, 2, 2, 8, 12)
    sq, sk, sv, _ = W.seeds(95)
    kn = W.normal_bf16(sk, (3, 2, 3, 8))
    vn = W.normal_bf16(sv, (3, 2, 3, 8))
    lens = [12, 5, 2]
    k2, v2 = append_rows(k, v, kn, vn, lens)
    for b, n in enumerate(lens):
        for t in range(3):
            r = n - 3 + t
            if r < 0:
                continue
            assert np.array_equal(k2[b, :, r], kn[b, :, t]) and np.array_equal(v2[b, :, r], vn[b, :, t])
    # sequence 2 (length 2) gets rows 0 and 1; its first new row (row -1) is dropped
    assert np.array_equal(k2[2, :, 2:], k[2, :, 2:])
    # one new row is the single-row append at k_len - 1
    k1, v1 = append_rows(k, v, kn[:, :, :1], vn[:, :, :1], lens)
    k0, v0 = append_kv(k, v, kn[:, :, :1], vn[:, :, :1], [n - 1 for n in lens])
    assert np.array_equal(k1, k0) and np.array_equal(v1, v0)


def test_paged_rows_follow_the_block_table():
    from oracle.append import append_paged, append_rows
    B, Hkv, page, max_pages, D = 2, 2, 4, 3, 8
    _, k, v = W.random_case(96, B, 2, Hkv, D, page * max_pages)
    sq, sk, sv, _ = W.seeds(97)
    kn = W.normal_bf16(sk, (B, Hkv, 2, D))
    vn = W.normal_bf16(sv, (B, Hkv, 2, D))
    to_pages = lambda x: np.ascontiguousarray(  # noqa: E731
        x.reshape(B, Hkv, max_pages, page, D).transpose(0, 2, 1, 3, 4).reshape(B * max_pages, Hkv, page, D))
    from_pages = lambda x: np.ascontiguousarray(  # noqa: E731
        x.reshape(B, max_pages, Hkv, page, D).transpose(0, 2, 1, 3, 4).reshape(B, Hkv, max_pages * page, D))
    table = np.arange(B * max_pages, dtype=np.int32).reshape(B, max_pages)
    lens = [9, 4]
    kp, vp = append_paged(to_pages(k), to_pages(v), table, kn, vn, lens)
    kc, vc = append_rows(k, v, kn, vn, lens)
    assert np.array_equal(from_pages(kp), kc) and np.array_equal(from_pages(vp), vc)
    # a page id outside the pool writes nothing
    bad = table.copy()
    bad[0, 2] = 99
    kp2, _ = append_paged(to_pages(k), to_pages(v), bad, kn, vn, lens)
    assert np.array_equal(kp2[2], to_pages(k)[2])
