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


def test_slot_writes_closed_form():
    from oracle.append import write_slots
    num_pages, Hkv, page, D = 3, 2, 4, 8
    _, k, v = W.random_case(98, num_pages, 2, Hkv, D, page)      # pools [3, 2, 4, 8]
    sq, sk, sv, _ = W.seeds(99)
    kr = W.normal_bf16(sk, (5, Hkv, D))
    vr = W.normal_bf16(sv, (5, Hkv, D))
    slots = np.array([5, -1, 0, 11, 12], np.int64)   # 12 = 3 pages * 4 rows: past the pool
    k2, v2 = write_slots(k, v, kr, vr, slots)
    placed = {(1, 1): 0, (0, 0): 2, (2, 3): 3}        # (page, row) -> token
    for pg in range(num_pages):
        for r in range(page):
            n = placed.get((pg, r))
            want_k = k[pg, :, r] if n is None else kr[n]
            want_v = v[pg, :, r] if n is None else vr[n]
            assert np.array_equal(k2[pg, :, r], want_k) and np.array_equal(v2[pg, :, r], want_v)


def test_slot_writes_equal_the_block_table_writes():
    from oracle.append import append_paged, write_slots
    B, Hkv, page, max_pages, D, Sq = 3, 2, 4, 3, 8, 2
    num_pages = 10
    _, k, v = W.random_case(100, num_pages, 2, Hkv, D, page)
    sq, sk, sv, _ = W.seeds(101)
    kn = W.normal_bf16(sk, (B, Hkv, Sq, D))
    vn = W.normal_bf16(sv, (B, Hkv, Sq, D))
    table = np.array([[7, 2, 9], [0, 5, -1], [3, 99, 4]], np.int32)   # 99: outside the pool
    lens = [10, 1, 6]
    want = append_paged(k, v, table, kn, vn, lens)
    # the slot of token t of sequence b, written out from the table (-1 where
    # append_paged writes nothing)
    slots = []
    for b in range(B):
        for t in range(Sq):
            r = lens[b] - Sq + t
            pg = int(table[b, r // page]) if r >= 0 else -1
            slots.append(pg * page + r % page if 0 <= pg < num_pages else -1)
    rows_k = np.ascontiguousarray(kn.transpose(0, 2, 1, 3).reshape(B * Sq, Hkv, D))
    rows_v = np.ascontiguousarray(vn.transpose(0, 2, 1, 3).reshape(B * Sq, Hkv, D))
    got = write_slots(k, v, rows_k, rows_v, np.array(slots, np.int64))
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])


def test_slot_writes_into_a_contiguous_cache():
    # a contiguous cache [B, Hkv, capacity, D] is a pool of B pages of `capacity`
    # rows: slot b * capacity + pos is the single-row append at pos
    from oracle.append import write_slots
    _, k, v = W.random_case(102, 3, 2, 2, 8, 10)
    _, kn, vn = W.random_case(103, 3, 2, 2, 8, 1)
    pos = [4, 0, 9]
    want = append_kv(k, v, kn, vn, pos)
    slots = np.array([b * 10 + p for b, p in enumerate(pos)], np.int64)
    got = write_slots(k, v, kn[:, :, 0], vn[:, :, 0], slots)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])


def test_slot_writes_of_no_tokens_change_nothing():
    from oracle.append import write_slots
    _, k, v = W.random_case(104, 2, 2, 2, 8, 4)
    got = write_slots(k, v, np.zeros((0, 2, 8), np.uint16), np.zeros((0, 2, 8), np.uint16),
                      np.zeros(0, np.int64))
    assert np.array_equal(got[0], k) and np.array_equal(got[1], v)
