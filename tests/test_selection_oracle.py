"""Pins for the selection oracle (CPU only): closed forms and a library sort."""

import numpy as np
import pytest

from oracle.selection import build_selection, total_order_key


def test_total_order_key_orders_like_floats():
    vals = [-np.inf, -3.5, -1.0, -1e-30, -0.0, 0.0, 1e-30, 1.0, 2.0, np.inf]
    keys = [total_order_key(v) for v in vals]
    assert keys == sorted(keys) and len(set(keys)) == len(keys)


def test_window_only_closed_form():
    # window 4 at base 100: position 9 sees positions 6..9 -> rows 100 + (6..9) % 4
    sel = build_selection(np.zeros((1, 10), np.float32), [9], 10, 0, 4, 100, 8)
    assert sel.tolist() == [[102, 103, 100, 101, -1, -1, -1, -1]]
    # early positions see fewer slots; a negative position sees none
    sel = build_selection(np.zeros((3, 1), np.float32), [0, 2, -1], 1, 0, 4, 100, 5)
    assert sel.tolist() == [[100, -1, -1, -1, -1], [100, 101, 102, -1, -1],
                            [-1, -1, -1, -1, -1]]


def test_index_part_is_top_k_by_score_listed_by_row():
    s = np.array([[0.5, 3.0, -1.0, 3.0, 2.0, 7.0]], np.float32)
    sel = build_selection(s, [0], 6, 4, 0, 0, 6)
    assert sel.tolist() == [[1, 3, 4, 5, -1, -1]]   # rows of 7, 3, 3, 2, ascending
    # a tie at the cut goes to the lower index: of the two 3.0s only row 1 fits
    assert build_selection(s, [0], 6, 2, 0, 0, 6).tolist() == [[1, 5, -1, -1, -1, -1]]


def test_width_limits_the_index_part():
    s = np.arange(10, dtype=np.float32)[None, :]
    sel = build_selection(s, [5], 10, 8, 3, 50, 6)
    # 3 window rows (positions 3, 4, 5 -> rows 50 + p % 3), then 6 - 3 = 3 best indices
    assert sel.tolist() == [[50, 51, 52, 7, 8, 9]]


def test_k_larger_than_candidates():
    s = np.array([[1.0, 2.0]], np.float32)
    assert build_selection(s, [0], 2, 5, 0, 0, 4).tolist() == [[0, 1, -1, -1]]


@pytest.mark.parametrize("seed", [1, 2])
def test_matches_numpy_lexsort(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    B, n, k = 3, 3000, 200
    s = rng.standard_normal((B, n), dtype=np.float32)
    s[:, ::7] = np.round(s[:, ::7])           # plenty of ties
    pos = [10, 500, 63]
    sel = build_selection(s, pos, n, k, 64, n, 320)
    for b in range(B):
        order = np.lexsort((np.arange(n), -s[b].astype(np.float64)))[:k]
        n_win = min(pos[b] + 1, 64)
        assert sel[b, n_win:n_win + k].tolist() == sorted(order.tolist())
        assert (sel[b, n_win + k:] == -1).all()
        win = [n + p % 64 for p in range(pos[b] - n_win + 1, pos[b] + 1)]
        assert sel[b, :n_win].tolist() == win


# IEEE 754 totalOrder on binary32, written as bit patterns in ascending order
# (the standard's list: negative NaNs by decreasing payload, -inf, negative
# finites by decreasing magnitude, -0, +0, positive finites, +inf, positive
# NaNs by increasing payload; signaling NaNs have the quiet bit clear).
TOTAL_ORDER_ASCENDING = [
    0xFFFFFFFF,  # -qNaN, largest payload
    0xFFC00001,  # -qNaN
    0xFFC00000,  # -qNaN (the default negative NaN)
    0xFFBFFFFF,  # -sNaN, largest payload
    0xFF800001,  # -sNaN, smallest payload
    0xFF800000,  # -inf
    0xFF7FFFFF,  # -max finite
    0xBF800000,  # -1.0
    0x80800000,  # -smallest normal
    0x80000001,  # -smallest subnormal
    0x80000000,  # -0
    0x00000000,  # +0
    0x00000001,  # +smallest subnormal
    0x00800000,  # +smallest normal
    0x3F800000,  # 1.0
    0x7F7FFFFF,  # +max finite
    0x7F800000,  # +inf
    0x7F800001,  # +sNaN, smallest payload
    0x7FBFFFFF,  # +sNaN, largest payload
    0x7FC00000,  # +qNaN (the default NaN)
    0x7FC00001,  # +qNaN
    0x7FFFFFFF,  # +qNaN, largest payload
]


def as_f32(bit_list):
    return np.array(bit_list, np.uint32).view(np.float32)


def test_total_order_key_follows_the_standard_list_including_nans():
    keys = [total_order_key(u) for u in TOTAL_ORDER_ASCENDING]
    assert all(a < b for a, b in zip(keys, keys[1:]))
    # the same ranks from float32 scalars (bits used as they are, signaling NaNs
    # included: a round trip through binary64 would quiet them)
    vals = as_f32(TOTAL_ORDER_ASCENDING)
    assert [total_order_key(vals[i]) for i in range(len(vals))] == keys


def test_selection_ranks_signed_zeros_by_total_order():
    # a plain float comparison calls -0 and +0 equal and would keep the lower row
    assert build_selection(as_f32([[0x80000000, 0x00000000]]), [0], 2, 1, 0, 0, 1).tolist() == [[1]]
    assert build_selection(as_f32([[0x00000000, 0x80000000]]), [0], 2, 1, 0, 0, 1).tolist() == [[0]]


def test_selection_ranks_nans_beyond_the_infinities():
    inf, ninf, nan, nnan = 0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00000
    sel = lambda bits, k: build_selection(as_f32([bits]), [0], len(bits), k, 0, 0, k).tolist()[0]  # noqa: E731
    assert sel([inf, nan], 1) == [1]          # +NaN outranks +inf
    assert sel([nan, inf], 1) == [0]
    assert sel([nnan, ninf], 1) == [1]        # -NaN ranks below -inf
    assert sel([ninf, nnan], 1) == [0]
    # payloads: the larger +NaN payload wins; a signaling +NaN ranks below every quiet one
    assert sel([0x7F800002, 0x7FC00000, 0x7F800001], 1) == [1]
    assert sel([0x7FC00001, 0x7FC00002], 1) == [1]
    assert sel([0xFFC00002, 0xFFC00001], 1) == [1]


def test_selection_of_a_shuffled_total_order_list():
    # every cut k of a shuffled copy of the standard's list keeps exactly the k
    # patterns that come last in it
    rng = np.random.Generator(np.random.PCG64(3))
    n = len(TOTAL_ORDER_ASCENDING)
    perm = rng.permutation(n)
    bits = [TOTAL_ORDER_ASCENDING[i] for i in perm]      # row r holds rank perm[r]
    scores = as_f32([bits])
    for k in range(n + 1):
        want = sorted(r for r in range(n) if perm[r] >= n - k)
        got = build_selection(scores, [0], n, k, 0, 0, max(k, 1)).tolist()[0][:k]
        assert got == want, k
