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
