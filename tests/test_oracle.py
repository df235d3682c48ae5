"""Pins for the fp64 oracle (CPU only).

The oracle is trusted only after it agrees with things other than itself:
hand-derived fixtures, closed forms, invariants, and fp64 attention from a
library routine. Each test is chosen so that a plausible mistake in the oracle
(a dropped scale, a sign error, a wrong head or batch index, a transposed
operand, an off-by-one in k_len, no max subtraction, a pad that is not a no-op)
fails at least one of them.
"""

import glob
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bits(x):
    return W.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def f(x):
    return W.bf16_bits_to_f32(x).astype(np.float64)


def rand_case(seed, B, Hq, Hkv, D, cap, std=1.0):
    return W.random_case(seed, B, Hq, Hkv, D, cap, std)


# ---------------------------------------------------------------- fixtures

def _closed_form(name, fx):
    if name == "three_keys_ln2":
        es = math.exp(fx["scale"])
        return [[[[1.0 / (1.0 + 2.0 * es), 0.0]]]]
    if name == "gqa_two_groups":
        return [[[[3.0, 6.0]], [[3.0, 6.0]], [[0.0, 2.0]], [[0.0, 2.0]]]]
    if name == "sparse_pads_duplicates":
        e, e3 = math.e, math.exp(3.0)
        return [[[[(40 * e3 + 20 * e) / (e3 + e)]]], [[[0.0]]],
                [[[(2 * e * 20 + e3 * 40) / (2 * e + e3)]]]]
    raise KeyError(name)


def _arr(x):
    return np.array([[[[float(t) for t in r] for r in h] for h in b] for b in x], dtype=np.float32)


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(GOLDEN, "*.json"))),
                         ids=lambda p: os.path.basename(p)[:-5])
def test_golden_fixture(path):
    name = os.path.basename(path)[:-5]
    fx = json.load(open(path))
    expected = np.array(fx["expected"], dtype=np.float64)
    # The stored numbers match the closed form they were derived from.
    np.testing.assert_allclose(expected, np.array(_closed_form(name, fx)), rtol=1e-15, atol=0)
    q, k, v = bits(_arr(fx["q"])), bits(_arr(fx["k"])), bits(_arr(fx["v"]))
    if fx["kind"] == "dense":
        out = oracle.dense(q, k, v, fx["scale"], fx["k_len"])
    else:
        out = oracle.sparse(q, k, v, np.array(fx["sel"], dtype=np.int32), fx["scale"],
                            fx["k_len"])
    assert np.isfinite(out).all()
    np.testing.assert_allclose(out, expected, rtol=fx["rtol"], atol=fx["atol"])


# ---------------------------------------------------------------- closed forms

def test_single_key_returns_its_value_row():
    q, k, v = rand_case(11, 2, 8, 2, 64, 16)
    out = oracle.dense(q, k, v, 0.125, 1)
    G = 4
    for b in range(2):
        for h in range(8):
            assert np.array_equal(out[b, h, 0], f(v[b, h // G, 0]))


def test_identical_keys_give_mean_of_values():
    q, k, v = rand_case(12, 2, 4, 2, 128, 64)
    k[:, :, :, :] = k[:, :, :1, :]          # every row equals row 0
    for k_len in (1, 7, 64):
        out = oracle.dense(q, k, v, 0.3, k_len)
        for b in range(2):
            for h in range(4):
                ref = f(v[b, h // 2, :k_len]).mean(axis=0)
                np.testing.assert_allclose(out[b, h, 0], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("zero", ["scale", "q"])
def test_zero_scores_give_mean_of_values(zero):
    q, k, v = rand_case(13, 1, 4, 4, 64, 50)
    scale = 0.0 if zero == "scale" else 0.7
    if zero == "q":
        q[:] = 0
    out = oracle.dense(q, k, v, scale, 37)
    for h in range(4):
        np.testing.assert_allclose(out[0, h, 0], f(v[0, h, :37]).mean(axis=0), atol=1e-12, rtol=0)


@pytest.mark.parametrize("s0,s1", [(0.5, -0.25), (1024.0, 1020.0), (-1024.0, -1032.0), (3.0, 3.0)])
def test_two_keys_logistic(s0, s1):
    # q = [a, 0, ...], k0 = [1, 0...] * s0/a, k1 = [1, 0...] * s1/a chosen bf16-exact;
    # scale = 1, so the scores are exactly s0 and s1. Large magnitudes require the
    # maximum to be subtracted before exponentiating.
    D = 64
    q = np.zeros((1, 1, 1, D), np.float32)
    k = np.zeros((1, 1, 2, D), np.float32)
    q[0, 0, 0, 0] = 1.0
    k[0, 0, 0, 0], k[0, 0, 1, 0] = s0, s1
    v = W.normal_bf16(np.random.SeedSequence(14), (1, 1, 2, D))
    assert np.array_equal(f(bits(k)), k)        # the chosen scores are bf16-exact
    out = oracle.dense(bits(q), bits(k), v, 1.0, 2)[0, 0, 0]
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))  # noqa: E731
    ref = sig(s0 - s1) * f(v[0, 0, 0]) + sig(s1 - s0) * f(v[0, 0, 1])
    assert np.isfinite(out).all()
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-15)


def test_scale_multiplies_the_score():
    # Doubling q and halving the scale leaves every score unchanged; doubling the
    # scale alone equals squaring the weights (exp(2s) = exp(s)^2), checked on two keys.
    D = 64
    q = np.zeros((1, 1, 1, D), np.float32)
    q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, 1, 2, D), np.float32)
    k[0, 0, 0, 0], k[0, 0, 1, 0] = 1.5, -0.5
    v = np.zeros((1, 1, 2, D), np.float32)
    v[0, 0, 0, 0], v[0, 0, 1, 0] = 1.0, 0.0
    a = oracle.dense(bits(q), bits(k), bits(v), 0.25, 2)[0, 0, 0, 0]
    b = oracle.dense(bits(2 * q), bits(k), bits(v), 0.125, 2)[0, 0, 0, 0]
    c = oracle.dense(bits(q), bits(k), bits(v), 0.5, 2)[0, 0, 0, 0]
    assert a == b
    w = math.exp(0.25 * 2.0)                   # weight ratio at scale 0.25
    assert abs(a - w / (w + 1)) < 1e-15
    assert abs(c - w * w / (w * w + 1)) < 1e-15


def test_gqa_head_map_probe():
    # Value rows of KV head j in batch b all equal 8*b + j: output row (b, h)
    # must be exactly 8*b + h // G whatever the weights are.
    B, Hq, Hkv, D, cap = 3, 12, 4, 64, 40
    q, k, _ = rand_case(15, B, Hq, Hkv, D, cap)
    v = np.zeros((B, Hkv, cap, D), np.float32)
    for b in range(B):
        for j in range(Hkv):
            v[b, j] = 8 * b + j
    out = oracle.dense(q, k, bits(v), 0.1, 33)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            assert np.allclose(out[b, h, 0], 8 * b + h // G, rtol=1e-14, atol=0)


def test_k_len_bounds_the_prefix():
    # Rows at and beyond k_len hold NaN; the output stays finite and equals the
    # output computed with those rows zeroed.
    q, k, v = rand_case(16, 2, 4, 2, 64, 32)
    kz, vz = k.copy(), v.copy()
    k[:, :, 20:], v[:, :, 20:] = W.BF16_NAN, W.BF16_NAN
    kz[:, :, 20:], vz[:, :, 20:] = 0, 0
    a = oracle.dense(q, k, v, 0.2, 20)
    b = oracle.dense(q, kz, vz, 0.2, 20)
    assert np.isfinite(a).all() and np.array_equal(a, b)
    c = oracle.dense(q, kz, vz, 0.2, 21)   # one more (zero) key changes the result
    assert not np.array_equal(b, c)


# ---------------------------------------------------------------- invariants

def test_joint_permutation_invariance():
    q, k, v = rand_case(17, 2, 8, 2, 128, 300)
    k_len = 257
    a = oracle.dense(q, k, v, 0.088, k_len)
    perm = np.random.Generator(np.random.PCG64(18)).permutation(k_len)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, :k_len] = k[:, :, perm]
    v2[:, :, :k_len] = v[:, :, perm]
    b = oracle.dense(q, k2, v2, 0.088, k_len)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_pads_are_exact_noops():
    B, Hq, D, rows = 3, 8, 128, 500
    q, k, v = rand_case(19, 1, Hq, 1, D, rows)
    q = np.repeat(q, B, axis=0)
    rng = np.random.Generator(np.random.PCG64(20))
    sel = np.stack([rng.choice(rows, size=40, replace=False) for _ in range(B)]).astype(np.int32)
    base = oracle.sparse(q, k, v, sel, 0.09)
    # appended pads
    for topk in (41, 64, 333):
        assert np.array_equal(oracle.sparse(q, k, v, W.repad(sel, topk), 0.09), base)
    # interleaved pads (same valid entries in the same order)
    inter = np.full((B, 120), -1, np.int32)
    inter[:, ::3] = sel
    assert np.array_equal(oracle.sparse(q, k, v, inter, 0.09), base)
    # any negative value is a pad
    inter2 = inter.copy()
    inter2[inter2 < 0] = -7
    assert np.array_equal(oracle.sparse(q, k, v, inter2, 0.09), base)


@pytest.mark.parametrize("Hkv", [1, 4])
def test_dense_equals_sparse_over_the_prefix(Hkv):
    B, Hq, D, cap, k_len = 2, 8, 64, 96, 77
    q, k, v = rand_case(21, B, Hq, Hkv, D, cap)
    dense = oracle.dense(q, k, v, 0.125, k_len)
    sel = np.tile(np.arange(k_len, dtype=np.int32), (B, 1))
    sparse = oracle.sparse(q, k, v, W.repad(sel, 128), 0.125, k_len)  # kv_batch == B
    assert np.array_equal(dense, sparse)


def test_shared_rows_equal_per_token_copies():
    B, Hq, D, rows = 3, 4, 64, 70
    q, k, v = rand_case(22, B, Hq, 1, D, rows)
    k1, v1 = k[:1], v[:1]
    sel = np.stack([np.random.Generator(np.random.PCG64(23 + b)).choice(rows, 30, replace=False)
                    for b in range(B)]).astype(np.int32)
    shared = oracle.sparse(q, k1, v1, sel, 0.1)
    copies = oracle.sparse(q, np.repeat(k1, B, 0), np.repeat(v1, B, 0), sel, 0.1)
    assert np.array_equal(shared, copies)


def test_duplicates_count_with_multiplicity():
    # Listing a row twice equals doubling its weight: with one other row and
    # zero scores, the output is (2 v_a + v_b) / 3.
    D = 64
    q = np.zeros((1, 2, 1, D), np.uint16)
    _, k, v = W.random_case(24, 1, 1, 1, D, 8)
    out = oracle.sparse(q, k, v, np.array([[5, 2, 5, -1]], np.int32), 1.0)
    ref = (2 * f(v[0, 0, 5]) + f(v[0, 0, 2])) / 3
    np.testing.assert_allclose(out[0, 0, 0], ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(out[0, 1, 0], ref, rtol=0, atol=1e-13)


def test_all_pad_row_is_zero_and_bad_index_is_an_error():
    q, k, v = rand_case(25, 2, 2, 1, 64, 16)
    out = oracle.sparse(q, k[:1], v[:1], np.array([[-1, -1], [3, -1]], np.int32), 0.1)
    assert np.array_equal(out[0], np.zeros_like(out[0]))
    assert np.array_equal(out[1, 0, 0], f(v[0, 0, 3]))
    with pytest.raises(ValueError):
        oracle.sparse(q, k[:1], v[:1], np.array([[16, -1], [3, -1]], np.int32), 0.1)
    with pytest.raises(ValueError):
        oracle.sparse(q, k[:1], v[:1], np.array([[9, -1], [3, -1]], np.int32), 0.1, k_len=8)


def test_row_subset_matches_full():
    q, k, v = rand_case(26, 2, 8, 2, 64, 40)
    full = oracle.dense(q, k, v, 0.125, 40).reshape(16, 64)
    rows = np.array([15, 0, 7, 7, 3])
    assert np.array_equal(oracle.dense(q, k, v, 0.125, 40, rows=rows), full[rows])
    assert np.array_equal(oracle.dense(q, k, v, 0.125, 40, threads=1).reshape(16, 64), full)


# ---------------------------------------------------------------- library routine

@pytest.mark.parametrize("B,Hq,Hkv,D,k_len,scale", [
    (1, 8, 8, 64, 300, 0.125),                       # the tiny dense workload
    (2, 32, 8, 128, 512, 1.0 / math.sqrt(128)),      # a reduced GQA workload
    (1, 64, 1, 128, 200, 1.0 / math.sqrt(128)),      # one KV head, 64 query heads
])
def test_matches_torch_fp64_attention(B, Hq, Hkv, D, k_len, scale):
    torch = pytest.importorskip("torch")
    q, k, v = rand_case(27, B, Hq, Hkv, D, k_len + 5)
    out = oracle.dense(q, k, v, scale, k_len)
    G = Hq // Hkv
    tq = torch.from_numpy(f(q))
    tk = torch.from_numpy(f(k[:, :, :k_len])).repeat_interleave(G, dim=1)
    tv = torch.from_numpy(f(v[:, :, :k_len])).repeat_interleave(G, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, scale=float(np.float32(scale))).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)
