"""Pins for the multi-token oracle (several query tokens per sequence), CPU only.

The live prefix k_len counts the new tokens (fuel-dispatch page
"DecodeFlashSpec", field k_len: cached length plus the tokens of this pass);
with causal masking token t of Sq sits at position k_len - Sq + t and sees rows
[0, k_len - Sq + t + 1). The metrale page "AttnV41" (forward) runs m tokens at
start_pos in one pass.
"""

import math

import numpy as np
import pytest

import oracle
import workloads as W


def f64(bits):
    return W.bf16_bits_to_f32(bits).astype(np.float64)


def case(seed, B, Hq, Hkv, Sq, D, cap, std=1.0):
    sq, sk, sv, _ = W.seeds(seed)
    return (W.normal_bf16(sq, (B, Hq, Sq, D), std), W.normal_bf16(sk, (B, Hkv, cap, D), std),
            W.normal_bf16(sv, (B, Hkv, cap, D), std))


def test_visible_keys():
    # k_len 10 with 4 new tokens: positions 6..9 see 7..10 rows
    assert [oracle.visible_keys(10, 4, t, True) for t in range(4)] == [7, 8, 9, 10]
    assert [oracle.visible_keys(10, 4, t, False) for t in range(4)] == [10] * 4
    assert [oracle.visible_keys(2, 4, t, True) for t in range(4)] == [0, 0, 1, 2]


@pytest.mark.parametrize("causal", [True, False])
def test_one_token_is_the_single_token_oracle(causal):
    q, k, v = case(130, 2, 8, 2, 1, 64, 90)
    assert np.array_equal(oracle.dense_tokens(q, k, v, 0.3, 77, causal),
                          oracle.dense(q, k, v, 0.3, 77))


def test_identical_keys_give_prefix_means():
    # every score equal: token t returns the mean of V over the rows it sees
    B, Hq, Hkv, Sq, D, cap = 1, 4, 2, 5, 64, 40
    q, _, v = case(131, B, Hq, Hkv, Sq, D, cap)
    k = np.broadcast_to(W.f32_to_bf16_bits(np.full((1, 1, 1, D), 0.5, np.float32)),
                        (B, Hkv, cap, D)).copy()
    out = oracle.dense_tokens(q, k, v, 0.2, 30, causal=True)
    vf = f64(v)
    for t in range(Sq):
        n = 30 - (Sq - 1 - t)
        want = np.repeat(vf[:, :, :n].mean(axis=2), Hq // Hkv, axis=1)
        np.testing.assert_allclose(out[:, :, t], want, rtol=0, atol=1e-12)
    # a differing last key changes only the last token
    k2 = k.copy()
    k2[:, :, 29] = W.f32_to_bf16_bits(np.full((1, 1, D), -3.0, np.float32))
    out2 = oracle.dense_tokens(q, k2, v, 0.2, 30, causal=True)
    assert np.array_equal(out2[:, :, :Sq - 1], out[:, :, :Sq - 1])
    assert not np.array_equal(out2[:, :, Sq - 1], out[:, :, Sq - 1])


def test_non_causal_tokens_all_see_the_whole_prefix():
    q, k, v = case(132, 2, 8, 4, 3, 64, 60)
    out = oracle.dense_tokens(q, k, v, 0.25, 55, causal=False)
    for t in range(3):
        assert np.array_equal(out[:, :, t:t + 1], oracle.dense(
            np.ascontiguousarray(q[:, :, t:t + 1]), k, v, 0.25, 55))
    # and the causal last token agrees with it
    assert np.array_equal(oracle.dense_tokens(q, k, v, 0.25, 55, causal=True)[:, :, 2],
                          out[:, :, 2])


def test_empty_prefix_gives_zeros():
    q, k, v = case(133, 1, 4, 4, 4, 64, 8)
    out = oracle.dense_tokens(q, k, v, 0.25, 2, causal=True)
    assert not out[:, :, :2].any() and out[:, :, 2:].any()


@pytest.mark.parametrize("B,Hq,Hkv,Sq,D,k_len", [(2, 8, 2, 4, 64, 70), (1, 16, 1, 16, 128, 40),
                                                  (3, 4, 4, 2, 128, 129)])
def test_matches_torch_fp64_attention_with_a_causal_mask(B, Hq, Hkv, Sq, D, k_len):
    torch = pytest.importorskip("torch")
    q, k, v = case(134 + Sq, B, Hq, Hkv, Sq, D, k_len + 3)
    scale = 1.0 / math.sqrt(D)
    out = oracle.dense_tokens(q, k, v, scale, k_len, causal=True)
    G = Hq // Hkv
    tq = torch.from_numpy(f64(q))
    tk = torch.from_numpy(f64(k[:, :, :k_len])).repeat_interleave(G, dim=1)
    tv = torch.from_numpy(f64(v[:, :, :k_len])).repeat_interleave(G, dim=1)
    pos = torch.arange(k_len)[None, :]
    allowed = pos <= (k_len - Sq + torch.arange(Sq))[:, None]     # [Sq, k_len]
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=allowed, scale=float(np.float32(scale))).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_ragged_tokens_are_per_sequence():
    q, k, v = case(140, 3, 8, 2, 3, 64, 50)
    lens = [50, 2, 0]
    out = oracle.dense_ragged(q, k, v, 0.2, lens, causal=True)
    for b in range(3):
        assert np.array_equal(out[b], oracle.dense_tokens(q[b:b + 1], k[b:b + 1], v[b:b + 1],
                                                          0.2, lens[b], True)[0])
    assert not out[2].any() and not out[1, :, 0].any()
