"""Several query tokens per sequence (verification rows) against the fp64 oracle.

q and out are [B, Hq, Sq, D] (fuel-dispatch page "DecodeFlashSpec", field q);
the live prefix k_len counts the Sq new tokens (field k_len), and with causal
masking token t sees rows [0, k_len - Sq + 1 + t) (the metrale page "AttnV41",
forward: m tokens at start_pos). Every call form is covered: host length,
device length, one length per sequence, paged cache, and split counts that put
the causal tail across split and run boundaries.
"""

import numpy as np
import pytest

import oracle
import workloads as W
from tests import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def da():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    H.ensure_built()
    import decode_attention_05_amd as m
    m.library()
    return m


def _case(seed, B, Hq, Hkv, Sq, D, cap):
    sq, sk, sv, _ = W.seeds(seed)
    return (W.normal_bf16(sq, (B, Hq, Sq, D)), W.normal_bf16(sk, (B, Hkv, cap, D)),
            W.normal_bf16(sv, (B, Hkv, cap, D)))


def _out(B, Hq, Sq, D):
    import torch
    return torch.full((B, Hq, Sq, D), float("nan"), dtype=torch.bfloat16, device="cuda")


def _check(got, ref, what):
    H.check_tolerance(got, ref, what)
    empty = ~ref.any(axis=-1)             # rows whose prefix is empty must be exact zeros
    assert not got[empty].any(), f"{what}: rows with no visible key must be zeros"


STATIC = [
    # B, Hq, Hkv, Sq, D, capacity, k_len, causal, force_chunk
    (2, 32, 8, 4, 128, 5000, 4097, True, 0),
    (3, 8, 8, 2, 64, 700, 700, True, 0),
    (1, 16, 1, 16, 128, 3000, 2500, True, 0),
    (2, 32, 8, 5, 128, 2048, 1500, False, 0),
    (4, 8, 2, 3, 128, 100, 3, True, 0),
    (2, 16, 2, 16, 128, 1000, 999, True, 32),   # the 16-token tail crosses split edges
    (2, 16, 4, 7, 64, 1000, 333, True, 64),
]


@pytest.mark.parametrize("B,Hq,Hkv,Sq,D,cap,k_len,causal,chunk", STATIC)
def test_host_length(da, B, Hq, Hkv, Sq, D, cap, k_len, causal, chunk):
    import torch
    q, k, v = _case(150 + Sq, B, Hq, Hkv, Sq, D, cap)
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, seq_q=Sq, causal=causal,
                               force_chunk=chunk)
    out = _out(B, Hq, Sq, D)
    H.log(f"tokens host B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} D={D} k_len={k_len} causal={causal} "
          f"S={plan.num_splits_max}")
    da.decode_attn_dense(plan, H.to_dev(q), H.to_dev(k), H.to_dev(v), out, 0.09, k_len,
                         da.workspace_for(plan))
    torch.cuda.synchronize()
    _check(H.from_dev(out), oracle.dense_tokens(q, k, v, 0.09, k_len, causal), f"Sq={Sq}")


def test_one_token_rows_match_the_single_token_call(da):
    # with causal masking, the last token of a pass is the single-token call at k_len
    import torch
    B, Hq, Hkv, Sq, D, cap, k_len = 2, 32, 8, 4, 128, 3000, 2600
    q, k, v = _case(160, B, Hq, Hkv, Sq, D, cap)
    multi = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, seq_q=Sq, causal=True)
    single = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap)
    a, b = _out(B, Hq, Sq, D), _out(B, Hq, 1, D)
    dk, dv = H.to_dev(k), H.to_dev(v)
    H.log("tokens: last row vs single-token call")
    da.decode_attn_dense(multi, H.to_dev(q), dk, dv, a, 0.09, k_len, da.workspace_for(multi))
    da.decode_attn_dense(single, H.to_dev(np.ascontiguousarray(q[:, :, -1:])), dk, dv, b, 0.09,
                         k_len, da.workspace_for(single))
    torch.cuda.synchronize()
    H.check_tolerance(H.from_dev(a)[:, :, -1:], oracle.dense(
        np.ascontiguousarray(q[:, :, -1:]), k, v, 0.09, k_len), "last row")
    H.check_tolerance(H.from_dev(b), oracle.dense(
        np.ascontiguousarray(q[:, :, -1:]), k, v, 0.09, k_len), "single")


def test_device_length(da):
    import torch
    B, Hq, Hkv, Sq, D, cap = 2, 16, 2, 8, 128, 4000
    q, k, v = _case(161, B, Hq, Hkv, Sq, D, cap)
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, seq_q=Sq, causal=True)
    dq, dk, dv = H.to_dev(q), H.to_dev(k), H.to_dev(v)
    ws = da.workspace_for(plan)
    klen = torch.zeros(1, dtype=torch.int32, device="cuda")
    for n in (4000, 3, 8, 1025, 33):
        out = _out(B, Hq, Sq, D)
        H.log(f"tokens device k_len={n}")
        klen.fill_(n)
        da.decode_attn_dense_devlen(plan, dq, dk, dv, out, 0.09, klen, ws)
        torch.cuda.synchronize()
        _check(H.from_dev(out), oracle.dense_tokens(q, k, v, 0.09, n, True), f"k_len={n}")


@pytest.mark.parametrize("Sq,causal,num_cus", [(4, True, 256), (16, True, 3), (3, False, 256),
                                               (2, True, 1)])
def test_ragged(da, Sq, causal, num_cus):
    import torch
    B, Hq, Hkv, D, cap = 6, 16, 4, 128, 3000
    lens = [3000, 0, 1, Sq, 1700, 33]
    q, k, v = _case(170 + Sq, B, Hq, Hkv, Sq, D, cap)
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, seq_q=Sq, causal=causal, ragged=True,
                               num_cus=num_cus)
    out = _out(B, Hq, Sq, D)
    H.log(f"tokens ragged Sq={Sq} causal={causal} wgs={plan.balanced_wgs} lens={lens}")
    da.decode_attn_dense_ragged(plan, H.to_dev(q), H.to_dev(k), H.to_dev(v), out, 0.09,
                                H.to_dev_i32(lens), workspace=da.workspace_for(plan))
    torch.cuda.synchronize()
    _check(H.from_dev(out), oracle.dense_ragged(q, k, v, 0.09, lens, causal), f"ragged Sq={Sq}")


def test_paged(da):
    import torch
    B, Hq, Hkv, Sq, D, page, max_pages = 3, 32, 8, 4, 128, 64, 20
    lens = [1280, 70, 4]
    rng = np.random.Generator(np.random.PCG64(180))
    table, num_pages = W.page_table(rng, lens, page, max_pages, 2)
    sq, sk, sv, _ = W.seeds(181)
    q = W.normal_bf16(sq, (B, Hq, Sq, D))
    kp = W.normal_bf16(sk, (num_pages, Hkv, page, D))
    vp = W.normal_bf16(sv, (num_pages, Hkv, page, D))
    cap = page * max_pages
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, seq_q=Sq, causal=True, page_size=page,
                               max_pages_per_seq=max_pages, num_pages=num_pages)
    out = _out(B, Hq, Sq, D)
    H.log(f"tokens paged Sq={Sq} lens={lens}")
    da.decode_attn_dense_paged(plan, H.to_dev(q), H.to_dev(kp), H.to_dev(vp), H.to_dev_i32(table),
                               H.to_dev_i32(lens), out, 0.09, workspace=da.workspace_for(plan))
    torch.cuda.synchronize()
    _check(H.from_dev(out), oracle.dense_paged(q, kp, vp, table, 0.09, lens, True), "paged")
