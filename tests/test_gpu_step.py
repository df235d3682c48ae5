"""The one-call decode pass (write the new K/V rows, then attend) against the oracle.

The pass's new rows belong at the end of each sequence's live prefix, which
counts them (fuel-dispatch page "DecodeFlashSpec", field k_len); the cache may
be paged (the metrale page "DflashScratch" writes its cache through slot
indices). The oracle appends the rows (oracle.append) and attends the result
(the ragged / paged dense oracle); the written cache is compared bit for bit.
"""

import numpy as np
import pytest

import oracle
import workloads as W
from oracle.append import append_kv, append_paged, append_rows
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


def _new_rows(seed, B, Hkv, Sq, D):
    _, sk, sv, _ = W.seeds(seed)
    return W.normal_bf16(sk, (B, Hkv, Sq, D)), W.normal_bf16(sv, (B, Hkv, Sq, D))


def _out(B, Hq, Sq, D):
    import torch
    return torch.full((B, Hq, Sq, D), float("nan"), dtype=torch.bfloat16, device="cuda")


@pytest.mark.parametrize("B,Hq,Hkv,Sq,D,cap,lens,causal", [
    (5, 16, 2, 1, 128, 3000, [3000, 1, 0, 1025, 33], True),
    (4, 32, 8, 4, 128, 2000, [2000, 2, 700, 4], True),
    (3, 64, 1, 1, 128, 1500, [1500, 999, 64], True),      # 4 head tiles per kv head
    (3, 8, 2, 3, 64, 900, [900, 300, 5], False),
])
def test_contiguous_step(da, B, Hq, Hkv, Sq, D, cap, lens, causal):
    import torch
    sq, sk, sv, _ = W.seeds(300 + Sq)
    q = W.normal_bf16(sq, (B, Hq, Sq, D))
    k = W.normal_bf16(sk, (B, Hkv, cap, D))
    v = W.normal_bf16(sv, (B, Hkv, cap, D))
    kn, vn = _new_rows(301 + Sq, B, Hkv, Sq, D)
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, seq_q=Sq, causal=causal, ragged=True)
    dk, dv = H.to_dev(k), H.to_dev(v)
    out = _out(B, Hq, Sq, D)
    H.log(f"step contiguous B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} D={D} lens={lens}")
    da.decode_attn_dense_step(plan, H.to_dev(q), dk, dv, H.to_dev(kn), H.to_dev(vn),
                              H.to_dev_i32(lens), out, 0.09, workspace=da.workspace_for(plan))
    torch.cuda.synchronize()
    ka, va = append_rows(k, v, kn, vn, lens)
    assert np.array_equal(H.from_dev(dk), ka) and np.array_equal(H.from_dev(dv), va)
    ref = oracle.dense_ragged(q, ka, va, 0.09, lens, causal)
    got = H.from_dev(out)
    H.check_tolerance(got, ref, f"step {lens}")
    assert not got[~ref.any(axis=-1)].any()


def test_wide_step_with_wave_runs(da):
    # the one-call pass on a batch wide enough for one run per wave
    import torch
    B, Hq, Hkv, Sq, D, cap = 64, 16, 8, 2, 64, 400
    rng = np.random.Generator(np.random.PCG64(360))
    lens = [int(x) for x in rng.integers(Sq, cap + 1, size=B)]
    sq, sk, sv, _ = W.seeds(361)
    q = W.normal_bf16(sq, (B, Hq, Sq, D))
    k = W.normal_bf16(sk, (B, Hkv, cap, D))
    v = W.normal_bf16(sv, (B, Hkv, cap, D))
    kn, vn = _new_rows(362, B, Hkv, Sq, D)
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, seq_q=Sq, causal=True, ragged=True,
                               num_cus=16)
    assert B * Hkv >= plan.balanced_wgs * 4
    dk, dv = H.to_dev(k), H.to_dev(v)
    out = _out(B, Hq, Sq, D)
    H.log(f"wide step B={B} wgs={plan.balanced_wgs}")
    da.decode_attn_dense_step(plan, H.to_dev(q), dk, dv, H.to_dev(kn), H.to_dev(vn),
                              H.to_dev_i32(lens), out, 0.1, workspace=da.workspace_for(plan))
    torch.cuda.synchronize()
    ka, va = append_rows(k, v, kn, vn, lens)
    assert np.array_equal(H.from_dev(dk), ka) and np.array_equal(H.from_dev(dv), va)
    H.check_tolerance(H.from_dev(out), oracle.dense_ragged(q, ka, va, 0.1, lens, True), "wide step")


def test_step_equals_append_then_attend(da):
    # bit for bit: the same keys in the same order, one kernel fewer
    import torch
    B, Hq, Hkv, D, cap = 4, 32, 8, 128, 4000
    lens = [4000, 17, 2500, 1]
    q, k, v = W.random_case(310, B, Hq, Hkv, D, cap)
    kn, vn = _new_rows(311, B, Hkv, 1, D)
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, ragged=True)
    ws = da.workspace_for(plan)
    dq, dkn, dvn, dl = H.to_dev(q), H.to_dev(kn), H.to_dev(vn), H.to_dev_i32(lens)
    k1, v1, k2, v2 = H.to_dev(k), H.to_dev(v), H.to_dev(k), H.to_dev(v)
    a, b = _out(B, Hq, 1, D), _out(B, Hq, 1, D)
    H.log("step == append + ragged")
    da.decode_attn_dense_step(plan, dq, k1, v1, dkn, dvn, dl, a, 0.09, workspace=ws)
    da.decode_attn_append_kv(k2, v2, dkn, dvn, H.to_dev_i32([n - 1 for n in lens]))
    da.decode_attn_dense_ragged(plan, dq, k2, v2, b, 0.09, dl, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16))
    assert torch.equal(v1.view(torch.int16), v2.view(torch.int16))
    ka, _ = append_kv(k, v, kn, vn, [n - 1 for n in lens])
    assert np.array_equal(H.from_dev(k1), ka)


@pytest.mark.parametrize("Sq,page", [(1, 64), (3, 32)])
def test_paged_step(da, Sq, page):
    import torch
    B, Hq, Hkv, D, max_pages = 4, 16, 4, 128, 24
    lens = [page * max_pages, 40, 1, 700]
    rng = np.random.Generator(np.random.PCG64(320 + Sq))
    table, num_pages = W.page_table(rng, lens, page, max_pages, 3)
    sq, sk, sv, _ = W.seeds(321 + Sq)
    q = W.normal_bf16(sq, (B, Hq, Sq, D))
    kp = W.normal_bf16(sk, (num_pages, Hkv, page, D))
    vp = W.normal_bf16(sv, (num_pages, Hkv, page, D))
    kn, vn = _new_rows(322 + Sq, B, Hkv, Sq, D)
    cap = page * max_pages
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, seq_q=Sq, causal=True, page_size=page,
                               max_pages_per_seq=max_pages, num_pages=num_pages)
    dk, dv = H.to_dev(kp), H.to_dev(vp)
    out = _out(B, Hq, Sq, D)
    H.log(f"step paged Sq={Sq} page={page} lens={lens}")
    da.decode_attn_dense_step(plan, H.to_dev(q), dk, dv, H.to_dev(kn), H.to_dev(vn),
                              H.to_dev_i32(lens), out, 0.09, block_table=H.to_dev_i32(table),
                              workspace=da.workspace_for(plan))
    torch.cuda.synchronize()
    ka, va = append_paged(kp, vp, table, kn, vn, lens)
    assert np.array_equal(H.from_dev(dk), ka) and np.array_equal(H.from_dev(dv), va)
    H.check_tolerance(H.from_dev(out), oracle.dense_paged(q, ka, va, table, 0.09, lens, True),
                      f"paged step Sq={Sq}")


def test_captured_decode_loop(da):
    # one captured step replayed as every sequence grows by one token per replay
    import torch
    B, Hq, Hkv, D, cap = 3, 32, 4, 128, 2048
    q, k, v = W.random_case(330, B, Hq, Hkv, D, cap)
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, ragged=True)
    dq, dk, dv = H.to_dev(q), H.to_dev(k), H.to_dev(v)
    kn_dev = torch.empty((B, Hkv, 1, D), dtype=torch.bfloat16, device="cuda")
    vn_dev = torch.empty_like(kn_dev)
    lens = [700, 1, 2040]
    lens_dev = H.to_dev_i32(lens)
    out = _out(B, Hq, 1, D)
    ws = da.workspace_for(plan)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        da.decode_attn_dense_step(plan, dq, dk, dv, kn_dev, vn_dev, lens_dev, out, 0.09,
                                  workspace=ws)
    kh, vh = k.copy(), v.copy()
    for it in range(5):
        kn, vn = _new_rows(340 + it, B, Hkv, 1, D)
        H.log(f"captured step {it} lens={lens}")
        kn_dev.copy_(H.to_dev(kn))
        vn_dev.copy_(H.to_dev(vn))
        lens_dev.copy_(H.to_dev_i32(lens))
        g.replay()
        torch.cuda.synchronize()
        kh, vh = append_rows(kh, vh, kn, vn, lens)
        H.check_tolerance(H.from_dev(out), oracle.dense_ragged(q, kh, vh, 0.09, lens),
                          f"replay {it}")
        lens = [n + 1 for n in lens]
    assert np.array_equal(H.from_dev(dk), kh) and np.array_equal(H.from_dev(dv), vh)
