"""Split plans: the log-sum-exp merge of split partials under stress.

A split plan cuts each (batch, kv head, head tile) unit's keys into S ranges;
merging the S partial softmax sums with weights 2^(m_s - M) is an exact
regrouping of the sums that define the attention output (fuel-dispatch page
"DecodeFlashSpec", the decomposed reference arm), so every case is checked
against the fp64 oracle. These tests check that plans can share one workspace,
that many calls in flight on one stream agree bit for bit, the merge's looped
path past 16 splits, and plans with thousands of units. The streaming-read
probe the benchmark compares the kernels with is checked here too: it must
read every word of its buffer.
"""

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


def _out(B, Hq, D, Sq=1):
    import torch
    return torch.full((B, Hq, Sq, D), float("nan"), dtype=torch.bfloat16, device="cuda")


def test_plans_share_one_workspace(da):
    # three plans with different unit counts, split counts and partial layouts
    # take turns on one buffer; each output equals the one from a private buffer
    import torch
    B, Hq, Hkv, D, cap = 4, 32, 4, 128, 6000
    q, k, v = W.random_case(710, B, Hq, Hkv, D, cap)
    dq, dk, dv = H.to_dev(q), H.to_dev(k), H.to_dev(v)
    lens = H.to_dev_i32([6000, 3, 2500, 4100])
    plans = {
        "split6": da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, num_cus=256),
        "split4": da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, num_cus=64),
        "ragged": da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, ragged=True, num_cus=64),
    }

    def call(name, ws, out):
        p = plans[name]
        if name == "ragged":
            da.decode_attn_dense_ragged(p, dq, dk, dv, out, 0.09, lens, workspace=ws)
        else:
            da.decode_attn_dense(p, dq, dk, dv, out, 0.09, 5999, ws)

    private = {}
    for name, p in plans.items():
        out = _out(B, Hq, D)
        call(name, da.workspace_for(p), out)
        private[name] = out
    shared = torch.zeros(max(int(p.workspace_bytes) for p in plans.values()), dtype=torch.uint8,
                         device="cuda")
    for rnd in range(3):
        for name in (["split6", "split4", "ragged"] if rnd % 2 == 0 else
                     ["ragged", "split4", "split6"]):
            out = _out(B, Hq, D)
            H.log(f"shared workspace round {rnd} {name}")
            call(name, shared, out)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), private[name].view(torch.int16)), name
    H.check_tolerance(H.from_dev(private["split6"]), oracle.dense(q, k, v, 0.09, 5999), "shared")


def test_back_to_back_calls_agree(da):
    # many launches in flight on one stream, every one reusing the same
    # workspace: identical bytes each time
    import torch
    B, Hq, Hkv, D, cap = 2, 32, 4, 128, 16384
    q, k, v = W.random_case(720, B, Hq, Hkv, D, cap)
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, num_cus=256)
    assert plan.num_splits_max == 16
    dq, dk, dv = H.to_dev(q), H.to_dev(k), H.to_dev(v)
    ws = da.workspace_for(plan)
    outs = [_out(B, Hq, D) for _ in range(40)]
    H.log("40 back-to-back split calls")
    for o in outs:
        da.decode_attn_dense(plan, dq, dk, dv, o, 0.09, cap, ws)
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0].view(torch.int16), o.view(torch.int16)) for o in outs[1:])
    H.check_tolerance(H.from_dev(outs[0]), oracle.dense(q, k, v, 0.09, cap), "back to back")


def test_more_than_sixteen_splits(da):
    # one unit split 64 ways: the merge's looped path
    import torch
    B, Hq, Hkv, D, cap = 1, 8, 1, 128, 65536
    q, k, v = W.random_case(730, B, Hq, Hkv, D, cap)
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, num_cus=256)
    assert plan.num_splits_max == 64
    out = _out(B, Hq, D)
    ws = da.workspace_for(plan)
    H.log("64 splits")
    da.decode_attn_dense(plan, H.to_dev(q), H.to_dev(k), H.to_dev(v), out, 0.09, 65000, ws)
    torch.cuda.synchronize()
    H.check_tolerance(H.from_dev(out), oracle.dense(q, k, v, 0.09, 65000), "64 splits")


def test_thousands_of_split_units(da):
    # 4160 units (one query head per kv head) of three splits each: 12480
    # workgroups, 4160 rows to merge
    import torch
    B, Hq, Hkv, D, cap = 520, 8, 8, 64, 96
    q, k, v = W.random_case(740, B, Hq, Hkv, D, cap)
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, force_splits=3)
    assert plan.num_splits_max == 3
    ws = da.workspace_for(plan)
    ws.fill_(0xFF)   # the workspace's contents on entry do not matter
    out = _out(B, Hq, D)
    H.log("4160 units, 3 splits")
    da.decode_attn_dense(plan, H.to_dev(q), H.to_dev(k), H.to_dev(v), out, 0.125, 90, ws)
    torch.cuda.synchronize()
    H.check_tolerance(H.from_dev(out), oracle.dense(q, k, v, 0.125, 90), "4160 units")




@pytest.mark.parametrize("nbytes", [16, 4096, 1 << 20, (1 << 20) + 48, (3 << 20) + 16 * 7])
def test_read_probe_reads_every_word(da, nbytes):
    # the streaming-read probe folds every 32-bit word into the sink with xor:
    # whole steps and the share's tail alike (shares of 256 workgroups)
    import numpy as np
    import torch
    rng = np.random.Generator(np.random.PCG64(760 + nbytes))
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    H.log(f"read probe {nbytes} bytes")
    da.decode_attn_read_probe(buf, sink)
    torch.cuda.synchronize()
    expect = np.bitwise_xor.reduce(words) if words.size else np.uint32(0)
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(expect)
