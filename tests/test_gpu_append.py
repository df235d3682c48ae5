"""KV append / ring write against its oracle (exact), and a whole plan-once decode
step -- append at the live end, then attend -- captured once and replayed as the
sequence grows, every step checked against the fp64 oracle."""

import numpy as np
import pytest

import oracle
import workloads as W
from oracle.append import append_kv
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


@pytest.mark.parametrize("D,window,win_base,pos", [
    (128, 0, 0, [5, 0, 63]),
    (64, 0, 0, [1, 2, 3]),
    (128, 16, 40, [3, 17, 1000]),     # ring rows 40 + pos % 16
    (128, 0, 0, [-1, 64, 10]),        # negative / past capacity: nothing written
])
def test_append_matches_oracle(da, D, window, win_base, pos):
    import torch
    _, k, v = W.random_case(100 + D, 3, 1, 2, D, 64)
    _, kn, vn = W.random_case(101 + D, 3, 1, 2, D, 1)
    dk, dv = H.to_dev(k), H.to_dev(v)
    dpos = torch.tensor(pos, dtype=torch.int32, device="cuda")
    H.log(f"append D={D} window={window} pos={pos}")
    da.decode_attn_append_kv(dk, dv, H.to_dev(kn), H.to_dev(vn), dpos, window, win_base)
    torch.cuda.synchronize()
    wk, wv = append_kv(k, v, kn, vn, pos, window, win_base)
    assert np.array_equal(H.from_dev(dk), wk) and np.array_equal(H.from_dev(dv), wv)


def test_decode_loop_in_one_graph(da):
    import torch
    B, Hq, Hkv, D, cap = 2, 16, 2, 128, 4096
    q, k, v = W.random_case(110, B, Hq, Hkv, D, cap)
    start = 2000
    k[:, :, start:] = 0
    v[:, :, start:] = 0
    dq, dk, dv = H.to_dev(q), H.to_dev(k), H.to_dev(v)
    kn_dev = torch.empty((B, Hkv, 1, D), dtype=torch.bfloat16, device="cuda")
    vn_dev = torch.empty_like(kn_dev)
    pos = torch.full((B,), start, dtype=torch.int32, device="cuda")
    klen = torch.full((1,), start + 1, dtype=torch.int32, device="cuda")
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap)
    ws = da.workspace_for(plan)
    out = torch.empty((B, Hq, 1, D), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        da.decode_attn_append_kv(dk, dv, kn_dev, vn_dev, pos)
        da.decode_attn_dense_devlen(plan, dq, dk, dv, out, 0.09, klen, ws)
    hk, hv = k.copy(), v.copy()
    for step in range(6):
        _, kn, vn = W.random_case(111 + step, B, 1, Hkv, D, 1)
        kn_dev.copy_(H.to_dev(kn))
        vn_dev.copy_(H.to_dev(vn))
        pos.fill_(start + step)
        klen.fill_(start + step + 1)
        H.log(f"decode step {step}")
        g.replay()
        torch.cuda.synchronize()
        hk, hv = append_kv(hk, hv, kn, vn, [start + step] * B)
        H.check_tolerance(H.from_dev(out), oracle.dense(q, hk, hv, 0.09, start + step + 1),
                          f"step {step}")
    assert np.array_equal(H.from_dev(dk), hk) and np.array_equal(H.from_dev(dv), hv)
