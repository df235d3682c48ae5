"""Plan-once decode: the live length in device memory, and HIP-graph capture.

One plan sized for the largest length serves every step; the dense call that
reads k_len from a device int32 is captured once into a graph and replayed
while the length changes between replays (fuel-dispatch page "DecodeFlashSpec",
field k_len: a symbol bound to the live length at each token). The sparse call
is captured with a fixed selection buffer whose contents change between
replays (metrale page "AttnV41", decode_fixed_topk: a constant launch width).
Every replay is checked against the fp64 oracle, with eager work and
synchronisations between replays.
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


LENGTHS = (1, 31, 32, 33, 700, 1025, 4097, 5000)


def _setup(da, seed=70, B=2, Hq=16, Hkv=2, D=128, cap=5000):
    import torch
    q, k, v = W.random_case(seed, B, Hq, Hkv, D, cap)
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap)
    dev = dict(q=H.to_dev(q), k=H.to_dev(k), v=H.to_dev(v),
               out=torch.empty((B, Hq, 1, D), dtype=torch.bfloat16, device="cuda"),
               ws=da.workspace_for(plan),
               klen=torch.zeros(1, dtype=torch.int32, device="cuda"))
    return (q, k, v), plan, dev


def test_device_length_matches_oracle(da):
    import torch
    (q, k, v), plan, d = _setup(da)
    assert plan.num_splits_max > 1
    for kl in LENGTHS:
        H.log(f"device k_len={kl}")
        d["klen"].fill_(kl)
        da.decode_attn_dense_devlen(plan, d["q"], d["k"], d["v"], d["out"], 0.09, d["klen"], d["ws"])
        torch.cuda.synchronize()
        H.check_tolerance(H.from_dev(d["out"]), oracle.dense(q, k, v, 0.09, kl), f"k_len={kl}")


def test_device_length_is_clamped(da):
    import torch
    (q, k, v), plan, d = _setup(da, seed=71)
    for raw, want in ((0, None), (-7, None), (10 ** 9, 5000)):
        d["klen"].fill_(raw)
        da.decode_attn_dense_devlen(plan, d["q"], d["k"], d["v"], d["out"], 0.09, d["klen"], d["ws"])
        torch.cuda.synchronize()
        got = H.from_dev(d["out"])
        if want is None:
            assert not got.any(), f"k_len={raw} must give zeros"
        else:
            H.check_tolerance(got, oracle.dense(q, k, v, 0.09, want), f"k_len={raw}")


def test_dense_graph_replay_follows_device_length(da):
    import torch
    (q, k, v), plan, d = _setup(da, seed=72)
    d["klen"].fill_(5000)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        da.decode_attn_dense_devlen(plan, d["q"], d["k"], d["v"], d["out"], 0.09, d["klen"],
                                    d["ws"])
    eager_out = torch.empty_like(d["out"])
    eager_plan = da.decode_attn_plan(2, 16, 2, 128, 5000, 5000)
    eager_ws = da.workspace_for(eager_plan)
    for kl in LENGTHS + (300, 5000, 2):
        H.log(f"graph replay k_len={kl}")
        d["klen"].fill_(kl)
        g.replay()
        torch.cuda.synchronize()
        H.check_tolerance(H.from_dev(d["out"]), oracle.dense(q, k, v, 0.09, kl),
                          f"replay k_len={kl}")
        # eager work between replays, on the same buffers' neighbours
        da.decode_attn_dense(eager_plan, d["q"], d["k"], d["v"], eager_out, 0.09, kl, eager_ws)
        torch.cuda.synchronize()
        H.check_tolerance(H.from_dev(eager_out), oracle.dense(q, k, v, 0.09, kl), f"eager {kl}")


def test_sparse_graph_replay_follows_selection(da):
    import torch
    B, Hq, D, rows, topk = 3, 32, 128, 3000, 256
    q, k, v = W.random_case(73, B, Hq, 1, D, rows)
    k, v = k[:1], v[:1]
    plan = da.decode_attn_plan(B, Hq, 1, D, rows, topk_max=topk, kv_batch=1)
    dq, dk, dv = H.to_dev(q), H.to_dev(k), H.to_dev(v)
    sel_dev = torch.full((B, topk), -1, dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, 1, D), dtype=torch.bfloat16, device="cuda")
    ws = da.workspace_for(plan)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        da.decode_attn_sparse(plan, dq, dk, dv, sel_dev, topk, out, 0.09, rows, ws)
    rng = np.random.Generator(np.random.PCG64(74))
    for it in range(5):
        n = [int(x) for x in rng.integers(1, topk, size=B)]
        sel = np.full((B, topk), -1, np.int32)
        for b in range(B):
            sel[b, :n[b]] = rng.choice(rows, n[b], replace=False)
        H.log(f"sparse graph replay {it} valid={n}")
        sel_dev.copy_(H.to_dev_i32(sel))
        g.replay()
        torch.cuda.synchronize()
        H.check_tolerance(H.from_dev(out), oracle.sparse(q, k, v, sel, 0.09), f"replay {it}")
