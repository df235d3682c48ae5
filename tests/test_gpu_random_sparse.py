"""Seeded random configurations of the index-selected sparse call against the
fp64 oracle, each also re-padded to two wider launch widths (bit-exact).

Each case draws a grouping G (query heads per kv head), a head dim, whether the
kv rows are shared by all tokens (kv_batch 1) or per token, a launch width that
is not a multiple of the 32-entry tile, a forced selection chunk (including 1
and values that cut tiles) or the plan's own, a compute-unit count to plan for,
and where the -1 pads sit (appended after the valid entries, or interleaved
with them). The valid entries may repeat (they count with multiplicity)."""

import os

import numpy as np
import pytest

import oracle
import workloads as W
from tests import helpers as H

pytestmark = pytest.mark.gpu

# DECODE_ATTN_RANDOM_CASES widens the sweep (the draws are seeded, so a larger
# count runs the default cases and then new ones)
N_CASES = int(os.environ.get("DECODE_ATTN_RANDOM_CASES", "24"))
GROUPS = [1, 2, 3, 6, 8, 64]


@pytest.fixture(scope="module")
def da():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    H.ensure_built()
    import decode_attention_05_amd as m
    m.library()
    return m


def draw(i):
    rng = np.random.Generator(np.random.PCG64(3000 + i))
    G = GROUPS[i % len(GROUPS)]                  # every grouping several times
    D = [64, 128][(i // len(GROUPS)) % 2]         # both head dims for every grouping
    Hkv = int(rng.choice([1, 2, 4])) if G < 64 else 1
    B = int(rng.integers(1, 5))
    kv_batch = 1 if (i % 3 == 0 or B == 1) else B
    cap = int(rng.integers(64, 6000))
    k_len = int(rng.integers(1, cap + 1))
    topk = int(rng.integers(1, 700))
    if topk % 32 == 0:
        topk += 1 + int(rng.integers(0, 30))
    topk_max = 2 * topk + 37                      # the widest re-padding
    force_chunk = [0, 1, 48, 96, topk_max][i % 5]
    num_cus = [0, 1, 7, 64][(i // 5) % 4]
    interleaved = bool(i % 2)
    sel = np.full((B, topk), -1, np.int32)
    for b in range(B):
        n = int(rng.integers(0, topk + 1)) if b else topk        # token 0 is full
        vals = rng.integers(0, k_len, size=n)                      # duplicates allowed
        pos = np.sort(rng.choice(topk, size=n, replace=False)) if interleaved else np.arange(n)
        sel[b, pos] = vals
    return dict(G=G, D=D, Hkv=Hkv, B=B, kv_batch=kv_batch, cap=cap, k_len=k_len, topk=topk,
                topk_max=topk_max, force_chunk=force_chunk, num_cus=num_cus,
                interleaved=interleaved, sel=sel, seed=4000 + i,
                scale=float(np.float32(1.0 / np.sqrt(D))))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_sparse_case(da, i):
    import torch
    c = draw(i)
    B, Hkv, D = c["B"], c["Hkv"], c["D"]
    Hq = Hkv * c["G"]
    sq, sk, sv, _ = W.seeds(c["seed"])
    q = W.normal_bf16(sq, (B, Hq, 1, D))
    k = W.normal_bf16(sk, (c["kv_batch"], Hkv, c["cap"], D))
    v = W.normal_bf16(sv, (c["kv_batch"], Hkv, c["cap"], D))
    plan = da.decode_attn_plan(B, Hq, Hkv, D, c["cap"], topk_max=c["topk_max"],
                               kv_batch=c["kv_batch"], force_chunk=c["force_chunk"],
                               num_cus=c["num_cus"])
    ws = da.workspace_for(plan)
    dq, dk, dv = H.to_dev(q), H.to_dev(k), H.to_dev(v)
    desc = {x: c[x] for x in c if x != "sel"}
    H.log(f"random sparse case {i}: {desc} chunk={plan.chunk} splits={plan.num_splits_max}")
    outs = []
    for width in (c["topk"], c["topk"] + 37, c["topk_max"]):
        sel = W.repad(c["sel"], width)
        out = torch.full((B, Hq, 1, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        da.decode_attn_sparse(plan, dq, dk, dv, H.to_dev_i32(sel), width, out, c["scale"],
                              c["k_len"], ws)
        torch.cuda.synchronize()
        outs.append(H.from_dev(out))
    ref = oracle.sparse(q, k, v, c["sel"], c["scale"], c["k_len"])
    H.check_tolerance(outs[0], ref, f"sparse case {i}")
    empty = (c["sel"] < 0).all(axis=1)
    assert not outs[0][empty].any(), f"case {i}: a token with no valid entry must get zeros"
    for j, o in enumerate(outs[1:], 1):
        assert np.array_equal(o, outs[0]), f"case {i}: re-padded width {j} changed the output"
