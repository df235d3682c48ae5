"""Seeded random configurations of every dense call form against the fp64 oracle.

Each case draws a shape (batch, heads, grouping, head_dim, tokens, capacity), a
call form (host length, device length, per-sequence lengths, paged cache), a
causal flag and a split setting, then compares every output element with the
oracle under the tolerance contract. The cases are fixed by the seed, so a
failure names a reproducible configuration.
"""

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
    rng = np.random.Generator(np.random.PCG64(1000 + i))
    form = ["host", "device", "ragged", "paged"][i % 4]
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 3, 4, 6, 8, 16, 64]))
    Sq = int(rng.choice([1, 1, 2, 3, 4, 8, 16]))
    B = int(rng.integers(1, 6))
    if B * Hkv * G * Sq > 2048:          # keep the oracle's work to about a second
        B = 1
    page = int(rng.choice([32, 64, 128]))
    max_pages = int(rng.integers(1, 40))
    cap = page * max_pages if form == "paged" else int(rng.integers(Sq, 5000))
    causal = bool(rng.integers(0, 2))
    force_chunk = int(rng.choice([0, 0, 32, 96, 1024]))
    num_cus = int(rng.choice([0, 0, 1, 7, 64]))
    lo = Sq if (causal and form == "host") else 0
    lens = [int(x) for x in rng.integers(lo, cap + 1, size=B)]
    if form == "host":
        lens = [max(1, lo, lens[0])] * B
    elif form == "device":
        lens = [lens[0]] * B
    return dict(form=form, B=B, Hq=Hkv * G, Hkv=Hkv, D=D, Sq=Sq, cap=cap, page=page,
                max_pages=max_pages, causal=causal, force_chunk=force_chunk, num_cus=num_cus,
                lens=lens, scale=float(np.float32(1.0 / np.sqrt(D))), seed=2000 + i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(da, i):
    import torch
    c = draw(i)
    B, Hq, Hkv, D, Sq, cap = c["B"], c["Hq"], c["Hkv"], c["D"], c["Sq"], c["cap"]
    sq, sk, sv, _ = W.seeds(c["seed"])
    q = W.normal_bf16(sq, (B, Hq, Sq, D))
    kw = dict(seq_q=Sq, causal=c["causal"], num_cus=c["num_cus"])
    if c["form"] == "paged":
        rng = np.random.Generator(np.random.PCG64(c["seed"]))
        table, num_pages = W.page_table(rng, c["lens"], c["page"], c["max_pages"], 2)
        k = W.normal_bf16(sk, (num_pages, Hkv, c["page"], D))
        v = W.normal_bf16(sv, (num_pages, Hkv, c["page"], D))
        kw.update(page_size=c["page"], max_pages_per_seq=c["max_pages"], num_pages=num_pages)
    else:
        k = W.normal_bf16(sk, (B, Hkv, cap, D))
        v = W.normal_bf16(sv, (B, Hkv, cap, D))
        if c["form"] == "ragged":
            kw.update(ragged=True)
    if c["force_chunk"] and c["form"] in ("host", "device"):
        splits = -(-cap // c["force_chunk"])
        if B * Hq * Sq * splits * (D + 2) * 4 <= (64 << 20):   # bounded workspace
            kw.update(force_chunk=c["force_chunk"])
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, **kw)
    out = torch.full((B, Hq, Sq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = da.workspace_for(plan)
    H.log(f"random case {i}: {c} splits={plan.num_splits_max} wgs={plan.balanced_wgs}")
    dq, dk, dv = H.to_dev(q), H.to_dev(k), H.to_dev(v)
    if c["form"] == "host":
        da.decode_attn_dense(plan, dq, dk, dv, out, c["scale"], c["lens"][0], ws)
    elif c["form"] == "device":
        da.decode_attn_dense_devlen(plan, dq, dk, dv, out, c["scale"],
                                    H.to_dev_i32(c["lens"][:1]), ws)
    elif c["form"] == "ragged":
        da.decode_attn_dense_ragged(plan, dq, dk, dv, out, c["scale"], H.to_dev_i32(c["lens"]),
                                    workspace=ws)
    else:
        da.decode_attn_dense_paged(plan, dq, dk, dv, H.to_dev_i32(table), H.to_dev_i32(c["lens"]),
                                   out, c["scale"], workspace=ws)
    torch.cuda.synchronize()
    got = H.from_dev(out)
    if c["form"] == "paged":
        ref = oracle.dense_paged(q, k, v, table, c["scale"], c["lens"], c["causal"])
    else:
        ref = oracle.dense_ragged(q, k, v, c["scale"], c["lens"], c["causal"])
    H.check_tolerance(got, ref, f"case {i}")
    empty = ~ref.any(axis=-1)
    assert not got[empty].any(), f"case {i}: rows with no visible key must be zeros"
