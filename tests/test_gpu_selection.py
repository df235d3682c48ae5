"""The on-device selection builder against the selection oracle (exact, integers),
and the built selection feeding the sparse attention, eager and in a HIP graph.
Every case runs both builders: one workgroup per token, and several workgroups
per token with a caller workspace (whose contents on entry are junk)."""

import os

import numpy as np
import pytest

import oracle
import workloads as W
from oracle.selection import build_selection
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


def junk_workspace(da, B, n_idx, k_idx, window, topk, stride):
    import torch
    n = da.decode_attn_select_workspace(B, n_idx, k_idx, window, topk, stride)
    return torch.full((max(n, 16),), 0xAB, dtype=torch.uint8, device="cuda") if n else None


def run_builder(da, scores, pos, n_idx, k_idx, window, win_base, topk, split=False):
    import torch
    # rows padded to a multiple of 4 floats (the builder reads 16-byte vectors)
    B, n = scores.shape
    stride = max(4, (n + 3) // 4 * 4)
    padded = np.full((B, stride), np.nan, np.float32)
    padded[:, :n] = scores
    sc = torch.from_numpy(padded).cuda()
    ps = torch.from_numpy(np.asarray(pos, np.int32)).cuda()
    sel = torch.full((scores.shape[0], topk), 12345, dtype=torch.int32, device="cuda")
    if split:
        ws = junk_workspace(da, B, n_idx, k_idx, window, topk, stride)
        da.decode_attn_build_selection_ws(sc, ps, sel, n_idx, k_idx, window, win_base, ws)
    else:
        da.decode_attn_build_selection(sc, ps, sel, n_idx, k_idx, window, win_base)
    torch.cuda.synchronize()
    return sel.cpu().numpy()


def scores_for(seed, B, n, kind="normal"):
    rng = np.random.Generator(np.random.PCG64(seed))
    s = rng.standard_normal((B, n), dtype=np.float32)
    if kind == "ties":
        s = np.round(s * 2) / 2          # a handful of distinct values
    elif kind == "special":
        s[:, ::97] = np.inf
        s[:, 1::89] = -np.inf
        s[:, 2::83] = 0.0
        s[:, 3::79] = -0.0
        s = with_nan_payloads(s)
    return s.astype(np.float32)


def with_nan_payloads(s):
    """Quiet and signaling NaNs of both signs and several payloads (their order
    under IEEE totalOrder is by sign, then payload bits)."""
    bits = s.astype(np.float32).view(np.uint32).copy()
    for start, step, pattern in ((4, 101, 0x7F800001), (6, 103, 0x7FBFFFFF), (8, 107, 0x7FC00001),
                                 (9, 109, 0xFF800001), (10, 113, 0xFFFFFFFF)):
        bits[:, start::step] = pattern
    return bits.view(np.float32)


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("kind", ["normal", "ties", "special"])
def test_sparse_workload_shapes(da, kind, split):
    # 4 tokens, 65408 index candidates, 1920 chosen, a 128-slot window ring at the
    # top of 65536 rows, launch width 2048.
    B, rows, W_, topk, k = 4, 65536, 128, 2048, 1920
    n_idx = rows - W_
    s = scores_for(80, B, n_idx, kind)
    pos = [200000, 127, 0, 50]
    H.log(f"selection builder kind={kind} split={split}")
    got = run_builder(da, s, pos, n_idx, k, W_, n_idx, topk, split)
    want = build_selection(s, pos, n_idx, k, W_, n_idx, topk)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("B,n_idx,k_idx,window,topk,pos", [
    (2, 5, 10, 0, 8, [0, 3]),            # k larger than the candidates
    (3, 1000, 300, 64, 100, [10, 500, 63]),  # the width cuts the index part
    (2, 3000, 0, 16, 32, [5, 40]),       # window only
    (2, 9000, 4096, 8, 4200, [3, 7]),    # the largest k
    (2, 100, 20, 4, 30, [-1, 2]),        # negative position: no window rows
    (1, 0, 5, 4, 6, [9]),                # no candidates
    (5, 1, 1, 1, 1, [0, 1, 2, 3, 4]),    # width 1: only the newest window row
])
@pytest.mark.parametrize("split", [False, True])
def test_edge_shapes(da, B, n_idx, k_idx, window, topk, pos, split):
    s = scores_for(81 + n_idx, B, max(n_idx, 1))
    got = run_builder(da, s, pos, n_idx, k_idx, window, 7000, topk, split)
    assert np.array_equal(got, build_selection(s, pos, n_idx, k_idx, window, 7000, topk))


@pytest.mark.parametrize("split", [False, True])
def test_built_selection_feeds_sparse_attention(da, split):
    import torch
    case = W.SPARSE_CASES["sparse"]
    _, (q, k, v, _) = H.sparse_case_inputs("sparse")
    n_idx = case.rows - case.window
    s = scores_for(82, case.B, n_idx)
    pos = [70000, 90, 131, 5000]
    sel_ref = build_selection(s, pos, n_idx, 1920, case.window, n_idx, case.topk)
    plan = da.decode_attn_plan(case.B, case.Hq, case.Hkv, case.D, case.rows, topk_max=case.topk,
                               kv_batch=1)
    dq, dk, dv = H.to_dev(q), H.to_dev(k), H.to_dev(v)
    sc = torch.from_numpy(s).cuda()
    ps = torch.from_numpy(np.asarray(pos, np.int32)).cuda()
    sel = torch.empty((case.B, case.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((case.B, case.Hq, 1, case.D), dtype=torch.bfloat16, device="cuda")
    ws = da.workspace_for(plan)
    sws = junk_workspace(da, case.B, n_idx, 1920, case.window, case.topk, n_idx) if split else None

    def build():
        if split:
            da.decode_attn_build_selection_ws(sc, ps, sel, n_idx, 1920, case.window, n_idx, sws)
        else:
            da.decode_attn_build_selection(sc, ps, sel, n_idx, 1920, case.window, n_idx)

    build()
    da.decode_attn_sparse(plan, dq, dk, dv, sel, case.topk, out, case.scale, case.rows, ws)
    torch.cuda.synchronize()
    assert np.array_equal(sel.cpu().numpy(), sel_ref)
    H.check_tolerance(H.from_dev(out), oracle.sparse(q, k, v, sel_ref, case.scale), "built")

    # the same two calls captured once; scores and positions change between replays
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        build()
        da.decode_attn_sparse(plan, dq, dk, dv, sel, case.topk, out, case.scale, case.rows, ws)
    for it in range(3):
        s2 = scores_for(83 + it, case.B, n_idx)
        pos2 = [1000 * it + b for b in range(case.B)]
        sc.copy_(torch.from_numpy(s2).cuda())
        ps.copy_(torch.from_numpy(np.asarray(pos2, np.int32)).cuda())
        H.log(f"selection+attention graph replay {it}")
        g.replay()
        torch.cuda.synchronize()
        ref_sel = build_selection(s2, pos2, n_idx, 1920, case.window, n_idx, case.topk)
        assert np.array_equal(sel.cpu().numpy(), ref_sel)
        H.check_tolerance(H.from_dev(out), oracle.sparse(q, k, v, ref_sel, case.scale),
                          f"replay {it}")


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("k_idx,case", [(3000, "sample misleads"), (1500, "sample agrees"),
                                        (4000, "large k"), (1920, "nan and ties"),
                                        (1920, "top in one part"), (300, "part overflow"),
                                        (1920, "far above the bound"),
                                        (1920, "far above the bound, ties")])
def test_prefiltered_and_fallback_paths(da, k_idx, case, split):
    # The builder first keeps the keys at or above a bound taken from a sample
    # of 256 runs of 8 keys; when fewer than k keys are kept it selects over all
    # keys instead. Giving every sampled key a huge score with k above the
    # sample size keeps only the sample (fewer than k) and forces that path;
    # with k below the sample size the kept keys are exactly the sample.
    B, n, W_, topk = 2, 65408, 0, 4096
    s = scores_for(90 + k_idx, B, n)
    if case in ("sample misleads", "sample agrees"):
        for j in range(256):
            start = (j * (n - 8) // 255) & ~3
            s[:, start:start + 8] = 1.0e6 + j
    elif case == "nan and ties":
        s = np.round(s * 8) / 8
        s[:, 5::301] = np.nan
        s[:, 7::211] = -np.nan
    elif case == "top in one part":
        # every selected key in the last 4096 candidates: that part keeps more
        # than it can hold, and the split builder redoes the token
        s[:, -4096:] += 50.0
    elif case.startswith("far above the bound"):
        # the selected keys sit orders of magnitude above the sample's bound, so
        # the merge's k-th largest key lies past its first digit's range (the
        # radix finish over the open-ended last digit); with ties, several keys
        # share the threshold value
        rng = np.random.Generator(np.random.PCG64(91))
        for b in range(B):
            rows = rng.choice(n, 2000, replace=False)
            vals = 1.0e6 + np.arange(2000, dtype=np.float32)
            if case.endswith("ties"):
                vals = 1.0e6 + (np.arange(2000) // 7).astype(np.float32)
            s[b, rows] = vals
    elif case == "part overflow":
        # a sample that lands on low scores sets a low bound: parts keep too much
        s = np.abs(s)
        for j in range(256):
            start = (j * (n - 8) // 255) & ~3
            s[:, start:start + 8] = -1.0
    pos = [-1] * B
    got = run_builder(da, s, pos, n, k_idx, W_, 0, topk, split)
    want = build_selection(s, pos, n, k_idx, W_, 0, topk)
    assert np.array_equal(got, want), case


# DECODE_ATTN_RANDOM_CASES widens the sweep (the draws are seeded, so a larger
# count runs the default cases and then new ones)
N_RANDOM = int(os.environ.get("DECODE_ATTN_RANDOM_CASES", "16"))


def draw_selection_case(i):
    rng = np.random.Generator(np.random.PCG64(500 + i))
    B = int(rng.integers(1, 5))
    n = int(rng.choice([1, 7, 100, 4095, 8191, 8192, 20000, 65408, 131072]))
    k = int(rng.choice([0, 1, 17, 640, 1920, 4096]))
    window = int(rng.choice([0, 1, 64, 128]))
    topk = int(rng.integers(max(1, window), window + min(k, n) + 64))
    kind = ["normal", "uniform", "ties", "special", "trend", "constant"][i % 6]
    s = rng.standard_normal((B, n)).astype(np.float32)
    if kind == "uniform":
        s = rng.uniform(-1, 1, (B, n)).astype(np.float32)
    elif kind == "ties":
        s = np.round(s * 4) / 4
    elif kind == "special":
        s[:, ::53] = np.inf
        s[:, 3::61] = -np.inf
        s[:, 5::67] = np.nan
        s[:, 7::71] = -0.0
        s = with_nan_payloads(s)
    elif kind == "trend":
        s = (np.arange(n, dtype=np.float32) / n + 0.01 * s).astype(np.float32)
    elif kind == "constant":
        s[:] = 0.5
    pos = [int(x) for x in rng.integers(-1, 2 * max(1, window) + 5, size=B)]
    return dict(B=B, n=n, k=k, window=window, topk=topk, kind=kind, pos=pos), s


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("i", range(N_RANDOM))
def test_random_selections(da, i, split):
    c, s = draw_selection_case(i)
    win_base = c["n"]
    H.log(f"random selection {i} split={split}: {c}")
    got = run_builder(da, s, c["pos"], c["n"], c["k"], c["window"], win_base, c["topk"], split)
    want = build_selection(s, c["pos"], c["n"], c["k"], c["window"], win_base, c["topk"])
    assert np.array_equal(got, want), c


def test_split_workspace_serves_problems_of_several_shapes(da):
    # the split builder's workspace holds nothing between calls: one buffer
    # serves problems of any shape in turn, junk from earlier calls left behind
    import torch
    shapes = [(4, 65408, 1920, 128, 2048), (2, 20000, 300, 0, 300), (7, 131072, 4096, 64, 4160),
              (4, 65408, 1920, 128, 2048)]
    size = max(da.decode_attn_select_workspace(*sh) for sh in shapes)
    ws = torch.full((size,), 0xAB, dtype=torch.uint8, device="cuda")
    for i, (B, n, k, W_, topk) in enumerate(shapes):
        s = scores_for(600 + i, B, n)
        pos = [13 * b + i for b in range(B)]
        sc = torch.from_numpy(s).cuda()
        ps = torch.from_numpy(np.asarray(pos, np.int32)).cuda()
        sel = torch.full((B, topk), 777, dtype=torch.int32, device="cuda")
        H.log(f"split builder shape {i}: B={B} n={n} k={k}")
        da.decode_attn_build_selection_ws(sc, ps, sel, n, k, W_, n, ws)
        torch.cuda.synchronize()
        assert np.array_equal(sel.cpu().numpy(), build_selection(s, pos, n, k, W_, n, topk)), i
