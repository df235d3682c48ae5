"""Ragged batches and paged caches against the fp64 oracle.

One live length per sequence, read on the device (the DflashScratch page of
metrale: a [kv_len, q_offset, q_rope_pos] triple per band, read at kernel
entry), and a paged cache addressed through a block table (the same page: the
cache is written and read through slot indices). The oracle for both is the
dense oracle applied one sequence at a time, over the pages gathered back into
contiguous rows.
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


def _out(B, Hq, D):
    import torch
    return torch.full((B, Hq, 1, D), float("nan"), dtype=torch.bfloat16, device="cuda")


def _clamped(lens, max_len):
    return np.clip(np.asarray(lens, dtype=np.int64), 0, max_len)


def _check_ragged(got_bits, q, k, v, scale, lens, what):
    ref = oracle.dense_ragged(q, k, v, scale, lens)
    H.check_tolerance(got_bits, ref, what)
    for b, n in enumerate(lens):
        if n == 0:
            assert not got_bits[b].any(), f"{what}: empty sequence {b} must give zeros"


RAGGED_SHAPES = [
    # B, Hq, Hkv, D, capacity, lengths (some beyond capacity or negative: clamped)
    (6, 16, 2, 128, 5000, [5000, 0, 1, 33, 1025, 4097]),
    (5, 8, 8, 64, 700, [700, 31, 32, 10 ** 9, -4]),
    (3, 64, 1, 128, 3000, [2999, 64, 1500]),
    (7, 32, 8, 128, 2048, [2048, 1537, 1, 700, 0, 2047, 96]),
]


@pytest.mark.parametrize("B,Hq,Hkv,D,cap,lens", RAGGED_SHAPES)
def test_ragged_matches_oracle(da, B, Hq, Hkv, D, cap, lens):
    q, k, v = W.random_case(80 + B, B, Hq, Hkv, D, cap)
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, ragged=True)
    out = _out(B, Hq, D)
    H.log(f"ragged B={B} Hq={Hq} Hkv={Hkv} D={D} cap={cap} S={plan.num_splits_max} lens={lens}")
    da.decode_attn_dense_ragged(plan, H.to_dev(q), H.to_dev(k), H.to_dev(v), out, 0.09,
                                H.to_dev_i32(np.asarray(lens, dtype=np.int64).clip(-2**31, 2**31 - 1)),
                                workspace=da.workspace_for(plan))
    import torch
    torch.cuda.synchronize()
    _check_ragged(H.from_dev(out), q, k, v, 0.09, _clamped(lens, cap), f"ragged {lens}")


def test_ragged_reads_strided_triples(da):
    # lengths taken out of [kv_len, q_offset, q_rope_pos] triples: stride 3
    B, Hq, Hkv, D, cap = 4, 16, 4, 128, 2500
    lens = [2500, 77, 1200, 0]
    q, k, v = W.random_case(90, B, Hq, Hkv, D, cap)
    triples = np.array([[n, 12345, -999] for n in lens], dtype=np.int32)
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, ragged=True)
    out = _out(B, Hq, D)
    H.log("ragged stride-3 triples")
    da.decode_attn_dense_ragged(plan, H.to_dev(q), H.to_dev(k), H.to_dev(v), out, 0.09,
                                H.to_dev_i32(triples.ravel()), k_lens_stride=3,
                                workspace=da.workspace_for(plan))
    import torch
    torch.cuda.synchronize()
    _check_ragged(H.from_dev(out), q, k, v, 0.09, lens, "stride 3")


def test_ragged_schedule_edges(da):
    # lengths that put run boundaries at stream starts, inside streams and on
    # sequences shorter than a run; one long sequence cut into many runs; all
    # sequences empty; a single sequence
    import torch
    B, Hq, Hkv, D, cap = 9, 32, 8, 128, 6000
    q, k, v = W.random_case(91, B, Hq, Hkv, D, cap)
    dq, dk, dv = H.to_dev(q), H.to_dev(k), H.to_dev(v)
    for num_cus, lens in ((256, [6000, 1, 32, 33, 0, 4500, 64, 0, 2]),
                          (4, [6000, 1, 32, 33, 0, 4500, 64, 0, 2]),
                          (1, [256] * 9),
                          (256, [0] * 9),
                          (3, [0, 0, 0, 0, 5999, 0, 0, 0, 0])):
        plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, ragged=True, num_cus=num_cus)
        out = _out(B, Hq, D)
        H.log(f"ragged schedule cus={num_cus} wgs={plan.balanced_wgs} lens={lens}")
        da.decode_attn_dense_ragged(plan, dq, dk, dv, out, 0.09, H.to_dev_i32(lens),
                                    workspace=da.workspace_for(plan))
        torch.cuda.synchronize()
        _check_ragged(H.from_dev(out), q, k, v, 0.09, lens, f"cus={num_cus} {lens}")


def test_ragged_is_deterministic_and_ignores_workspace_contents(da):
    import torch
    B, Hq, Hkv, D, cap = 6, 64, 4, 128, 3000
    q, k, v = W.random_case(92, B, Hq, Hkv, D, cap)
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, ragged=True, num_cus=16)
    dq, dk, dv = H.to_dev(q), H.to_dev(k), H.to_dev(v)
    lens = H.to_dev_i32([3000, 17, 2999, 640, 1, 1500])
    ws = da.workspace_for(plan)
    outs = []
    for fill in (0.0, float("nan"), 1e30):
        ws.view(torch.float32).fill_(fill)
        out = _out(B, Hq, D)
        H.log(f"ragged determinism, workspace filled with {fill}")
        da.decode_attn_dense_ragged(plan, dq, dk, dv, out, 0.09, lens, workspace=ws)
        torch.cuda.synchronize()
        outs.append(out.clone())
    assert all(torch.equal(outs[0].view(torch.int16), o.view(torch.int16)) for o in outs[1:])
    _check_ragged(H.from_dev(outs[0]), q, k, v, 0.09, [3000, 17, 2999, 640, 1, 1500], "G=16")


PAGED_SHAPES = [
    # B, Hq, Hkv, D, page_size, max_pages, lengths
    (5, 16, 2, 128, 32, 40, [1280, 0, 1, 33, 1000]),
    (4, 32, 8, 128, 64, 30, [1920, 64, 65, 1100]),
    (3, 8, 8, 64, 128, 12, [1536, 127, 513]),
    (2, 64, 1, 128, 256, 9, [2304, 2000]),
]


def _paged_case(seed, B, Hq, Hkv, D, page_size, max_pages, lens, spare=3):
    rng = np.random.Generator(np.random.PCG64(seed))
    table, num_pages = W.page_table(rng, lens, page_size, max_pages, spare)
    sq, sk, sv, _ = W.seeds(seed + 1000)
    q = W.normal_bf16(sq, (B, Hq, 1, D))
    kp = W.normal_bf16(sk, (num_pages, Hkv, page_size, D))
    vp = W.normal_bf16(sv, (num_pages, Hkv, page_size, D))
    used = set(int(x) for x in table.ravel() if x >= 0)
    for pg in range(num_pages):         # pages no sequence owns hold NaN: never read
        if pg not in used:
            kp[pg] = W.BF16_NAN
            vp[pg] = W.BF16_NAN
    return q, kp, vp, table, num_pages


@pytest.mark.parametrize("B,Hq,Hkv,D,page_size,max_pages,lens", PAGED_SHAPES)
def test_paged_matches_oracle(da, B, Hq, Hkv, D, page_size, max_pages, lens):
    import torch
    q, kp, vp, table, num_pages = _paged_case(100 + page_size, B, Hq, Hkv, D, page_size,
                                              max_pages, lens)
    # entries past a sequence's pages are ignored, whatever they hold
    junk = table.copy()
    for b, n in enumerate(lens):
        junk[b, -(-n // page_size):] = [10 ** 6, -5][b % 2]
    cap = page_size * max_pages
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, page_size=page_size,
                               max_pages_per_seq=max_pages, num_pages=num_pages)
    out = _out(B, Hq, D)
    H.log(f"paged B={B} Hq={Hq} Hkv={Hkv} D={D} page={page_size} pool={num_pages} "
          f"S={plan.num_splits_max} lens={lens}")
    da.decode_attn_dense_paged(plan, H.to_dev(q), H.to_dev(kp), H.to_dev(vp), H.to_dev_i32(junk),
                               H.to_dev_i32(lens), out, 0.09, workspace=da.workspace_for(plan))
    torch.cuda.synchronize()
    got = H.from_dev(out)
    ref = oracle.dense_paged(q, kp, vp, table, 0.09, lens)
    H.check_tolerance(got, ref, f"paged {lens}")
    for b, n in enumerate(lens):
        if n == 0:
            assert not got[b].any()


def test_paged_with_identity_table_is_the_ragged_call(da):
    # one page pool laid out as the contiguous cache, pages in order: bit-identical
    import torch
    B, Hq, Hkv, D, page, max_pages = 3, 32, 4, 128, 64, 50
    cap = page * max_pages
    q, k, v = W.random_case(95, B, Hq, Hkv, D, cap)
    # [B, Hkv, cap, D] -> pages [B * max_pages, Hkv, page, D]
    to_pages = lambda x: np.ascontiguousarray(  # noqa: E731
        x.reshape(B, Hkv, max_pages, page, D).transpose(0, 2, 1, 3, 4)
        .reshape(B * max_pages, Hkv, page, D))
    table = np.arange(B * max_pages, dtype=np.int32).reshape(B, max_pages)
    lens = [cap, 1234, 64]
    ragged = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, ragged=True)
    paged = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, page_size=page,
                                max_pages_per_seq=max_pages, num_pages=B * max_pages)
    assert ragged.balanced_wgs == paged.balanced_wgs
    a, b = _out(B, Hq, D), _out(B, Hq, D)
    H.log("paged identity table == ragged")
    dl = H.to_dev_i32(lens)
    da.decode_attn_dense_ragged(ragged, H.to_dev(q), H.to_dev(k), H.to_dev(v), a, 0.09, dl,
                                workspace=da.workspace_for(ragged))
    da.decode_attn_dense_paged(paged, H.to_dev(q), H.to_dev(to_pages(k)), H.to_dev(to_pages(v)),
                               H.to_dev_i32(table), dl, b, 0.09, workspace=da.workspace_for(paged))
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_paged_skips_out_of_range_pages_inside_the_length(da):
    # a page id outside the pool inside a sequence's length is never read: the
    # result is attention over the remaining pages
    import torch
    B, Hq, Hkv, D, page, max_pages = 2, 16, 2, 128, 32, 10
    lens = [320, 200]
    q, kp, vp, table, num_pages = _paged_case(97, B, Hq, Hkv, D, page, max_pages, lens)
    bad = table.copy()
    bad[0, 3] = num_pages          # one full page of sequence 0 dropped
    bad[1, 0] = -1                 # the first page of sequence 1 dropped
    cap = page * max_pages
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, page_size=page,
                               max_pages_per_seq=max_pages, num_pages=num_pages)
    out = _out(B, Hq, D)
    H.log("paged out-of-range ids inside the length")
    da.decode_attn_dense_paged(plan, H.to_dev(q), H.to_dev(kp), H.to_dev(vp), H.to_dev_i32(bad),
                               H.to_dev_i32(lens), out, 0.09, workspace=da.workspace_for(plan))
    torch.cuda.synchronize()
    kept = np.full_like(table, -1)
    kept[0, :9] = np.delete(table[0], 3)[:9]
    kept[1, :6] = table[1, 1:7]
    ref = oracle.dense_paged(q, kp, vp, kept, 0.09, [288, 168])
    H.check_tolerance(H.from_dev(out), ref, "dropped pages")


def test_paged_graph_replay_follows_lengths_and_table(da):
    import torch
    B, Hq, Hkv, D, page, max_pages = 4, 32, 8, 128, 64, 40
    cap = page * max_pages
    rng = np.random.Generator(np.random.PCG64(98))
    pool = B * max_pages
    sq, sk, sv, _ = W.seeds(99)
    q = W.normal_bf16(sq, (B, Hq, 1, D))
    kp = W.normal_bf16(sk, (pool, Hkv, page, D))
    vp = W.normal_bf16(sv, (pool, Hkv, page, D))
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, page_size=page,
                               max_pages_per_seq=max_pages, num_pages=pool)
    dq, dk, dv = H.to_dev(q), H.to_dev(kp), H.to_dev(vp)
    table_dev = torch.full((B, max_pages), -1, dtype=torch.int32, device="cuda")
    lens_dev = torch.zeros(B, dtype=torch.int32, device="cuda")
    out = _out(B, Hq, D)
    ws = da.workspace_for(plan)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        da.decode_attn_dense_paged(plan, dq, dk, dv, table_dev, lens_dev, out, 0.09, workspace=ws)
    for it in range(4):
        lens = [int(x) for x in rng.integers(0, cap + 1, size=B)]
        lens[it % B] = cap
        table, _ = W.page_table(rng, lens, page, max_pages, pool - sum(-(-n // page) for n in lens))
        H.log(f"paged graph replay {it} lens={lens}")
        table_dev.copy_(H.to_dev_i32(table))
        lens_dev.copy_(H.to_dev_i32(lens))
        g.replay()
        torch.cuda.synchronize()
        H.check_tolerance(H.from_dev(out), oracle.dense_paged(q, kp, vp, table, 0.09, lens),
                          f"replay {it}")


@pytest.mark.parametrize("name", ["ragged", "paged", "wide"])
def test_full_size_sampled(da, name):
    # the benchmark's own workload and launch, checked on sampled sequences and heads
    import torch
    case = W.RAGGED_CASES[name]
    cap = case.len_hi
    if case.page_size:
        q, kp, vp, table, lens = W.paged_inputs(case)
        plan = da.decode_attn_plan(case.B, case.Hq, case.Hkv, case.D, cap, cap,
                                   page_size=case.page_size, max_pages_per_seq=case.max_pages,
                                   num_pages=kp.shape[0])
    else:
        q, k, v, lens = W.ragged_inputs(case)
        plan = da.decode_attn_plan(case.B, case.Hq, case.Hkv, case.D, cap, cap, ragged=True)
    out = _out(case.B, case.Hq, case.D)
    H.log(f"full size {name} S={plan.num_splits_max}")
    ws = da.workspace_for(plan)
    if case.page_size:
        da.decode_attn_dense_paged(plan, H.to_dev(q), H.to_dev(kp), H.to_dev(vp),
                                   H.to_dev_i32(table), H.to_dev_i32(lens), out, case.scale,
                                   workspace=ws)
    else:
        da.decode_attn_dense_ragged(plan, H.to_dev(q), H.to_dev(k), H.to_dev(v), out, case.scale,
                                    H.to_dev_i32(lens), workspace=ws)
    torch.cuda.synchronize()
    got = H.from_dev(out)
    rng = np.random.Generator(np.random.PCG64(7))
    for b in sorted(set([0, int(np.argmin(lens))] + rng.choice(case.B, 3, replace=False).tolist())):
        if case.page_size:
            kb = oracle.unpage(kp, table[b:b + 1], cap)
            vb = oracle.unpage(vp, table[b:b + 1], cap)
        else:
            kb, vb = k[b:b + 1], v[b:b + 1]
        heads = rng.choice(case.Hq, 4, replace=False)
        ref = oracle.dense(q[b:b + 1], kb, vb, case.scale, int(lens[b]), rows=heads)
        H.check_tolerance(got[b, heads, 0], ref, f"{name} b={b} heads={heads.tolist()}")


@pytest.mark.parametrize("B,num_cus,Sq,ties", [(64, 0, 1, False), (64, 5, 2, True),
                                                (63, 0, 1, True), (65, 0, 1, True)])
def test_length_order_boundaries(da, B, num_cus, Sq, ties):
    # up to 64 sequences are laid shortest first (ties in index order), ranked
    # in one wave: 64 uses every lane, 65 falls back to index order. Lengths
    # with many ties, zeros and the extremes.
    import torch
    Hq, Hkv, D, cap = 8, 2, 64, 700
    rng = np.random.Generator(np.random.PCG64(450 + B + int(ties)))
    pool = [0, 1, 31, 32, 33, 300, cap] if ties else None
    lens = ([int(x) for x in rng.choice(pool, size=B)] if ties
            else [int(x) for x in rng.integers(0, cap + 1, size=B)])
    lens[B // 2] = cap
    sq, sk, sv, _ = W.seeds(451 + B)
    q = W.normal_bf16(sq, (B, Hq, Sq, D))
    k = W.normal_bf16(sk, (B, Hkv, cap, D))
    v = W.normal_bf16(sv, (B, Hkv, cap, D))
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, seq_q=Sq, causal=True, ragged=True,
                               num_cus=num_cus)
    out = torch.full((B, Hq, Sq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    H.log(f"length order B={B} Sq={Sq} ties={ties} wgs={plan.balanced_wgs}")
    da.decode_attn_dense_ragged(plan, H.to_dev(q), H.to_dev(k), H.to_dev(v), out, 0.1,
                                H.to_dev_i32(lens), workspace=da.workspace_for(plan))
    torch.cuda.synchronize()
    got = H.from_dev(out)
    ref = oracle.dense_ragged(q, k, v, 0.1, lens, True)
    H.check_tolerance(got, ref, f"B={B}")
    assert not got[~ref.any(axis=-1)].any()


@pytest.mark.parametrize("B,Hq,Hkv,D,num_cus,Sq,paged", [
    (512, 16, 8, 64, 0, 1, False),    # ~3950 streams: one run per wave on 256 CUs
    (520, 16, 8, 64, 0, 1, True),     # paged, beyond 512 sequences (two length groups)
    (40, 16, 4, 128, 4, 4, False),    # shortest-first order with wave runs, 4 tokens
    (24, 32, 8, 128, 2, 1, True),     # head tiles of 4 heads, paged
    (12, 16, 4, 64, 3, 16, False),    # 16 tokens: one head per stream, 16 rows, D = 64
    (30, 64, 1, 128, 2, 2, True),     # 64 heads on one kv head: 8 head tiles, paged
    (20, 32, 4, 64, 2, 3, True),      # D = 64, 3 causal tokens, paged
])
def test_wave_runs(da, B, Hq, Hkv, D, num_cus, Sq, paged):
    # at least as many streams as the grid has waves: every wave streams its own
    # run and writes its own rows or partials, with no workgroup merge
    import torch
    cap, page = 640, 64
    rng = np.random.Generator(np.random.PCG64(470 + B))
    lens = [int(x) for x in np.exp(rng.uniform(np.log(20), np.log(cap), size=B))]
    lens[::29] = [0] * len(lens[::29])
    lens[1] = cap
    sq, sk, sv, _ = W.seeds(471 + B)
    q = W.normal_bf16(sq, (B, Hq, Sq, D))
    kw = dict(seq_q=Sq, causal=True, num_cus=num_cus)
    if paged:
        max_pages = cap // page
        table, num_pages = W.page_table(rng, lens, page, max_pages, 2)
        k = W.normal_bf16(sk, (num_pages, Hkv, page, D))
        v = W.normal_bf16(sv, (num_pages, Hkv, page, D))
        plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, page_size=page,
                                   max_pages_per_seq=max_pages, num_pages=num_pages, **kw)
    else:
        k = W.normal_bf16(sk, (B, Hkv, cap, D))
        v = W.normal_bf16(sv, (B, Hkv, cap, D))
        plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, ragged=True, **kw)
    G = Hq // Hkv
    gt = max(d for d in range(1, 16 // Sq + 1) if G % d == 0)   # query heads per stream
    streams = sum(1 for n in lens if n > 0) * Hkv * (G // gt)
    assert streams >= plan.balanced_wgs * 4
    out = torch.full((B, Hq, Sq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    H.log(f"wave runs B={B} Hq={Hq} Hkv={Hkv} D={D} Sq={Sq} paged={paged} wgs={plan.balanced_wgs}")
    ws = da.workspace_for(plan)
    if paged:
        da.decode_attn_dense_paged(plan, H.to_dev(q), H.to_dev(k), H.to_dev(v), H.to_dev_i32(table),
                                   H.to_dev_i32(lens), out, 0.1, workspace=ws)
    else:
        da.decode_attn_dense_ragged(plan, H.to_dev(q), H.to_dev(k), H.to_dev(v), out, 0.1,
                                    H.to_dev_i32(lens), workspace=ws)
    torch.cuda.synchronize()
    got = H.from_dev(out)
    ref = (oracle.dense_paged(q, k, v, table, 0.1, lens, True) if paged
           else oracle.dense_ragged(q, k, v, 0.1, lens, True))
    H.check_tolerance(got, ref, f"wave runs B={B}")
    assert not got[~ref.any(axis=-1)].any()


def test_wave_runs_of_many_short_streams(da):
    # 1024 sequences of 1 to 70 keys, 8 kv heads, D = 128: ~8 tiles per run cut
    # into up to eight whole streams, more finished pieces than a wave's record
    # buffer holds (written out mid-run), and runs that move across several
    # 64-sequence windows of lengths
    import torch
    B, Hq, Hkv, D, cap = 1024, 32, 8, 128, 96
    rng = np.random.Generator(np.random.PCG64(490))
    lens = [int(x) for x in rng.integers(1, 71, size=B)]
    lens[::37] = [0] * len(lens[::37])
    sq, sk, sv, _ = W.seeds(491)
    q = W.normal_bf16(sq, (B, Hq, 1, D))
    k = W.normal_bf16(sk, (B, Hkv, cap, D))
    v = W.normal_bf16(sv, (B, Hkv, cap, D))
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, ragged=True)
    assert B * Hkv >= plan.balanced_wgs * 4   # one run per wave
    out = _out(B, Hq, D)
    H.log(f"wave runs of many short streams B={B} wgs={plan.balanced_wgs}")
    da.decode_attn_dense_ragged(plan, H.to_dev(q), H.to_dev(k), H.to_dev(v), out, 0.1,
                                H.to_dev_i32(lens), workspace=da.workspace_for(plan))
    torch.cuda.synchronize()
    _check_ragged(H.from_dev(out), q, k, v, 0.1, lens, "many short streams")


def test_few_live_streams_in_a_wide_batch(da):
    # 512 sequences x 8 kv heads take one run per wave, but only 90 sequences
    # are non-empty (720 streams): runs skip runs of empty sequences, across the
    # 64-sequence windows of lengths each wave keeps, and most runs are empty
    import torch
    B, Hq, Hkv, D, cap = 512, 16, 8, 64, 300
    rng = np.random.Generator(np.random.PCG64(480))
    lens = [0] * B
    for b in rng.choice(B, size=90, replace=False):
        lens[int(b)] = int(rng.integers(1, cap + 1))
    sq, sk, sv, _ = W.seeds(481)
    q = W.normal_bf16(sq, (B, Hq, 1, D))
    k = W.normal_bf16(sk, (B, Hkv, cap, D))
    v = W.normal_bf16(sv, (B, Hkv, cap, D))
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, ragged=True)
    assert 90 * Hkv < plan.balanced_wgs * 4 <= B * Hkv
    out = _out(B, Hq, D)
    H.log("wide batch, few live streams")
    da.decode_attn_dense_ragged(plan, H.to_dev(q), H.to_dev(k), H.to_dev(v), out, 0.1,
                                H.to_dev_i32(lens), workspace=da.workspace_for(plan))
    torch.cuda.synchronize()
    _check_ragged(H.from_dev(out), q, k, v, 0.1, lens, "few live streams")


@pytest.mark.parametrize("B,num_cus,Sq", [(200, 0, 1), (130, 7, 3), (1000, 0, 1)])
def test_many_sequences(da, B, num_cus, Sq):
    # more than 64 sequences: the schedule reads the lengths in several
    # 64-sequence chunks (totals, the prefix scan that locates a run's first
    # stream, the combine's stream offsets)
    import torch
    Hq, Hkv, D, cap = 4, 2, 64, 600
    rng = np.random.Generator(np.random.PCG64(400 + B))
    lens = [int(x) for x in rng.integers(0, cap + 1, size=B)]
    lens[::17] = [0] * len(lens[::17])
    sq, sk, sv, _ = W.seeds(401 + B)
    q = W.normal_bf16(sq, (B, Hq, Sq, D))
    k = W.normal_bf16(sk, (B, Hkv, cap, D))
    v = W.normal_bf16(sv, (B, Hkv, cap, D))
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, seq_q=Sq, causal=True, ragged=True,
                               num_cus=num_cus)
    out = torch.full((B, Hq, Sq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    H.log(f"ragged many sequences B={B} Sq={Sq} wgs={plan.balanced_wgs}")
    da.decode_attn_dense_ragged(plan, H.to_dev(q), H.to_dev(k), H.to_dev(v), out, 0.1,
                                H.to_dev_i32(lens), workspace=da.workspace_for(plan))
    torch.cuda.synchronize()
    got = H.from_dev(out)
    ref = oracle.dense_ragged(q, k, v, 0.1, lens, True)
    H.check_tolerance(got, ref, f"B={B}")
    assert not got[~ref.any(axis=-1)].any()
