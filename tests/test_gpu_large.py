"""GPU parity at the largest addresses the library accepts.

Every KV buffer here is larger than 4 GiB, so the (batch, kv head) slabs,
pages and selected rows that the kernels (split-K, length-balanced per
workgroup and per wave, sparse) read lie beyond what a 32-bit byte offset from
the buffer's start can reach; the sparse case also reads the last
rows of the largest slab a plan allows (capacity * head_dim * 2 bytes just under
4 GiB, the limit the plan call enforces). Rows that are never written hold NaN,
so a read of any of them would show in the output.

The oracle sees compact host copies holding exactly the rows each call may use
(the live prefixes, the gathered pages, the selected rows), which is the same
attention by definition: rows outside the attended set take no part in it.
"""

import numpy as np
import pytest

import oracle
import workloads as W
from tests import helpers as H

pytestmark = pytest.mark.gpu

D = 128
SCALE = float(np.float32(1.0 / np.sqrt(128.0)))


@pytest.fixture(scope="module")
def da():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    H.ensure_built()
    import decode_attention_05_amd as m
    m.library()
    return m


def nan_buffer(shape):
    import torch
    return torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")


def release():
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# Dense and ragged: [2, 8, 2^21, 128] bf16 caches (8 GiB each); the slab of
# (b = 1, kv head 7) starts 7.5 GiB into the buffer. Rows [0, LIVE) are written.
CAP = 1 << 21
LIVE = 65536


@pytest.fixture(scope="module")
def big_cache(da):
    B, Hq, Hkv = 2, 16, 8
    sq, sk, sv, _ = W.seeds(31)
    q = W.normal_bf16(sq, (B, Hq, 1, D))
    k = W.normal_bf16(sk, (B, Hkv, LIVE, D))
    v = W.normal_bf16(sv, (B, Hkv, LIVE, D))
    H.log(f"large dense caches: [{B}, {Hkv}, {CAP}, {D}] bf16, {LIVE} live rows")
    dk, dv = nan_buffer((B, Hkv, CAP, D)), nan_buffer((B, Hkv, CAP, D))
    dk[:, :, :LIVE] = H.to_dev(k)
    dv[:, :, :LIVE] = H.to_dev(v)
    yield q, k, v, H.to_dev(q), dk, dv
    del dk, dv
    release()


@pytest.mark.parametrize("k_len", [1000, LIVE])
def test_dense_caches_beyond_4gib(da, big_cache, k_len):
    import torch
    q, k, v, dq, dk, dv = big_cache
    B, Hq, Hkv = q.shape[0], q.shape[1], k.shape[1]
    plan = da.decode_attn_plan(B, Hq, Hkv, D, CAP, LIVE)
    H.log(f"dense beyond 4 GiB: k_len={k_len} splits<={plan.num_splits_max}")
    out = torch.empty((B, Hq, 1, D), dtype=torch.bfloat16, device="cuda")
    da.decode_attn_dense(plan, dq, dk, dv, out, SCALE, k_len, da.workspace_for(plan))
    torch.cuda.synchronize()
    H.check_tolerance(H.from_dev(out), oracle.dense(q, k, v, SCALE, k_len),
                      f"dense beyond 4 GiB, k_len {k_len}")


def test_ragged_caches_beyond_4gib(da, big_cache):
    import torch
    q, k, v, dq, dk, dv = big_cache
    B, Hq, Hkv = q.shape[0], q.shape[1], k.shape[1]
    lens = np.array([3000, LIVE], dtype=np.int32)
    plan = da.decode_attn_plan(B, Hq, Hkv, D, CAP, LIVE, ragged=True)
    H.log(f"ragged beyond 4 GiB: lengths {lens.tolist()}")
    out = torch.empty((B, Hq, 1, D), dtype=torch.bfloat16, device="cuda")
    da.decode_attn_dense_ragged(plan, dq, dk, dv, out, SCALE, H.to_dev_i32(lens),
                                workspace=da.workspace_for(plan))
    torch.cuda.synchronize()
    H.check_tolerance(H.from_dev(out), oracle.dense_ragged(q, k, v, SCALE, lens, causal=True),
                      "ragged beyond 4 GiB")


def test_wave_runs_over_caches_beyond_4gib(da):
    # 640 sequences x 8 kv heads of 4096-row slabs (1 MiB each, 5 GiB per cache):
    # one run per wave, and the slabs of sequences 512 and up start past 4 GiB.
    import torch
    B, Hq, Hkv, cap, live = 640, 32, 8, 4096, 160
    rng = np.random.Generator(np.random.PCG64(35))
    lens = rng.integers(1, live + 1, size=B).astype(np.int32)
    sq, sk, sv, _ = W.seeds(36)
    q = W.normal_bf16(sq, (B, Hq, 1, D))
    k = W.normal_bf16(sk, (B, Hkv, live, D))
    v = W.normal_bf16(sv, (B, Hkv, live, D))
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, ragged=True)
    assert B * Hkv >= plan.balanced_wgs * 4   # one run per wave
    H.log(f"wave runs beyond 4 GiB: [{B}, {Hkv}, {cap}, {D}] caches, lengths 1..{live}")
    dk, dv = nan_buffer((B, Hkv, cap, D)), nan_buffer((B, Hkv, cap, D))
    dk[:, :, :live] = H.to_dev(k)
    dv[:, :, :live] = H.to_dev(v)
    out = torch.empty((B, Hq, 1, D), dtype=torch.bfloat16, device="cuda")
    da.decode_attn_dense_ragged(plan, H.to_dev(q), dk, dv, out, SCALE, H.to_dev_i32(lens),
                                workspace=da.workspace_for(plan))
    torch.cuda.synchronize()
    got = H.from_dev(out)
    del dk, dv
    release()
    H.check_tolerance(got, oracle.dense_ragged(q, k, v, SCALE, lens, causal=True),
                      "wave runs beyond 4 GiB")


def test_paged_pool_beyond_4gib(da):
    # A pool of 8448 pages x 8 kv heads x 256 rows (4.4 GB per cache): the pages
    # used lie past the first 4 GiB, except one near the start.
    import torch
    B, Hq, Hkv, page, max_pages, num_pages = 2, 16, 8, 256, 8, 8448
    cap = page * max_pages
    table = np.array([[8447 - i for i in range(max_pages)],
                      [8200, 3, 8300, 8201, 8400, 8302, -1, -1]], dtype=np.int32)
    lens = np.array([cap, 1500], dtype=np.int32)   # sequence 1 uses its first 6 pages
    sq, sk, sv, _ = W.seeds(32)
    q = W.normal_bf16(sq, (B, Hq, 1, D))
    k = W.normal_bf16(sk, (B, Hkv, cap, D))   # logical rows of each sequence
    v = W.normal_bf16(sv, (B, Hkv, cap, D))
    H.log(f"paged beyond 4 GiB: pool [{num_pages}, {Hkv}, {page}, {D}], lengths {lens.tolist()}")
    dk, dv = nan_buffer((num_pages, Hkv, page, D)), nan_buffer((num_pages, Hkv, page, D))
    kd, vd = H.to_dev(k), H.to_dev(v)
    for b in range(B):
        for j in range(max_pages):
            pg = int(table[b, j])
            if pg >= 0:
                dk[pg] = kd[b, :, j * page:(j + 1) * page]
                dv[pg] = vd[b, :, j * page:(j + 1) * page]
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, page_size=page,
                               max_pages_per_seq=max_pages, num_pages=num_pages)
    out = torch.empty((B, Hq, 1, D), dtype=torch.bfloat16, device="cuda")
    da.decode_attn_dense_paged(plan, H.to_dev(q), dk, dv, H.to_dev_i32(table),
                               H.to_dev_i32(lens), out, SCALE, workspace=da.workspace_for(plan))
    torch.cuda.synchronize()
    got = H.from_dev(out)
    del dk, dv, kd, vd
    release()
    # rows past a sequence's length are never attended, so the logical rows
    # stand in for the pages (the oracle's own unpage would need the whole pool)
    H.check_tolerance(got, oracle.dense_ragged(q, k, v, SCALE, lens, causal=True),
                      "paged beyond 4 GiB")


def test_sparse_top_rows_of_the_largest_slab(da):
    # kv_batch 2, one kv head, capacity 2^24 - 1 rows: each slab is 256 bytes
    # short of 4 GiB and the second starts just below 4 GiB. The selection
    # names the last rows of each slab, row 0, rows around 2^23 and random
    # rows, with pads in the middle and at the end.
    import torch
    B, Hq, Hkv, topk = 2, 16, 1, 2048
    cap = (1 << 24) - 1
    rng = np.random.Generator(np.random.PCG64(33))
    sel = np.full((B, topk), -1, dtype=np.int32)
    for b in range(B):
        fixed = [cap - 1, cap - 2, cap - 33, 0, 1 << 23, (1 << 23) - 1]
        pool = rng.choice(cap - 64, 1900, replace=False) + 1
        rows = np.unique(np.concatenate([fixed, pool]))[:1990]
        rng.shuffle(rows)
        sel[b, :len(rows)] = rows
        sel[b, rng.choice(len(rows), 40, replace=False)] = -1   # pads among the entries
    sq, sk, sv, _ = W.seeds(34)
    q = W.normal_bf16(sq, (B, Hq, 1, D))
    kc = W.normal_bf16(sk, (B, Hkv, topk, D))   # the row that entry t names
    vc = W.normal_bf16(sv, (B, Hkv, topk, D))
    sel_c = np.where(sel >= 0, np.arange(topk, dtype=np.int32)[None, :], -1).astype(np.int32)
    H.log(f"sparse largest slab: kv [{B}, {Hkv}, {cap}, {D}], topk {topk}, "
          f"max row {int(sel.max())}")
    dk, dv = nan_buffer((B, Hkv, cap, D)), nan_buffer((B, Hkv, cap, D))
    kd, vd = H.to_dev(kc), H.to_dev(vc)
    for b in range(B):
        ok = np.nonzero(sel[b] >= 0)[0]
        rows = torch.from_numpy(sel[b, ok].astype(np.int64)).cuda()
        idx = torch.from_numpy(ok.astype(np.int64)).cuda()
        dk[b, 0].index_copy_(0, rows, kd[b, 0].index_select(0, idx))
        dv[b, 0].index_copy_(0, rows, vd[b, 0].index_select(0, idx))
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, topk_max=topk, kv_batch=B)
    out = torch.empty((B, Hq, 1, D), dtype=torch.bfloat16, device="cuda")
    da.decode_attn_sparse(plan, H.to_dev(q), dk, dv, H.to_dev_i32(sel), topk, out, SCALE, cap,
                          da.workspace_for(plan))
    torch.cuda.synchronize()
    got = H.from_dev(out)
    del dk, dv, kd, vd
    release()
    H.check_tolerance(got, oracle.sparse(q, kc, vc, sel_c, SCALE), "sparse largest slab")
