"""Slot-addressed KV writes (decode_attn_write_slots) against the write oracle
(bit-exact: they copy bf16 rows), and the write composed with paged attention
in one captured HIP graph."""

import numpy as np
import pytest

import oracle
import workloads as W
from oracle.append import write_slots
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


def rows(seed, N, Hkv, D):
    sq, sk, sv, _ = W.seeds(seed)
    return W.normal_bf16(sk, (N, Hkv, D)), W.normal_bf16(sv, (N, Hkv, D))


def run_write(da, kp, vp, kr, vr, slots):
    import torch
    dkp, dvp = H.to_dev(kp), H.to_dev(vp)
    ds = torch.from_numpy(np.asarray(slots, np.int64)).cuda()
    da.decode_attn_write_slots(dkp, dvp, H.to_dev(kr), H.to_dev(vr), ds)
    torch.cuda.synchronize()
    return H.from_dev(dkp).reshape(kp.shape), H.from_dev(dvp).reshape(vp.shape)


@pytest.mark.parametrize("num_pages,Hkv,page,D,N", [
    (37, 2, 16, 128, 50),     # several tokens per page, some pages untouched
    (9, 8, 64, 64, 300),      # D = 64, eight kv heads
    (4, 1, 1, 8, 4),          # one-row pages, the smallest head
    (3, 3, 32, 512, 40),      # the largest head
])
def test_random_slots_match_the_oracle(da, num_pages, Hkv, page, D, N):
    rng = np.random.Generator(np.random.PCG64(num_pages * 1000 + N))
    _, kp, vp = W.random_case(700 + N, num_pages, 1, Hkv, D, page)
    kr, vr = rows(701 + N, N, Hkv, D)
    pool = num_pages * page
    slots = rng.choice(pool, size=min(N, pool), replace=False).astype(np.int64)
    slots = np.concatenate([slots, np.full(N - len(slots), -1, np.int64)])
    slots[::7] = -1                          # padding tokens
    slots[3::11] = pool + rng.integers(0, 5, size=len(slots[3::11]))   # past the pool
    H.log(f"write_slots pages={num_pages} Hkv={Hkv} page={page} D={D} N={N}")
    got = run_write(da, kp, vp, kr, vr, slots)
    want = write_slots(kp, vp, kr, vr, slots)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])


def test_slots_beyond_32_bits_never_alias(da):
    # 2^32 + s must not be taken for slot s, nor a large negative value for a valid slot
    _, kp, vp = W.random_case(710, 4, 1, 2, 128, 8)
    kr, vr = rows(711, 4, 2, 128)
    slots = np.array([(1 << 32) + 5, -(1 << 32) + 3, (1 << 62), 9], np.int64)
    got = run_write(da, kp, vp, kr, vr, slots)
    want = write_slots(kp, vp, kr, vr, slots)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
    # only slot 9 (page 1, row 1 of 8-row pages) was written
    changed = np.nonzero((got[0] != kp).any(axis=(1, 3)))
    assert [(int(p), int(r)) for p, r in zip(*changed)] == [(1, 1)]


def test_no_tokens_is_a_no_op(da):
    import torch
    _, kp, vp = W.random_case(712, 2, 1, 2, 64, 4)
    dkp, dvp = H.to_dev(kp), H.to_dev(vp)
    empty = torch.empty((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    da.decode_attn_write_slots(dkp, dvp, empty, empty, torch.empty(0, dtype=torch.int64,
                                                                   device="cuda"))
    torch.cuda.synchronize()
    assert np.array_equal(H.from_dev(dkp).reshape(kp.shape), kp)


def test_duplicate_slots_write_pieces_of_those_rows(da):
    # two tokens naming one slot is a caller error; every 16-byte piece of that
    # slot's rows then holds the same piece of one of the two tokens' rows (the
    # pieces are written independently), and nothing else changes
    _, kp, vp = W.random_case(713, 2, 1, 2, 128, 8)
    kr, vr = rows(714, 3, 2, 128)
    slots = np.array([3, 3, 10], np.int64)
    gk, gv = run_write(da, kp, vp, kr, vr, slots)
    for got, new in ((gk, kr), (gv, vr)):
        for h in range(2):
            for c in range(0, 128, 8):
                piece = got[0, h, 3, c:c + 8]
                assert any(np.array_equal(piece, new[n, h, c:c + 8]) for n in (0, 1)), (h, c)
    want = write_slots(kp, vp, kr[2:], vr[2:], slots[2:])
    mask = np.ones(8, bool)
    mask[3] = False
    assert np.array_equal(gk[:, :, mask], want[0][:, :, mask])
    assert np.array_equal(gv[:, :, mask], want[1][:, :, mask])
    assert np.array_equal(gk[1], want[0][1]) and np.array_equal(gv[1], want[1][1])


def test_slot_write_then_paged_attention_in_one_graph(da):
    # One decode step of a paged cache, captured once: the pass's new rows go to
    # their slots, then the paged attention reads them. Between replays the
    # lengths grow, the slots move to the new positions and the rows change.
    import torch
    B, Hq, Hkv, D, page, max_pages, Sq = 3, 8, 2, 128, 32, 4, 2
    rng = np.random.Generator(np.random.PCG64(720))
    num_pages = B * max_pages + 3
    table = rng.permutation(num_pages)[:B * max_pages].reshape(B, max_pages).astype(np.int32)
    sq, sk, sv, _ = W.seeds(721)
    kp = W.normal_bf16(sk, (num_pages, Hkv, page, D))
    vp = W.normal_bf16(sv, (num_pages, Hkv, page, D))
    q = W.normal_bf16(sq, (B, Hq, Sq, D))
    cap = page * max_pages
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, page_size=page, max_pages_per_seq=max_pages,
                               num_pages=num_pages, seq_q=Sq, causal=True)
    dkp, dvp, dq = H.to_dev(kp), H.to_dev(vp), H.to_dev(q)
    dtab = H.to_dev_i32(table)
    dlens = torch.zeros(B, dtype=torch.int32, device="cuda")
    dslots = torch.zeros(B * Sq, dtype=torch.int64, device="cuda")
    dkr = torch.zeros((B * Sq, Hkv, D), dtype=torch.bfloat16, device="cuda")
    dvr = torch.zeros_like(dkr)
    out = torch.empty((B, Hq, Sq, D), dtype=torch.bfloat16, device="cuda")
    ws = da.workspace_for(plan)

    def slots_for(lens):
        s = []
        for b in range(B):
            for t in range(Sq):
                r = lens[b] - Sq + t
                s.append(int(table[b, r // page]) * page + r % page if r >= 0 else -1)
        return np.array(s, np.int64)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        da.decode_attn_write_slots(dkp, dvp, dkr, dvr, dslots)
        da.decode_attn_dense_paged(plan, dq, dkp, dvp, dtab, dlens, out, 0.08838835,
                                   workspace=ws)
    host_k, host_v = kp, vp
    lens = np.array([1, 40, 97], np.int32)
    for step in range(4):
        kr, vr = rows(730 + step, B * Sq, Hkv, D)
        slots = slots_for(lens)
        dlens.copy_(torch.from_numpy(lens).cuda())
        dslots.copy_(torch.from_numpy(slots).cuda())
        dkr.copy_(H.to_dev(kr))
        dvr.copy_(H.to_dev(vr))
        H.log(f"slot write + paged attention replay {step}, lengths {lens.tolist()}")
        g.replay()
        torch.cuda.synchronize()
        host_k, host_v = write_slots(host_k, host_v, kr, vr, slots)
        assert np.array_equal(H.from_dev(dkp).reshape(kp.shape), host_k)
        ref = oracle.dense_paged(q, host_k, host_v, table, 0.08838835, lens, causal=True)
        H.check_tolerance(H.from_dev(out), ref, f"replay {step}")
        lens = np.minimum(lens + Sq + step, cap).astype(np.int32)
