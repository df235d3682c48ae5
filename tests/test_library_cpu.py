"""CPU-side checks of the C-ABI library: it loads, exports every declared symbol,
plans every workload, and fails closed on every invalid argument -- all without
a GPU (no call here reaches a kernel launch)."""

import ctypes
import os
import re

import pytest

from tests.helpers import ensure_built

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def da():
    ensure_built()
    import decode_attention_05_amd as m
    m.library()
    return m


def declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names.update(re.findall(r"\b(decode_attn_\w+)\s*\(", text))
    return names


def test_exports_every_declared_symbol(da):
    names = declared_functions()
    assert {"decode_attn_plan", "decode_attn_dense", "decode_attn_dense_devlen",
            "decode_attn_sparse", "decode_attn_status_str", "decode_attn_last_error"} <= names
    lib = ctypes.CDLL(da.library_path)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"
    assert set(da.EXPORTED_SYMBOLS) <= names


def test_struct_layout_matches_header(da, tmp_path):
    # Compile a probe against the header with the system C compiler and compare
    # every field offset and both struct sizes with the binding's ctypes mirror.
    probe = tmp_path / "probe.c"
    fields_p = [f for f, _ in da.Problem._fields_]
    fields_l = [f for f, _ in da.Plan._fields_]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "decode_attn.h"',
             "int main(void) {",
             '  printf("%zu\\n", sizeof(decode_attn_problem));',
             '  printf("%zu\\n", sizeof(decode_attn_plan_t));']
    lines += [f'  printf("%zu\\n", offsetof(decode_attn_problem, {f}));' for f in fields_p]
    lines += [f'  printf("%zu\\n", offsetof(decode_attn_plan_t, {f}));' for f in fields_l]
    lines += ["  return 0;", "}"]
    probe.write_text("\n".join(lines))
    exe = tmp_path / "probe"
    import subprocess
    subprocess.check_call(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(probe),
                           "-o", str(exe)])
    got = [int(x) for x in subprocess.check_output([str(exe)]).split()]
    want = [ctypes.sizeof(da.Problem), ctypes.sizeof(da.Plan)]
    want += [getattr(da.Problem, f).offset for f in fields_p]
    want += [getattr(da.Plan, f).offset for f in fields_l]
    assert got == want


def test_status_strings(da):
    assert da.decode_attn_status_str(0) == "DA_OK"
    assert da.decode_attn_status_str(2) == "DA_ERR_UNSUPPORTED"
    assert da.decode_attn_status_str(99) == "DA_ERR_UNKNOWN"


def plan(da, **kw):
    base = dict(batch=4, num_q_heads=64, num_kv_heads=8, head_dim=128, capacity=4096, num_cus=256)
    base.update(kw)
    return da.decode_attn_plan(**base)


@pytest.mark.parametrize("field,value", [("has_alibi", True), ("window_left", 128),
                                         ("window_right", 0), ("has_softcap", True),
                                         ("seq_q", 17), ("seq_q", 0), ("head_dim", 96)])
def test_rejected_features(da, field, value):
    with pytest.raises(da.DecodeAttnError) as ei:
        plan(da, **{field: value})
    assert ei.value.status == 2  # DA_ERR_UNSUPPORTED
    name = field if field not in ("has_alibi", "has_softcap") else field[4:]
    assert name in str(ei.value)


def test_several_query_tokens(da):
    # heads per workgroup shrink so that heads x tokens fit one 16-row tile;
    # the workspace counts every token's rows; sparse plans take one token
    one = plan(da, num_cus=256)
    four = plan(da, seq_q=4, num_cus=256)
    assert four.prob.seq_q == 4
    sixteen = plan(da, seq_q=16, ragged=True)
    assert sixteen.workspace_bytes >= 512 * 2 * 16 * 130 * 4
    assert four.num_splits_max <= one.num_splits_max
    with pytest.raises(da.DecodeAttnError) as ei:
        da.decode_attn_plan(4, 64, 1, 128, 65536, topk_max=64, kv_batch=1, num_cus=256, seq_q=2)
    assert ei.value.status == 2 and "seq_q" in str(ei.value)
    # a causal static call must cover its own tokens
    lib = da.library()
    fake = ctypes.c_void_p(0x10000)
    P = plan(da, seq_q=4, causal=True)
    assert lib.decode_attn_dense(ctypes.byref(P), fake, fake, fake, fake, 0.1, 3,
                                 ctypes.c_void_p(0x20000), P.workspace_bytes, None) == 1
    assert "query tokens" in da.decode_attn_last_error()


def test_slab_size_limit(da):
    # one (batch, kv head) slab of capacity * head_dim bf16 must stay under 4 GiB:
    # the largest capacity is 2^24 - 1 rows at head_dim 128 and 2^25 - 1 at 64
    for D, cap in ((128, (1 << 24) - 1), (64, (1 << 25) - 1)):
        P = plan(da, head_dim=D, capacity=cap, max_k_len=cap)
        assert P.prob.capacity == cap
        S = da.decode_attn_plan(2, 16, 1, D, cap, topk_max=2048, kv_batch=2, num_cus=256)
        assert S.prob.capacity == cap
        with pytest.raises(da.DecodeAttnError) as ei:
            plan(da, head_dim=D, capacity=cap + 1, max_k_len=cap + 1)
        assert ei.value.status == 2 and "4 GiB" in str(ei.value)


def test_causal_is_accepted(da):
    a, b = plan(da, causal=True), plan(da, causal=False)
    assert (a.num_splits_max, a.chunk, a.workspace_bytes) == (b.num_splits_max, b.chunk,
                                                             b.workspace_bytes)


@pytest.mark.parametrize("kw", [dict(num_q_heads=12, num_kv_heads=8), dict(batch=0),
                                dict(num_kv_heads=0), dict(capacity=0),
                                dict(max_k_len=0), dict(max_k_len=4097),
                                dict(topk_max=-1), dict(topk_max=16, kv_batch=2),
                                dict(kv_batch=3), dict(num_cus=-1), dict(force_splits=-2)])
def test_invalid_problems(da, kw):
    with pytest.raises(da.DecodeAttnError) as ei:
        plan(da, **kw)
    assert ei.value.status == 1


def test_dense_plans_for_the_workloads(da):
    # With 256 compute units: split only when there are fewer (batch, kv head)
    # units than CUs, give each CU one workgroup, keep >= 1024 keys per split.
    tiny = da.decode_attn_plan(1, 8, 8, 64, 512, 300, num_cus=256)
    assert tiny.num_splits_max == 1 and tiny.workspace_bytes == 0
    gqa = da.decode_attn_plan(8, 32, 8, 128, 8192, 4096, num_cus=256)
    assert gqa.num_splits_max == 4 and gqa.chunk == 1024
    assert gqa.workspace_bytes == 8 * 32 * 4 * 130 * 4
    long = da.decode_attn_plan(4, 64, 8, 128, 131072, 131072, num_cus=256)
    assert long.num_splits_max == 8 and long.chunk == 16384
    assert long.workspace_bytes == 4 * 64 * 8 * 130 * 4
    # 48 units: 5 splits (240 workgroups), not 6 (288: 32 CUs would get two)
    six = da.decode_attn_plan(6, 64, 8, 128, 65536, 65536, num_cus=256)
    assert six.num_splits_max == 5
    batch = da.decode_attn_plan(128, 32, 8, 128, 2048, 1537, num_cus=256)
    assert batch.num_splits_max == 1 and batch.workspace_bytes == 0
    # query heads beyond 16 per kv head are served by several head tiles
    wide = da.decode_attn_plan(4, 64, 1, 128, 8192, 8192, num_cus=256)
    assert wide.group == 64 and wide.num_splits_max == 8  # 16 units -> 16 splits, capped at 8192/1024


def test_sparse_plan_chunk_is_independent_of_call(da):
    p = da.decode_attn_plan(4, 64, 1, 128, 65536, topk_max=2048, kv_batch=1, num_cus=256)
    assert p.sparse and p.chunk % 16 == 0
    assert p.num_splits_max == -(-2048 // p.chunk)
    q = da.decode_attn_plan(4, 64, 1, 128, 65536, topk_max=4096, kv_batch=1, num_cus=256,
                            force_chunk=p.chunk)
    assert q.chunk == p.chunk


def test_compute_calls_fail_closed_before_any_launch(da):
    lib = da.library()
    P = plan(da)
    fake = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: every call below fails first
    ws = ctypes.c_void_p(0x20000)
    call = lambda *a: lib.decode_attn_dense(ctypes.byref(P), *a)  # noqa: E731
    # NULL pointer
    assert call(None, fake, fake, fake, 0.1, 10, ws, P.workspace_bytes, None) == 1
    # misaligned
    assert call(ctypes.c_void_p(0x10002), fake, fake, fake, 0.1, 10, ws, P.workspace_bytes,
                None) == 1
    # non-finite scale
    assert call(fake, fake, fake, fake, float("nan"), 10, ws, P.workspace_bytes, None) == 1
    assert call(fake, fake, fake, fake, float("inf"), 10, ws, P.workspace_bytes, None) == 1
    # k_len outside [1, max_k_len]
    assert call(fake, fake, fake, fake, 0.1, 0, ws, P.workspace_bytes, None) == 1
    assert call(fake, fake, fake, fake, 0.1, 4097, ws, P.workspace_bytes, None) == 1
    assert "k_len" in da.decode_attn_last_error()
    # workspace missing or too small
    assert P.workspace_bytes > 0
    assert call(fake, fake, fake, fake, 0.1, 10, None, P.workspace_bytes, None) == 3
    assert call(fake, fake, fake, fake, 0.1, 10, ws, P.workspace_bytes - 1, None) == 3
    # a sparse plan handed to the dense call
    S = da.decode_attn_plan(2, 8, 1, 128, 1000, topk_max=64, kv_batch=1, num_cus=256)
    assert lib.decode_attn_dense(ctypes.byref(S), fake, fake, fake, fake, 0.1, 10, ws,
                                 S.workspace_bytes, None) == 1
    # sparse: topk outside [1, topk_max], k_len outside [1, capacity], misaligned sel
    scall = lambda sel, topk, k_len: lib.decode_attn_sparse(  # noqa: E731
        ctypes.byref(S), fake, fake, fake, sel, topk, fake, 0.1, k_len, ws, S.workspace_bytes, None)
    assert scall(fake, 0, 1000) == 1
    assert scall(fake, 65, 1000) == 1
    assert scall(fake, 64, 1001) == 1
    assert scall(fake, 64, 0) == 1
    assert scall(None, 64, 1000) == 1
    assert scall(ctypes.c_void_p(0x10002), 64, 1000) == 1
    # device-resident length: NULL or misaligned pointer
    dl = lambda p: lib.decode_attn_dense_devlen(ctypes.byref(P), fake, fake, fake, fake, 0.1, p, ws,  # noqa: E731
                                                P.workspace_bytes, None)
    assert dl(None) == 1
    assert dl(ctypes.c_void_p(0x10002)) == 1
    assert lib.decode_attn_dense_devlen(ctypes.byref(S), fake, fake, fake, fake, 0.1, fake, ws,
                                        S.workspace_bytes, None) == 1
    # the dense plan handed to the sparse call
    assert lib.decode_attn_sparse(ctypes.byref(P), fake, fake, fake, fake, 8, fake, 0.1, 10, ws,
                                  P.workspace_bytes, None) == 1


def test_selection_builder_fails_closed(da):
    lib = da.library()
    fake = ctypes.c_void_p(0x10000)
    P = da.SelectProblem(4, 65408, 65408, 1920, 128, 65408, 2048)
    call = lambda prob, s=fake, p=fake, o=fake: lib.decode_attn_build_selection(  # noqa: E731
        ctypes.byref(prob), s, p, o, None)
    assert call(P, p=None) == 1
    assert call(P, o=None) == 1
    assert call(P, s=None) == 1
    assert call(P, o=ctypes.c_void_p(0x10002)) == 1
    for field, bad in (("k_idx", 4097), ("k_idx", -1), ("batch", 0), ("topk", 0),
                       ("score_stride", 100), ("window", -1), ("win_base", -5)):
        Q = da.SelectProblem(4, 65408, 65408, 1920, 128, 65408, 2048)
        setattr(Q, field, bad)
        assert call(Q) == 1, field
    big = da.SelectProblem(4, 131073, 131076, 1920, 128, 0, 2048)
    assert call(big) == 2  # more candidates than the builder's row bitmap holds
    odd = da.SelectProblem(4, 65407, 65407, 1920, 128, 0, 2048)
    assert call(odd) == 1  # score rows must be a multiple of 4 floats apart


def test_append_fails_closed(da):
    lib = da.library()
    fake = ctypes.c_void_p(0x10000)
    call = lambda prob, kc=fake, pos=fake: lib.decode_attn_append_kv(  # noqa: E731
        ctypes.byref(prob), kc, fake, fake, fake, pos, None)
    good = da.AppendProblem(4, 8, 128, 4096, 0, 0)
    assert call(good, kc=None) == 1
    assert call(good, pos=None) == 1
    assert call(good, kc=ctypes.c_void_p(0x10008)) == 1
    assert call(good, pos=ctypes.c_void_p(0x10002)) == 1
    for field, bad in (("head_dim", 12), ("head_dim", 1024), ("batch", 0), ("capacity", 0),
                       ("window", -1), ("win_base", 4090)):
        p = da.AppendProblem(4, 8, 128, 4096, 16 if field == "win_base" else 0, 0)
        setattr(p, field, bad)
        assert call(p) == 1, field


def paged_plan(da, **kw):
    base = dict(batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128, capacity=64 * 128,
                page_size=64, max_pages_per_seq=128, num_pages=600, num_cus=256)
    base.update(kw)
    return da.decode_attn_plan(**base)


def test_paged_plans(da):
    p = paged_plan(da)
    # chunks start on 32-key tiles, so with pages a multiple of 32 keys no tile crosses a page
    assert p.prob.page_size == 64 and p.chunk % 32 == 0
    for kw, status in ((dict(page_size=48), 1), (dict(page_size=16), 1),
                       (dict(max_pages_per_seq=0), 1), (dict(num_pages=0), 1),
                       (dict(capacity=64 * 128 + 32), 1), (dict(topk_max=16, kv_batch=4), 2),
                       (dict(force_chunk=48), 1)):
        with pytest.raises(da.DecodeAttnError) as ei:
            paged_plan(da, **kw)
        assert ei.value.status == status, kw


def test_ragged_plans(da):
    # the length-balanced schedule: two resident workgroups per CU, up to one
    # run per wave (4 per workgroup), two partial slots of heads_per_wg rows per run
    dense = plan(da)
    R = plan(da, ragged=True)
    assert dense.balanced_wgs == 0 and R.balanced_wgs == 512 and R.prob.ragged == 1
    assert (R.num_splits_max, R.chunk) == (dense.num_splits_max, dense.chunk)
    assert R.workspace_bytes == max(dense.workspace_bytes, 512 * 4 * 2 * 8 * 130 * 4)
    assert paged_plan(da).balanced_wgs == 512  # paged plans are always ragged
    tiny = da.decode_attn_plan(1, 8, 8, 64, 512, 300, num_cus=256, ragged=True)
    assert tiny.workspace_bytes == 512 * 4 * 2 * 1 * 66 * 4
    with pytest.raises(da.DecodeAttnError) as ei:
        da.decode_attn_plan(4, 64, 1, 128, 65536, topk_max=64, kv_batch=1, num_cus=256,
                            ragged=True)
    assert ei.value.status == 2 and "ragged" in str(ei.value)


def test_ragged_and_paged_fail_closed(da):
    lib = da.library()
    fake = ctypes.c_void_p(0x10000)
    ws = ctypes.c_void_p(0x20000)
    D = plan(da)
    P = plan(da, ragged=True)
    G = paged_plan(da)
    rag = lambda pl, lens=fake, stride=1, w=ws: lib.decode_attn_dense_ragged(  # noqa: E731
        ctypes.byref(pl), fake, fake, fake, fake, 0.1, lens, stride, w, pl.workspace_bytes, None)
    pag = lambda pl, bt=fake, lens=fake, stride=1: lib.decode_attn_dense_paged(  # noqa: E731
        ctypes.byref(pl), fake, fake, fake, bt, lens, stride, fake, 0.1, ws, pl.workspace_bytes,
        None)
    assert rag(P, lens=None) == 1
    assert rag(P, lens=ctypes.c_void_p(0x10002)) == 1
    assert rag(P, stride=0) == 1
    assert rag(P, w=None) == 3
    assert rag(D) == 1                          # a plan made without ragged = 1
    assert "ragged" in da.decode_attn_last_error()
    assert rag(G) == 1                          # a paged plan needs the paged call
    assert "paged" in da.decode_attn_last_error()
    assert pag(P) == 1                          # a contiguous plan handed to the paged call
    assert pag(G, bt=None) == 1
    assert pag(G, bt=ctypes.c_void_p(0x10002)) == 1
    assert pag(G, lens=None) == 1
    assert pag(G, stride=-3) == 1
    # the one-call decode pass: new rows required and aligned, plans as above
    step = lambda pl, kn=fake, vn=fake, bt=None: lib.decode_attn_dense_step(  # noqa: E731
        ctypes.byref(pl), fake, fake, fake, kn, vn, bt, fake, 1, fake, 0.1, ws, pl.workspace_bytes,
        None)
    assert step(P, kn=None) == 1
    assert step(P, vn=ctypes.c_void_p(0x10008)) == 1
    assert step(D) == 1                 # not a ragged plan
    assert step(G) == 1                 # a paged plan without a block table
    assert step(P, bt=fake) == 1        # a block table with a contiguous plan
    # the fixed-length calls refuse a paged plan
    assert lib.decode_attn_dense(ctypes.byref(G), fake, fake, fake, fake, 0.1, 10, ws,
                                 G.workspace_bytes, None) == 1
    assert lib.decode_attn_dense_devlen(ctypes.byref(G), fake, fake, fake, fake, 0.1, fake, ws,
                                        G.workspace_bytes, None) == 1


def test_read_probe_fails_closed(da):
    lib = da.library()
    fake = ctypes.c_void_p(0x10000)
    assert lib.decode_attn_read_probe(None, 1024, fake, None) == 1
    assert lib.decode_attn_read_probe(fake, 1024, None, None) == 1
    assert lib.decode_attn_read_probe(ctypes.c_void_p(0x10004), 1024, fake, None) == 1
    assert lib.decode_attn_read_probe(fake, 1000, fake, None) == 1
    assert lib.decode_attn_read_probe(fake, 0, fake, None) == 1


def test_missing_library_fails_loudly():
    # No fallback implementation: without the built library every entry point
    # raises instead of computing anything another way.
    import subprocess
    import sys
    code = ("import decode_attention_05_amd as d\n"
            "d.library_path = '/nonexistent/libdecode_attn.so'\n"
            "d._lib = None\n"
            "try:\n"
            "    d.decode_attn_plan(1, 8, 8, 64, 512, 300, num_cus=256)\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=root,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    assert "raised:" in r.stdout and "no fallback" in r.stdout


def test_write_slots_validation(da):
    lib = da.library()
    P = ctypes.c_void_p

    def call(prob, k=0x10000, v=0x20000, kr=0x30000, vr=0x40000, sl=0x50000):
        return lib.decode_attn_write_slots(ctypes.byref(prob), P(k), P(v), P(kr), P(vr), P(sl), None)

    good = dict(num_tokens=4, num_kv_heads=2, head_dim=128, page_size=16, num_pages=8)
    for field, bad in [("num_tokens", -1), ("num_kv_heads", 0), ("head_dim", 100),
                       ("head_dim", 1024), ("page_size", 0), ("num_pages", 0)]:
        kw = dict(good, **{field: bad})
        assert call(da.SlotProblem(**kw)) == 1, field
    prob = da.SlotProblem(**good)
    assert call(prob, k=0) == 1                     # NULL pool
    assert call(prob, kr=0x30008) == 1              # rows not 16-byte aligned
    assert call(prob, sl=0x50004) == 1              # slots not 8-byte aligned
    assert "aligned" in da.decode_attn_last_error()
    assert lib.decode_attn_write_slots(None, None, None, None, None, None, None) == 1
    # no tokens: nothing is enqueued and no pointer is read (NULLs accepted)
    empty = da.SlotProblem(**dict(good, num_tokens=0))
    assert lib.decode_attn_write_slots(ctypes.byref(empty), None, None, None, None, None, None) == 0


def test_split_selection_workspace_and_errors(da):
    lib = da.library()
    P = ctypes.c_void_p
    # fewer than 8192 candidates: the one-workgroup builder, no workspace
    assert da.decode_attn_select_workspace(4, 5000, 100, 16, 200) == 0
    # 65408 candidates: 16 parts of 4096, each a 256-byte head share and 512 items of 8 bytes
    assert da.decode_attn_select_workspace(4, 65408, 1920, 128, 2048) == 4 * (256 + 16 * 512 * 8)
    with pytest.raises(da.DecodeAttnError):
        da.decode_attn_select_workspace(4, 200000, 1920, 128, 2048)   # beyond 131072 candidates
    prob = da.SelectProblem(4, 65408, 65408, 1920, 128, 65408, 2048)
    fake = P(0x100000)
    assert lib.decode_attn_build_selection_ws(ctypes.byref(prob), fake, fake, fake, None, 0,
                                              None) == 3           # DA_ERR_WORKSPACE
    assert lib.decode_attn_build_selection_ws(ctypes.byref(prob), fake, fake, fake, fake, 1024,
                                              None) == 3
    assert "workspace" in da.decode_attn_last_error()
    need = 4 * (256 + 16 * 512 * 8)
    assert lib.decode_attn_build_selection_ws(ctypes.byref(prob), fake, fake, fake, P(0x100008),
                                              need, None) == 1     # misaligned workspace


def test_split_env_override_for_tuning(da, monkeypatch):
    # DECODE_ATTN_SPLITS caps the dense split count like force_splits (tuning
    # runs); explicit force fields and sparse plans ignore it, as does junk
    long = dict(num_cus=256)
    assert da.decode_attn_plan(4, 64, 8, 128, 131072, **long).num_splits_max == 8
    monkeypatch.setenv("DECODE_ATTN_SPLITS", "3")
    P = da.decode_attn_plan(4, 64, 8, 128, 131072, **long)
    assert P.num_splits_max == 3 and P.prob.force_splits == 3
    assert da.decode_attn_plan(4, 64, 8, 128, 131072, force_splits=5, **long).num_splits_max == 5
    sparse = da.decode_attn_plan(4, 64, 1, 128, 65536, topk_max=2048, kv_batch=1, **long)
    assert sparse.prob.force_splits == 0 and sparse.num_splits_max == 16
    for junk in ("0", "-2", "abc", "4x"):
        monkeypatch.setenv("DECODE_ATTN_SPLITS", junk)
        assert da.decode_attn_plan(4, 64, 8, 128, 131072, **long).num_splits_max == 8
