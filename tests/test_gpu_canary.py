"""Guard regions around every buffer a call writes: no kernel writes outside the
output, the workspace, or the cache rows it owns (caller-owned buffers, the
flashinfer page "packed_fused_kda_decode": rows that are not written must not
change, and neither must anything past the buffers).

Each written buffer is carved out of a larger device allocation whose leading
and trailing 4 KiB hold a byte pattern; after the call (and a second call on
the same buffers) the pattern must be intact. Inputs the calls only read are
ordinary tensors."""

import numpy as np
import pytest

import workloads as W
from tests import helpers as H

pytestmark = pytest.mark.gpu

GUARD = 4096
FILL = 0xA5


@pytest.fixture(scope="module")
def da():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    H.ensure_built()
    import decode_attention_05_amd as m
    m.library()
    return m


class Guarded:
    """A device tensor of `shape`/`dtype` between two guard regions."""

    def __init__(self, shape, dtype, init=None):
        import torch
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        self.raw = torch.full((GUARD + n + GUARD,), FILL, dtype=torch.uint8, device="cuda")
        self.t = self.raw[GUARD:GUARD + n].view(dtype).view(*shape) if n else \
            torch.empty(shape, dtype=dtype, device="cuda")
        if init is not None:
            self.t.copy_(init)

    def intact(self):
        head = self.raw[:GUARD].cpu().numpy()
        tail = self.raw[-GUARD:].cpu().numpy()
        return bool((head == FILL).all() and (tail == FILL).all())


def guarded_ws(plan):
    import torch
    n = int(plan.workspace_bytes)
    return Guarded((max(n, 16),), torch.uint8)


def twice(fn):
    import torch
    fn()
    fn()
    torch.cuda.synchronize()


@pytest.mark.parametrize("B,Hq,Hkv,D,cap,k_len,Sq,kw", [
    (1, 8, 8, 64, 512, 300, 1, {}),                       # one split: direct bf16 output
    (8, 32, 8, 128, 8192, 4096, 1, {}),                   # split-K with the merge kernel
    (2, 16, 4, 128, 3000, 2999, 3, {"causal": True}),     # several tokens
    (1, 64, 1, 128, 20000, 20000, 1, {"force_chunk": 96}),  # many splits, ragged last one
])
def test_dense_writes_stay_inside(da, B, Hq, Hkv, D, cap, k_len, Sq, kw):
    import torch
    sq, sk, sv, _ = W.seeds(900 + B + Sq)
    q = W.to_dev(W.normal_bf16(sq, (B, Hq, Sq, D)))
    k = W.to_dev(W.normal_bf16(sk, (B, Hkv, cap, D)))
    v = W.to_dev(W.normal_bf16(sv, (B, Hkv, cap, D)))
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, k_len, seq_q=Sq, **kw)
    out = Guarded((B, Hq, Sq, D), torch.bfloat16)
    ws = guarded_ws(plan)
    H.log(f"canary dense B={B} Hq={Hq} D={D} k_len={k_len} Sq={Sq} {kw}")
    twice(lambda: da.decode_attn_dense(plan, q, k, v, out.t, 0.1, k_len, ws.t))
    assert out.intact() and ws.intact()
    kl = torch.tensor([k_len], dtype=torch.int32, device="cuda")
    twice(lambda: da.decode_attn_dense_devlen(plan, q, k, v, out.t, 0.1, kl, ws.t))
    assert out.intact() and ws.intact()
    if Sq == 1 and not kw:
        twice(lambda: da.decode_attn_dense_static(plan, q, k, v, out.t, 0.1, k_len))
        assert out.intact()


@pytest.mark.parametrize("topk,kw", [(2048, {}), (300, {"force_chunk": 48}), (77, {})])
def test_sparse_writes_stay_inside(da, topk, kw):
    import torch
    B, Hq, Hkv, D, rows = 4, 64, 1, 128, 9000
    sq, sk, sv, _ = W.seeds(910 + topk)
    q = W.to_dev(W.normal_bf16(sq, (B, Hq, 1, D)))
    k = W.to_dev(W.normal_bf16(sk, (1, Hkv, rows, D)))
    v = W.to_dev(W.normal_bf16(sv, (1, Hkv, rows, D)))
    rng = np.random.Generator(np.random.PCG64(911))
    sel = np.full((B, topk), -1, np.int32)
    for b in range(B):
        n = topk - 13 * b if topk > 13 * b else 0
        sel[b, :n] = rng.choice(rows, n, replace=False)
    plan = da.decode_attn_plan(B, Hq, Hkv, D, rows, topk_max=topk, kv_batch=1, **kw)
    out = Guarded((B, Hq, 1, D), torch.bfloat16)
    ws = guarded_ws(plan)
    dsel = W.to_dev_i32(sel)
    twice(lambda: da.decode_attn_sparse(plan, q, k, v, dsel, topk, out.t, 0.088, rows, ws.t))
    assert out.intact() and ws.intact()


@pytest.mark.parametrize("paged", [False, True])
def test_ragged_paged_and_step_writes_stay_inside(da, paged):
    import torch
    B, Hq, Hkv, D, page, max_pages, Sq = 5, 16, 4, 128, 64, 8, 2
    cap = page * max_pages
    sq, sk, sv, _ = W.seeds(920)
    lens = np.array([cap, 1, 0, 300, 129], np.int32)
    q = W.to_dev(W.normal_bf16(sq, (B, Hq, Sq, D)))
    if paged:
        rng = np.random.Generator(np.random.PCG64(921))
        table, num_pages = W.page_table(rng, lens, page, max_pages, 3)
        shape = (num_pages, Hkv, page, D)
        plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, page_size=page,
                                   max_pages_per_seq=max_pages, num_pages=num_pages, seq_q=Sq,
                                   causal=True)
        dtab = W.to_dev_i32(table)
    else:
        shape = (B, Hkv, cap, D)
        plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, cap, ragged=True, seq_q=Sq, causal=True)
        dtab = None
    kc = Guarded(shape, torch.bfloat16, W.to_dev(W.normal_bf16(sk, shape)))
    vc = Guarded(shape, torch.bfloat16, W.to_dev(W.normal_bf16(sv, shape)))
    kn = W.to_dev(W.normal_bf16(sk, (B, Hkv, Sq, D)))
    vn = W.to_dev(W.normal_bf16(sv, (B, Hkv, Sq, D)))
    out = Guarded((B, Hq, Sq, D), torch.bfloat16)
    ws = guarded_ws(plan)
    dl = W.to_dev_i32(lens)
    H.log(f"canary ragged/paged/step paged={paged}")
    if paged:
        twice(lambda: da.decode_attn_dense_paged(plan, q, kc.t, vc.t, dtab, dl, out.t, 0.1,
                                                 workspace=ws.t))
    else:
        twice(lambda: da.decode_attn_dense_ragged(plan, q, kc.t, vc.t, out.t, 0.1, dl,
                                                  workspace=ws.t))
    assert out.intact() and ws.intact() and kc.intact() and vc.intact()
    twice(lambda: da.decode_attn_dense_step(plan, q, kc.t, vc.t, kn, vn, dl, out.t, 0.1,
                                            block_table=dtab, workspace=ws.t))
    assert out.intact() and ws.intact() and kc.intact() and vc.intact()


def test_cache_writes_stay_inside(da):
    import torch
    # single-row append (linear and ring, positions out of range included) and
    # slot writes (padding tokens and slots past the pool included)
    B, Hkv, D, cap = 3, 2, 128, 64
    sq, sk, sv, _ = W.seeds(930)
    kc = Guarded((B, Hkv, cap, D), torch.bfloat16, W.to_dev(W.normal_bf16(sk, (B, Hkv, cap, D))))
    vc = Guarded((B, Hkv, cap, D), torch.bfloat16, W.to_dev(W.normal_bf16(sv, (B, Hkv, cap, D))))
    kn = W.to_dev(W.normal_bf16(sk, (B, Hkv, 1, D)))
    vn = W.to_dev(W.normal_bf16(sv, (B, Hkv, 1, D)))
    pos = W.to_dev_i32(np.array([cap - 1, cap, -1], np.int32))
    twice(lambda: da.decode_attn_append_kv(kc.t, vc.t, kn, vn, pos))
    twice(lambda: da.decode_attn_append_kv(kc.t, vc.t, kn, vn, pos, window=16, win_base=cap - 16))
    assert kc.intact() and vc.intact()
    num_pages, page = 5, 32
    kp = Guarded((num_pages, Hkv, page, D), torch.bfloat16)
    vp = Guarded((num_pages, Hkv, page, D), torch.bfloat16)
    kp.t.zero_()
    vp.t.zero_()
    N = 40
    kr = W.to_dev(W.normal_bf16(sk, (N, Hkv, D)))
    vr = W.to_dev(W.normal_bf16(sv, (N, Hkv, D)))
    slots = np.arange(N, dtype=np.int64) * 4 - 3      # -3, 1, 5, ..., 153 (past 160? no), ...
    slots[-1] = num_pages * page                        # one past the pool
    slots[-2] = num_pages * page - 1                    # the pool's last row
    ds = torch.from_numpy(slots).cuda()
    twice(lambda: da.decode_attn_write_slots(kp.t, vp.t, kr, vr, ds))
    assert kp.intact() and vp.intact()


def test_selection_writes_stay_inside(da):
    import torch
    B, n, k, window, topk = 3, 20000, 700, 64, 800
    rng = np.random.Generator(np.random.PCG64(940))
    scores = torch.from_numpy(rng.standard_normal((B, n), dtype=np.float32)).cuda()
    pos = W.to_dev_i32(np.array([5, 1000, -1], np.int32))
    sel = Guarded((B, topk), torch.int32)
    twice(lambda: da.decode_attn_build_selection(scores, pos, sel.t, n, k, window, n))
    assert sel.intact()
