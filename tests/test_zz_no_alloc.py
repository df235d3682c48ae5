"""decode_attn_dense_static (the entry point that allocates nothing: its split
workspace is a static device array of the library) against decode_attn_dense
with a caller-owned workspace: bit-identical output on two calls in a row, the
second with a smaller problem, plus the size limit."""

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


def both(da, seed, B, Hq, Hkv, D, cap, k_len, **kw):
    import torch
    q, k, v = W.random_case(seed, B, Hq, Hkv, D, cap)
    plan = da.decode_attn_plan(B, Hq, Hkv, D, cap, k_len, **kw)
    dq, dk, dv = H.to_dev(q), H.to_dev(k), H.to_dev(v)
    ref_out = torch.empty((B, Hq, 1, D), dtype=torch.bfloat16, device="cuda")
    da.decode_attn_dense(plan, dq, dk, dv, ref_out, 0.088388, k_len, da.workspace_for(plan))
    out = torch.full((B, Hq, 1, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    da.decode_attn_dense_static(plan, dq, dk, dv, out, 0.088388, k_len)
    torch.cuda.synchronize()
    return plan, H.from_dev(out), H.from_dev(ref_out), oracle.dense(q, k, v, 0.088388, k_len)


def test_static_workspace_matches_the_caller_workspace_twice(da):
    # first call: 16 splits over 4 x 4 units (the static array holds the partials)
    H.log("static workspace: first call (B4 Hq32 Hkv4 D128 k_len 20000, 16 splits)")
    plan, got, want, ref = both(da, 800, 4, 32, 4, 128, 24576, 20000, force_splits=16)
    assert plan.num_splits_max > 1 and plan.workspace_bytes > 0
    assert np.array_equal(got, want)
    H.check_tolerance(got, ref, "static, first call")
    # second call: a smaller problem (fewer rows, fewer splits, D = 64) reusing the array
    H.log("static workspace: second call (B2 Hq8 Hkv2 D64 k_len 3000, 3 splits)")
    plan2, got2, want2, ref2 = both(da, 801, 2, 8, 2, 64, 4096, 3000, force_splits=3)
    assert 1 < plan2.num_splits_max < plan.num_splits_max
    assert plan2.workspace_bytes < plan.workspace_bytes
    assert np.array_equal(got2, want2)
    H.check_tolerance(got2, ref2, "static, second call")


def test_unsplit_plans_need_no_workspace(da):
    plan, got, want, ref = both(da, 802, 2, 8, 8, 128, 1000, 700)
    assert plan.workspace_bytes == 0
    assert np.array_equal(got, want)


def test_plans_beyond_the_static_size_are_rejected(da):
    import torch
    # 2 x 64 heads x 1024 splits x 130 floats = 68 MB of partials > 16 MiB
    plan = da.decode_attn_plan(2, 64, 8, 128, 1 << 17, 1 << 17, force_chunk=128)
    assert plan.workspace_bytes > (16 << 20)
    q = torch.zeros((2, 64, 1, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((2, 8, 1 << 17, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros_like(q)
    with pytest.raises(da.DecodeAttnError) as ei:
        da.decode_attn_dense_static(plan, q, kv, kv, out, 0.1, 1 << 17)
    assert ei.value.status == 3 and "static workspace" in str(ei.value)
