"""Single-token decode attention on MI355X: a thin Python binding of the C ABI.

Every compute step runs in the HIP kernels of ``libdecode_attn.so``; this module
only marshals arguments (tensor pointers, sizes, the current HIP stream) into
the C functions declared in ``include/decode_attn.h`` and checks that the
tensors it is handed match the plan, so that no kernel is ever given a buffer
smaller than the plan implies. PyTorch provides device memory and streams.

Names mirror the C ABI: ``decode_attn_plan``, ``decode_attn_dense``,
``decode_attn_sparse``, ``decode_attn_status_str``, ``decode_attn_last_error``.
If the shared library has not been built, loading it raises: there is no
fallback implementation.
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "DecodeAttnError", "Problem", "Plan", "library", "library_path",
    "decode_attn_plan", "decode_attn_dense", "decode_attn_dense_static", "decode_attn_dense_devlen",
    "decode_attn_dense_ragged",
    "decode_attn_dense_paged", "decode_attn_dense_step", "decode_attn_sparse",
    "decode_attn_build_selection", "decode_attn_build_selection_ws", "decode_attn_select_workspace",
    "SelectProblem", "decode_attn_append_kv", "AppendProblem",
    "decode_attn_write_slots", "SlotProblem",
    "decode_attn_set_timing_events", "decode_attn_read_probe", "decode_attn_status_str",
    "decode_attn_last_error",
    "workspace_for",
    "EXPORTED_SYMBOLS", "PreparedCall",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libdecode_attn.so")

DA_OK, DA_ERR_INVALID_ARG, DA_ERR_UNSUPPORTED, DA_ERR_WORKSPACE, DA_ERR_HIP = range(5)

EXPORTED_SYMBOLS = ("decode_attn_plan", "decode_attn_dense", "decode_attn_dense_static",
                    "decode_attn_dense_devlen",
                    "decode_attn_dense_ragged", "decode_attn_dense_paged", "decode_attn_dense_step",
                    "decode_attn_read_probe",
                    "decode_attn_sparse", "decode_attn_build_selection",
                    "decode_attn_build_selection_ws", "decode_attn_select_workspace",
                    "decode_attn_append_kv",
                    "decode_attn_write_slots",
                    "decode_attn_set_timing_events", "decode_attn_status_str",
                    "decode_attn_last_error")


class Problem(ctypes.Structure):
    """Mirror of ``decode_attn_problem``."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("seq_q", ctypes.c_int32), ("capacity", ctypes.c_int64),
        ("max_k_len", ctypes.c_int64), ("topk_max", ctypes.c_int32),
        ("kv_batch", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("has_alibi", ctypes.c_int32), ("window_left", ctypes.c_int64),
        ("window_right", ctypes.c_int64), ("has_softcap", ctypes.c_int32),
        ("num_cus", ctypes.c_int32), ("force_splits", ctypes.c_int32),
        ("force_chunk", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int64),
        ("ragged", ctypes.c_int32),
    ]


class Plan(ctypes.Structure):
    """Mirror of ``decode_attn_plan_t`` (plain data)."""
    _fields_ = [
        ("prob", Problem), ("group", ctypes.c_int32), ("num_splits_max", ctypes.c_int32),
        ("chunk", ctypes.c_int32), ("num_cus", ctypes.c_int32), ("kind", ctypes.c_int32),
        ("balanced_wgs", ctypes.c_int32), ("workspace_bytes", ctypes.c_uint64),
    ]

    @property
    def sparse(self) -> bool:
        return self.kind == 1


class SelectProblem(ctypes.Structure):
    """Mirror of ``decode_attn_select_problem``."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_idx", ctypes.c_int32), ("score_stride", ctypes.c_int64),
        ("k_idx", ctypes.c_int32), ("window", ctypes.c_int32), ("win_base", ctypes.c_int64),
        ("topk", ctypes.c_int32),
    ]


class AppendProblem(ctypes.Structure):
    """Mirror of ``decode_attn_append_problem``."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("capacity", ctypes.c_int64), ("window", ctypes.c_int32), ("win_base", ctypes.c_int64),
    ]


class SlotProblem(ctypes.Structure):
    """Mirror of ``decode_attn_slot_problem``."""
    _fields_ = [
        ("num_tokens", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int64),
    ]


class DecodeAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{_status_name(status)}: {message}")


_lib = None


def library():
    """Load ``libdecode_attn.so`` (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(
                f"{library_path} is missing: build it with `python -m decode_attention_05_amd.build`"
                " (there is no fallback implementation)")
        lib = ctypes.CDLL(library_path)
        P = ctypes.c_void_p
        lib.decode_attn_plan.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(Plan)]
        lib.decode_attn_plan.restype = ctypes.c_int
        lib.decode_attn_dense.argtypes = [ctypes.POINTER(Plan), P, P, P, P, ctypes.c_float,
                                          ctypes.c_int64, P, ctypes.c_size_t, P]
        lib.decode_attn_dense.restype = ctypes.c_int
        lib.decode_attn_dense_static.argtypes = [ctypes.POINTER(Plan), P, P, P, P, ctypes.c_float,
                                                 ctypes.c_int64, P]
        lib.decode_attn_dense_static.restype = ctypes.c_int
        lib.decode_attn_dense_devlen.argtypes = [ctypes.POINTER(Plan), P, P, P, P, ctypes.c_float,
                                                 P, P, ctypes.c_size_t, P]
        lib.decode_attn_dense_devlen.restype = ctypes.c_int
        lib.decode_attn_dense_ragged.argtypes = [ctypes.POINTER(Plan), P, P, P, P, ctypes.c_float,
                                                 P, ctypes.c_int32, P, ctypes.c_size_t, P]
        lib.decode_attn_dense_ragged.restype = ctypes.c_int
        lib.decode_attn_dense_paged.argtypes = [ctypes.POINTER(Plan), P, P, P, P, P,
                                                ctypes.c_int32, P, ctypes.c_float, P,
                                                ctypes.c_size_t, P]
        lib.decode_attn_dense_paged.restype = ctypes.c_int
        lib.decode_attn_dense_step.argtypes = [ctypes.POINTER(Plan), P, P, P, P, P, P, P,
                                               ctypes.c_int32, P, ctypes.c_float, P,
                                               ctypes.c_size_t, P]
        lib.decode_attn_dense_step.restype = ctypes.c_int
        lib.decode_attn_read_probe.argtypes = [P, ctypes.c_size_t, P, P]
        lib.decode_attn_read_probe.restype = ctypes.c_int
        lib.decode_attn_sparse.argtypes = [ctypes.POINTER(Plan), P, P, P, P, ctypes.c_int32, P,
                                           ctypes.c_float, ctypes.c_int64, P, ctypes.c_size_t, P]
        lib.decode_attn_sparse.restype = ctypes.c_int
        lib.decode_attn_build_selection.argtypes = [ctypes.POINTER(SelectProblem), P, P, P, P]
        lib.decode_attn_build_selection.restype = ctypes.c_int
        lib.decode_attn_build_selection_ws.argtypes = [ctypes.POINTER(SelectProblem), P, P, P, P,
                                                       ctypes.c_size_t, P]
        lib.decode_attn_build_selection_ws.restype = ctypes.c_int
        lib.decode_attn_select_workspace.argtypes = [ctypes.POINTER(SelectProblem),
                                                     ctypes.POINTER(ctypes.c_size_t)]
        lib.decode_attn_select_workspace.restype = ctypes.c_int
        lib.decode_attn_append_kv.argtypes = [ctypes.POINTER(AppendProblem), P, P, P, P, P, P]
        lib.decode_attn_append_kv.restype = ctypes.c_int
        lib.decode_attn_write_slots.argtypes = [ctypes.POINTER(SlotProblem), P, P, P, P, P, P]
        lib.decode_attn_write_slots.restype = ctypes.c_int
        lib.decode_attn_set_timing_events.argtypes = [P, P]
        lib.decode_attn_set_timing_events.restype = ctypes.c_int
        lib.decode_attn_status_str.argtypes = [ctypes.c_int]
        lib.decode_attn_status_str.restype = ctypes.c_char_p
        lib.decode_attn_last_error.argtypes = []
        lib.decode_attn_last_error.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def _status_name(s: int) -> str:
    try:
        return library().decode_attn_status_str(s).decode()
    except Exception:  # pragma: no cover - only while reporting another error
        return f"status {s}"


def decode_attn_read_probe(buf, sink, stream=None):
    """Read all of ``buf`` (a contiguous device tensor, a multiple of 16 bytes) the
    way the attention kernels stream K and V, folding it into ``sink`` (a
    one-element int32 device tensor): the measured streaming-read ceiling."""
    import torch
    if not (isinstance(buf, torch.Tensor) and buf.is_cuda and buf.is_contiguous()):
        raise TypeError("buf must be a contiguous device tensor")
    _tensor_ptr(sink, "sink", (1,), torch.int32)
    _check(library().decode_attn_read_probe(ctypes.c_void_p(buf.data_ptr()),
                                            buf.numel() * buf.element_size(),
                                            ctypes.c_void_p(sink.data_ptr()), _stream_ptr(stream)))


def decode_attn_set_timing_events(ev_before, ev_after):
    """Record raw hipEvent_t handles around every later partial-kernel launch on this thread."""
    _check(library().decode_attn_set_timing_events(ev_before, ev_after))


def decode_attn_status_str(s: int) -> str:
    return library().decode_attn_status_str(s).decode()


def decode_attn_last_error() -> str:
    return library().decode_attn_last_error().decode()


def _check(status: int):
    if status != DA_OK:
        raise DecodeAttnError(status, decode_attn_last_error())


class PreparedCall:
    """One library call with its arguments checked and marshalled once (the
    ``prepare=True`` form of every compute wrapper). Calling it enqueues the
    same call again on the same buffers and on the stream chosen when it was
    prepared (by default torch's current stream at that moment), without
    re-checking shapes in Python; it keeps the plan, the problem struct and the
    tensors alive."""

    __slots__ = ("_fn", "_args", "_keep", "_result")

    def __init__(self, fn, args, keep, result):
        self._fn, self._args, self._keep, self._result = fn, args, keep, result

    def __call__(self):
        status = self._fn(*self._args)
        if status != DA_OK:
            raise DecodeAttnError(status, decode_attn_last_error())
        return self._result


def _run(fn, args, result, prepare, keep):
    if prepare:
        return PreparedCall(fn, tuple(args), keep, result)
    _check(fn(*args))
    return result


def decode_attn_plan(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                     capacity: int, max_k_len: int | None = None, *, topk_max: int = 0,
                     kv_batch: int = 0, seq_q: int = 1, causal: bool = False,
                     has_alibi: bool = False, window_left: int = -1, window_right: int = -1,
                     has_softcap: bool = False, num_cus: int = 0, force_splits: int = 0,
                     force_chunk: int = 0, page_size: int = 0, max_pages_per_seq: int = 0,
                     num_pages: int = 0, ragged: bool = False) -> Plan:
    """Validate a problem and return its plan (see ``decode_attn_plan`` in the header)."""
    prob = Problem(batch, num_q_heads, num_kv_heads, head_dim, seq_q, capacity,
                   capacity if max_k_len is None else max_k_len, topk_max, kv_batch,
                   int(bool(causal)), int(bool(has_alibi)), window_left, window_right,
                   int(bool(has_softcap)), num_cus, force_splits, force_chunk, page_size,
                   max_pages_per_seq, num_pages, int(bool(ragged)))
    plan = Plan()
    _check(library().decode_attn_plan(ctypes.byref(prob), ctypes.byref(plan)))
    return plan


def workspace_for(plan: Plan, device="cuda"):
    """A device byte buffer of the plan's workspace size (None when it needs none)."""
    import torch
    n = int(plan.workspace_bytes)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=device)


def _tensor_ptr(t, name, shape, dtype):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _ws_ptr(plan, workspace):
    if workspace is None:
        return None, 0
    import torch
    if not (isinstance(workspace, torch.Tensor) and workspace.is_cuda and workspace.is_contiguous()):
        raise TypeError("workspace must be a contiguous device tensor")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def _stream_ptr(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def decode_attn_dense(plan: Plan, q, k, v, out, softmax_scale: float, k_len: int,
                      workspace=None, stream=None, prepare=False):
    """Enqueue dense decode attention on ``stream`` (default: torch's current stream).
    With ``prepare=True`` return a PreparedCall instead of calling."""
    import torch
    p = plan.prob
    B, Hq, Hkv, D, cap = p.batch, p.num_q_heads, p.num_kv_heads, p.head_dim, p.capacity
    Sq = p.seq_q
    bf = torch.bfloat16
    args = (_tensor_ptr(q, "q", (B, Hq, Sq, D), bf), _tensor_ptr(k, "k", (B, Hkv, cap, D), bf),
            _tensor_ptr(v, "v", (B, Hkv, cap, D), bf), _tensor_ptr(out, "out", (B, Hq, Sq, D), bf))
    ws, wsb = _ws_ptr(plan, workspace)
    return _run(library().decode_attn_dense,
                (ctypes.byref(plan), *args, float(softmax_scale), int(k_len), ws, wsb,
                 _stream_ptr(stream)), out, prepare, (plan, q, k, v, out, workspace))


def decode_attn_dense_static(plan: Plan, q, k, v, out, softmax_scale: float, k_len: int,
                             stream=None, prepare=False):
    """decode_attn_dense with the library's static device workspace (no caller
    workspace; for callers that cannot allocate). Calls that overlap on one
    device race."""
    import torch
    p = plan.prob
    B, Hq, Hkv, D, cap = p.batch, p.num_q_heads, p.num_kv_heads, p.head_dim, p.capacity
    Sq = p.seq_q
    bf = torch.bfloat16
    args = (_tensor_ptr(q, "q", (B, Hq, Sq, D), bf), _tensor_ptr(k, "k", (B, Hkv, cap, D), bf),
            _tensor_ptr(v, "v", (B, Hkv, cap, D), bf), _tensor_ptr(out, "out", (B, Hq, Sq, D), bf))
    return _run(library().decode_attn_dense_static,
                (ctypes.byref(plan), *args, float(softmax_scale), int(k_len), _stream_ptr(stream)),
                out, prepare, (plan, q, k, v, out))


def decode_attn_dense_devlen(plan: Plan, q, k, v, out, softmax_scale: float, k_len_dev,
                             workspace=None, stream=None, prepare=False):
    """Dense decode attention whose live length is the int32 in ``k_len_dev`` (a
    one-element device tensor), read by the kernel: capturable once, replayable."""
    import torch
    p = plan.prob
    B, Hq, Hkv, D, cap = p.batch, p.num_q_heads, p.num_kv_heads, p.head_dim, p.capacity
    Sq = p.seq_q
    bf = torch.bfloat16
    args = (_tensor_ptr(q, "q", (B, Hq, Sq, D), bf), _tensor_ptr(k, "k", (B, Hkv, cap, D), bf),
            _tensor_ptr(v, "v", (B, Hkv, cap, D), bf), _tensor_ptr(out, "out", (B, Hq, Sq, D), bf))
    klen = _tensor_ptr(k_len_dev, "k_len_dev", (1,), torch.int32)
    ws, wsb = _ws_ptr(plan, workspace)
    return _run(library().decode_attn_dense_devlen,
                (ctypes.byref(plan), *args, float(softmax_scale), klen, ws, wsb,
                 _stream_ptr(stream)), out, prepare, (plan, q, k, v, out, k_len_dev, workspace))


def _lens_ptr(k_lens, B, stride):
    import torch
    if not (isinstance(k_lens, torch.Tensor) and k_lens.is_cuda and k_lens.dtype == torch.int32
            and k_lens.is_contiguous()):
        raise TypeError("k_lens must be a contiguous int32 device tensor")
    if k_lens.numel() < (B - 1) * stride + 1:
        raise ValueError(f"k_lens holds {k_lens.numel()} values, needs {(B - 1) * stride + 1}")
    return k_lens.data_ptr()


def decode_attn_dense_ragged(plan: Plan, q, k, v, out, softmax_scale: float, k_lens,
                             k_lens_stride: int = 1, workspace=None, stream=None,
                             prepare=False):
    """Dense decode attention with sequence b's length k_lens[b * k_lens_stride] (device)."""
    import torch
    p = plan.prob
    B, Hq, Hkv, D, cap = p.batch, p.num_q_heads, p.num_kv_heads, p.head_dim, p.capacity
    Sq = p.seq_q
    bf = torch.bfloat16
    args = (_tensor_ptr(q, "q", (B, Hq, Sq, D), bf), _tensor_ptr(k, "k", (B, Hkv, cap, D), bf),
            _tensor_ptr(v, "v", (B, Hkv, cap, D), bf), _tensor_ptr(out, "out", (B, Hq, Sq, D), bf))
    lens = _lens_ptr(k_lens, B, k_lens_stride)
    ws, wsb = _ws_ptr(plan, workspace)
    return _run(library().decode_attn_dense_ragged,
                (ctypes.byref(plan), *args, float(softmax_scale), lens, int(k_lens_stride), ws,
                 wsb, _stream_ptr(stream)), out, prepare, (plan, q, k, v, out, k_lens, workspace))


def decode_attn_dense_paged(plan: Plan, q, k_pages, v_pages, block_table, k_lens, out,
                            softmax_scale: float, k_lens_stride: int = 1, workspace=None,
                            stream=None, prepare=False):
    """Dense decode attention over page pools [num_pages,Hkv,page_size,D] through
    block_table [B, max_pages_per_seq] (int32, device)."""
    import torch
    p = plan.prob
    B, Hq, Hkv, D, Sq = p.batch, p.num_q_heads, p.num_kv_heads, p.head_dim, p.seq_q
    bf = torch.bfloat16
    pool = (p.num_pages, Hkv, p.page_size, D)
    qp = _tensor_ptr(q, "q", (B, Hq, Sq, D), bf)
    kp = _tensor_ptr(k_pages, "k_pages", pool, bf)
    vp = _tensor_ptr(v_pages, "v_pages", pool, bf)
    bt = _tensor_ptr(block_table, "block_table", (B, p.max_pages_per_seq), torch.int32)
    lens = _lens_ptr(k_lens, B, k_lens_stride)
    op = _tensor_ptr(out, "out", (B, Hq, Sq, D), bf)
    ws, wsb = _ws_ptr(plan, workspace)
    return _run(library().decode_attn_dense_paged,
                (ctypes.byref(plan), qp, kp, vp, bt, lens, int(k_lens_stride), op,
                 float(softmax_scale), ws, wsb, _stream_ptr(stream)), out, prepare,
                (plan, q, k_pages, v_pages, block_table, k_lens, out, workspace))


def decode_attn_dense_step(plan: Plan, q, k_cache, v_cache, k_new, v_new, k_lens, out,
                           softmax_scale: float, block_table=None, k_lens_stride: int = 1,
                           workspace=None, stream=None, prepare=False):
    """Write the pass's new K/V rows [B, Hkv, Sq, D] at rows [k_len - Sq, k_len) of
    each sequence's cache and attend, in one call (contiguous caches with a
    ragged plan, or page pools with a paged plan and ``block_table``)."""
    import torch
    p = plan.prob
    B, Hq, Hkv, D, Sq = p.batch, p.num_q_heads, p.num_kv_heads, p.head_dim, p.seq_q
    bf = torch.bfloat16
    if p.page_size > 0:
        shape = (p.num_pages, Hkv, p.page_size, D)
        bt = _tensor_ptr(block_table, "block_table", (B, p.max_pages_per_seq), torch.int32)
    else:
        shape = (B, Hkv, p.capacity, D)
        if block_table is not None:
            raise ValueError("block_table is for paged plans")
        bt = None
    qp = _tensor_ptr(q, "q", (B, Hq, Sq, D), bf)
    kc = _tensor_ptr(k_cache, "k_cache", shape, bf)
    vc = _tensor_ptr(v_cache, "v_cache", shape, bf)
    kn = _tensor_ptr(k_new, "k_new", (B, Hkv, Sq, D), bf)
    vn = _tensor_ptr(v_new, "v_new", (B, Hkv, Sq, D), bf)
    lens = _lens_ptr(k_lens, B, k_lens_stride)
    op = _tensor_ptr(out, "out", (B, Hq, Sq, D), bf)
    ws, wsb = _ws_ptr(plan, workspace)
    return _run(library().decode_attn_dense_step,
                (ctypes.byref(plan), qp, kc, vc, kn, vn, bt, lens, int(k_lens_stride), op,
                 float(softmax_scale), ws, wsb, _stream_ptr(stream)), out, prepare,
                (plan, q, k_cache, v_cache, k_new, v_new, block_table, k_lens, out, workspace))


def decode_attn_sparse(plan: Plan, q, k, v, sel, topk: int, out, softmax_scale: float,
                       k_len: int | None = None, workspace=None, stream=None, prepare=False):
    """Enqueue index-selected sparse decode attention (sel: int32 [B, topk])."""
    import torch
    p = plan.prob
    B, Hq, Hkv, D, cap = p.batch, p.num_q_heads, p.num_kv_heads, p.head_dim, p.capacity
    bf = torch.bfloat16
    args = (_tensor_ptr(q, "q", (B, Hq, 1, D), bf),
            _tensor_ptr(k, "k", (p.kv_batch, Hkv, cap, D), bf),
            _tensor_ptr(v, "v", (p.kv_batch, Hkv, cap, D), bf),
            _tensor_ptr(sel, "sel", (B, topk), torch.int32))
    outp = _tensor_ptr(out, "out", (B, Hq, 1, D), bf)
    ws, wsb = _ws_ptr(plan, workspace)
    return _run(library().decode_attn_sparse,
                (ctypes.byref(plan), *args, int(topk), outp, float(softmax_scale),
                 int(cap if k_len is None else k_len), ws, wsb, _stream_ptr(stream)), out,
                prepare, (plan, q, k, v, sel, out, workspace))


def _select_problem(scores, sel, n_idx, k_idx, window, win_base):
    B, topk = sel.shape
    return SelectProblem(B, int(n_idx), int(scores.shape[1]), int(k_idx), int(window),
                         int(win_base), int(topk))


def decode_attn_build_selection(scores, pos, sel, n_idx: int, k_idx: int, window: int,
                                win_base: int, stream=None, prepare=False):
    """Fill ``sel`` [B, topk] int32 on the device: window ring rows, then the k_idx
    best-scoring candidates of ``scores`` [B, >= n_idx] fp32, then -1 (``pos`` [B] int32)."""
    import torch
    B, topk = sel.shape
    stride = scores.shape[1]
    prob = _select_problem(scores, sel, n_idx, k_idx, window, win_base)
    sp = _tensor_ptr(scores, "scores", (B, stride), torch.float32)
    pp = _tensor_ptr(pos, "pos", (B,), torch.int32)
    selp = _tensor_ptr(sel, "sel", (B, topk), torch.int32)
    return _run(library().decode_attn_build_selection,
                (ctypes.byref(prob), sp, pp, selp, _stream_ptr(stream)), sel, prepare,
                (prob, scores, pos, sel))


def decode_attn_select_workspace(batch: int, n_idx: int, k_idx: int, window: int, topk: int,
                                 score_stride: int | None = None) -> int:
    """Workspace bytes of decode_attn_build_selection_ws for this shape (host only)."""
    stride = n_idx + (-n_idx) % 4 if score_stride is None else score_stride
    prob = SelectProblem(int(batch), int(n_idx), int(max(stride, 4)), int(k_idx), int(window), 0,
                         int(topk))
    n = ctypes.c_size_t(0)
    _check(library().decode_attn_select_workspace(ctypes.byref(prob), ctypes.byref(n)))
    return int(n.value)


def decode_attn_build_selection_ws(scores, pos, sel, n_idx: int, k_idx: int, window: int,
                                   win_base: int, workspace=None, stream=None, prepare=False):
    """decode_attn_build_selection with several workgroups per token and a
    caller-owned device workspace of decode_attn_select_workspace bytes."""
    import torch
    B, topk = sel.shape
    stride = scores.shape[1]
    prob = _select_problem(scores, sel, n_idx, k_idx, window, win_base)
    sp = _tensor_ptr(scores, "scores", (B, stride), torch.float32)
    pp = _tensor_ptr(pos, "pos", (B,), torch.int32)
    selp = _tensor_ptr(sel, "sel", (B, topk), torch.int32)
    if workspace is None:
        ws, wsb = None, 0
    else:
        if not (isinstance(workspace, torch.Tensor) and workspace.is_cuda
                and workspace.is_contiguous()):
            raise TypeError("workspace must be a contiguous device tensor")
        ws, wsb = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    return _run(library().decode_attn_build_selection_ws,
                (ctypes.byref(prob), sp, pp, selp, ws, wsb, _stream_ptr(stream)), sel, prepare,
                (prob, scores, pos, sel, workspace))


def decode_attn_append_kv(k_cache, v_cache, k_new, v_new, pos, window: int = 0, win_base: int = 0,
                          stream=None, prepare=False):
    """Write token b's rows k_new/v_new [B,Hkv,1,D] into the caches [B,Hkv,capacity,D] at
    row pos[b] (or win_base + pos[b] % window); ``pos`` is an int32 device tensor [B]."""
    import torch
    B, Hkv, cap, D = k_cache.shape
    bf = torch.bfloat16
    prob = AppendProblem(B, Hkv, D, cap, int(window), int(win_base))
    args = (_tensor_ptr(k_cache, "k_cache", (B, Hkv, cap, D), bf),
            _tensor_ptr(v_cache, "v_cache", (B, Hkv, cap, D), bf),
            _tensor_ptr(k_new, "k_new", (B, Hkv, 1, D), bf),
            _tensor_ptr(v_new, "v_new", (B, Hkv, 1, D), bf),
            _tensor_ptr(pos, "pos", (B,), torch.int32))
    return _run(library().decode_attn_append_kv, (ctypes.byref(prob), *args, _stream_ptr(stream)),
                (k_cache, v_cache), prepare, (prob, k_cache, v_cache, k_new, v_new, pos))


def decode_attn_write_slots(k_pages, v_pages, k_rows, v_rows, slot_mapping, stream=None,
                            prepare=False):
    """Write token n's rows k_rows/v_rows [N, Hkv, D] at slot slot_mapping[n] (int64
    device tensor [N]) of the page pools [num_pages, Hkv, page_size, D]: row
    slot % page_size of page slot // page_size; negative slots write nothing."""
    import torch
    num_pages, Hkv, page_size, D = k_pages.shape
    N = k_rows.shape[0]
    bf = torch.bfloat16
    prob = SlotProblem(N, Hkv, D, page_size, num_pages)
    args = (_tensor_ptr(k_pages, "k_pages", (num_pages, Hkv, page_size, D), bf),
            _tensor_ptr(v_pages, "v_pages", (num_pages, Hkv, page_size, D), bf),
            _tensor_ptr(k_rows, "k_rows", (N, Hkv, D), bf),
            _tensor_ptr(v_rows, "v_rows", (N, Hkv, D), bf),
            _tensor_ptr(slot_mapping, "slot_mapping", (N,), torch.int64))
    return _run(library().decode_attn_write_slots, (ctypes.byref(prob), *args, _stream_ptr(stream)),
                (k_pages, v_pages), prepare, (prob, k_pages, v_pages, k_rows, v_rows, slot_mapping))
