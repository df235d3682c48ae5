"""Seeded synthetic inputs for single-token decode attention.

This module is the only code shared by the oracle side and the GPU side. It
draws inputs and nothing else: it holds none of the attention arithmetic.

Values are drawn with numpy's PCG64 generator as float32 standard normals,
multiplied by a standard deviation, and rounded to bfloat16 with IEEE
round-to-nearest-even. The workload seed is split (numpy SeedSequence) into
one child each for q, K, V and the selection, and every array is drawn in
fixed blocks from its own children, so large arrays fill in parallel and the
bits depend only on seed and shape. Every array is returned as raw bfloat16 bit patterns (uint16) so
that both sides see exactly the same bits.

Workloads (shapes follow the problem statement of the fuel-dispatch page
"DecodeFlashSpec", fields q, k, v, softmax_scale, k_len; the sparse layout
follows the metrale page "AttnV41", decode_fixed_topk and decode_prep):

* ``tiny``     dense, B=1 Hq=8 Hkv=8 D=64, capacity 512, k_len 300, scale 1/8
* ``gqa``      dense, B=8 Hq=32 Hkv=8 D=128, capacity 8192, k_len 4096;
               rows at and beyond k_len hold NaN
* ``long``     dense, B=4 Hq=64 Hkv=8 D=128, capacity = k_len = 131072
* ``batch``    dense, B=128 Hq=32 Hkv=8 D=128, capacity 2048, k_len 1537,
               values with standard deviation 0.5
* ``sparse``   B=4 Hq=64, one shared KV head of 65536 rows, D=128, topk 2048:
               128 window slots, then distinct random indices, then -1 pads
* ``ragged``   B=32 Hq=32 Hkv=8 D=128, one live length per sequence: 32768
               for sequence 0, log-uniform in [512, 32768] for the rest
* ``paged``    the same lengths over a paged cache of 64-row pages, shuffled
* ``verify``   the ``ragged`` batch with 4 query tokens per sequence (causal: the
               last 4 positions of each live prefix), as in verifying drafted tokens
* ``wide``     B=512 Hq=32 Hkv=8 D=128, one live length per sequence: 2048 for
               sequence 0, log-uniform in [128, 2048] for the rest (a wide serving
               batch: more key streams than the GPU has waves)
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (IEEE round-to-nearest-even); NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


BLOCK = 1 << 20  # elements per independently seeded block


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_bf16(seed: np.random.SeedSequence, shape, std: float = 1.0) -> np.ndarray:
    """float32 N(0, std^2) draws rounded to bfloat16 bits.

    The flat array is cut into blocks of BLOCK elements; block i is drawn from
    the i-th child of ``seed`` (``seed.spawn``), so the result depends only on
    the seed and the shape, never on how many threads fill it.
    """
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    nblocks = max(1, -(-n // BLOCK))
    children = seed.spawn(nblocks)

    def fill(i):
        lo, hi = i * BLOCK, min(n, (i + 1) * BLOCK)
        rng = np.random.Generator(np.random.PCG64(children[i]))
        x = rng.standard_normal(size=hi - lo, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[lo:hi] = f32_to_bf16_bits(x)

    if nblocks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblocks)))
    return out.reshape(shape)


def seeds(seed: int, n: int = 4):
    """Independent child seeds for q, K, V and the selection, in that order."""
    return np.random.SeedSequence(seed).spawn(n)


@dataclass
class DenseCase:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    capacity: int
    k_len: int
    scale: float            # the float32 value handed to the kernel
    std: float = 1.0
    poison: bool = False    # fill rows >= k_len with NaN
    seed: int = 0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def kv_bytes(self) -> int:
        """Live K+V bytes: the rows [0, k_len) of every (b, kv-head)."""
        return 2 * self.B * self.Hkv * self.k_len * self.D * 2

    def algorithmic_bytes(self) -> int:
        """Live K+V rows plus q plus out, all bfloat16."""
        return self.kv_bytes() + 2 * (self.B * self.Hq * self.D * 2)


@dataclass
class SparseCase:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    rows: int               # KV rows per (kv_batch, kv-head); also k_len
    topk: int
    window: int
    counts: tuple           # random (index) entries per token, before padding
    kv_batch: int = 1       # 1: rows shared by all tokens; B: one set per token
    scale: float = 0.0
    std: float = 1.0
    seed: int = 0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def valid_counts(self):
        return [self.window + c for c in self.counts]

    def algorithmic_bytes(self) -> int:
        """Gathered K+V rows (valid entries only) plus selection, q and out."""
        rows = sum(self.valid_counts())
        return (rows * self.Hkv * self.D * 2 * 2 + self.B * self.topk * 4
                + 2 * (self.B * self.Hq * self.D * 2))


def _f32(x: float) -> float:
    return float(np.float32(x))


DENSE_CASES = {
    "tiny": DenseCase("tiny", 1, 8, 8, 64, 512, 300, _f32(1.0 / 8.0), seed=1),
    "gqa": DenseCase("gqa", 8, 32, 8, 128, 8192, 4096, _f32(1.0 / math.sqrt(128)),
                     poison=True, seed=2),
    "long": DenseCase("long", 4, 64, 8, 128, 131072, 131072, _f32(1.0 / math.sqrt(128)), seed=3),
    "batch": DenseCase("batch", 128, 32, 8, 128, 2048, 1537, _f32(1.0 / math.sqrt(128)),
                       std=0.5, seed=4),
}

SPARSE_CASES = {
    "sparse": SparseCase("sparse", 4, 64, 1, 128, 65536, 2048, 128, (1920, 1920, 1920, 1920),
                         scale=_f32(1.0 / math.sqrt(128)), seed=5),
    "sparse_mixed": SparseCase("sparse_mixed", 4, 64, 1, 128, 65536, 2048, 128,
                               (1920, 1337, 960, 0), scale=_f32(1.0 / math.sqrt(128)), seed=5),
}


def dense_inputs(case: DenseCase, seed: int | None = None):
    """q [B,Hq,1,D], k and v [B,Hkv,capacity,D] as bfloat16 bits."""
    sq, sk, sv, _ = seeds(case.seed if seed is None else seed)
    q = normal_bf16(sq, (case.B, case.Hq, 1, case.D), case.std)
    k = normal_bf16(sk, (case.B, case.Hkv, case.capacity, case.D), case.std)
    v = normal_bf16(sv, (case.B, case.Hkv, case.capacity, case.D), case.std)
    if case.poison and case.k_len < case.capacity:
        k[:, :, case.k_len:, :] = BF16_NAN
        v[:, :, case.k_len:, :] = BF16_NAN
    return q, k, v


def selection(rng: np.random.Generator, B: int, rows: int, topk: int, window: int,
              counts) -> np.ndarray:
    """Padded selection [B, topk] int32.

    Per token: the window slots (the last ``window`` rows, ascending), then
    ``counts[b]`` distinct random indices from the rows before the window, in
    random order, then -1 up to ``topk``.
    """
    sel = np.full((B, topk), -1, dtype=np.int32)
    win = np.arange(rows - window, rows, dtype=np.int32)
    for b in range(B):
        n = int(counts[b])
        if window + n > topk:
            raise ValueError("selection wider than topk")
        idx = rng.choice(rows - window, size=n, replace=False).astype(np.int32)
        sel[b, :window] = win
        sel[b, window:window + n] = idx
    return sel


def sparse_inputs(case: SparseCase, seed: int | None = None):
    """q [B,Hq,1,D]; k, v [kv_batch,Hkv,rows,D]; sel [B,topk] int32."""
    sq, sk, sv, ss = seeds(case.seed if seed is None else seed)
    q = normal_bf16(sq, (case.B, case.Hq, 1, case.D), case.std)
    k = normal_bf16(sk, (case.kv_batch, case.Hkv, case.rows, case.D), case.std)
    v = normal_bf16(sv, (case.kv_batch, case.Hkv, case.rows, case.D), case.std)
    sel = selection(np.random.Generator(np.random.PCG64(ss)), case.B, case.rows, case.topk,
                    case.window, case.counts)
    return q, k, v, sel


@dataclass
class RaggedCase:
    """A batch whose sequences have different live lengths.

    Sequence 0 has the longest length ``len_hi``; the others are drawn
    log-uniformly from [len_lo, len_hi]. With ``page_size`` > 0 the cache is
    paged: one pool of pages [num_pages, Hkv, page_size, D] per K and V, each
    sequence holding ceil(len / page_size) distinct pages at shuffled positions
    of the pool, -1 in its block-table row past its length.
    """
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    len_lo: int
    len_hi: int             # also the capacity (rows per sequence) of the plan
    scale: float
    page_size: int = 0
    seq_q: int = 1          # query tokens per sequence (causal, the last seq_q positions)
    std: float = 1.0
    seed: int = 0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def max_pages(self) -> int:
        return -(-self.len_hi // self.page_size)

    def lengths(self) -> np.ndarray:
        return ragged_lengths(seeds(self.seed)[3], self.B, self.len_lo, self.len_hi)

    def algorithmic_bytes(self) -> int:
        """Live K+V rows of every sequence plus q and out (plus the block table if paged)."""
        n = int(self.lengths().sum())
        extra = self.B * self.max_pages * 4 if self.page_size else 0
        return (2 * n * self.Hkv * self.D * 2 + 2 * (self.B * self.Hq * self.seq_q * self.D * 2)
                + extra)


RAGGED_CASES = {
    "ragged": RaggedCase("ragged", 32, 32, 8, 128, 512, 32768, _f32(1.0 / math.sqrt(128)),
                         seed=6),
    "paged": RaggedCase("paged", 32, 32, 8, 128, 512, 32768, _f32(1.0 / math.sqrt(128)),
                        page_size=64, seed=6),
    "verify": RaggedCase("verify", 32, 32, 8, 128, 512, 32768, _f32(1.0 / math.sqrt(128)),
                         seq_q=4, seed=6),
    # a wide serving batch: 512 sequences of 128..2048 keys (4,096 streams)
    "wide": RaggedCase("wide", 512, 32, 8, 128, 128, 2048, _f32(1.0 / math.sqrt(128)), seed=7),
}


def ragged_lengths(seed: np.random.SeedSequence, B: int, lo: int, hi: int) -> np.ndarray:
    """int32 [B]: hi for sequence 0, then log-uniform integers in [lo, hi]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = np.exp(rng.uniform(math.log(lo), math.log(hi + 1), size=B))
    lens = np.clip(np.floor(x), lo, hi).astype(np.int32)
    lens[0] = hi
    return lens


def page_table(rng: np.random.Generator, lens, page_size: int, max_pages: int,
               spare: int = 0):
    """Block table [B, max_pages] int32 and the pool size.

    Sequence b needs ceil(lens[b] / page_size) pages; all pages of all
    sequences (plus ``spare`` unused ones) are one shuffled pool, handed out in
    a random order. Entries past a sequence's pages are -1.
    """
    need = [-(-int(n) // page_size) for n in lens]
    if max(need, default=0) > max_pages:
        raise ValueError("a sequence needs more pages than a block-table row holds")
    num_pages = sum(need) + spare
    perm = rng.permutation(num_pages).astype(np.int32)
    table = np.full((len(lens), max_pages), -1, dtype=np.int32)
    at = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[at:at + n]
        at += n
    return table, num_pages


def ragged_inputs(case: RaggedCase, seed: int | None = None):
    """Contiguous layout: q [B,Hq,seq_q,D], k, v [B,Hkv,len_hi,D], lengths [B] int32."""
    sq, sk, sv, sl = seeds(case.seed if seed is None else seed)
    q = normal_bf16(sq, (case.B, case.Hq, case.seq_q, case.D), case.std)
    k = normal_bf16(sk, (case.B, case.Hkv, case.len_hi, case.D), case.std)
    v = normal_bf16(sv, (case.B, case.Hkv, case.len_hi, case.D), case.std)
    return q, k, v, ragged_lengths(sl, case.B, case.len_lo, case.len_hi)


def paged_inputs(case: RaggedCase, seed: int | None = None, spare: int = 0):
    """Paged layout: q [B,Hq,seq_q,D], k_pages, v_pages [num_pages,Hkv,page_size,D],
    block table [B, max_pages] int32, lengths [B] int32."""
    sq, sk, sv, sl = seeds(case.seed if seed is None else seed)
    lens = ragged_lengths(sl, case.B, case.len_lo, case.len_hi)
    table, num_pages = page_table(np.random.Generator(np.random.PCG64(sl.spawn(1)[0])), lens,
                                  case.page_size, case.max_pages, spare)
    q = normal_bf16(sq, (case.B, case.Hq, case.seq_q, case.D), case.std)
    pool = (num_pages, case.Hkv, case.page_size, case.D)
    return q, normal_bf16(sk, pool, case.std), normal_bf16(sv, pool, case.std), table, lens


def random_case(seed: int, B: int, Hq: int, Hkv: int, D: int, cap: int, std: float = 1.0):
    """Small seeded q, K, V (bfloat16 bits) of arbitrary shape, for tests."""
    sq, sk, sv, _ = seeds(seed)
    return (normal_bf16(sq, (B, Hq, 1, D), std), normal_bf16(sk, (B, Hkv, cap, D), std),
            normal_bf16(sv, (B, Hkv, cap, D), std))


def repad(sel: np.ndarray, topk: int) -> np.ndarray:
    """The same valid prefix re-padded with -1 to a new width ``topk``."""
    B, old = sel.shape
    out = np.full((B, topk), -1, dtype=np.int32)
    keep = min(old, topk)
    out[:, :keep] = sel[:, :keep]
    if keep < old and (sel[:, keep:] >= 0).any():
        raise ValueError("re-padding would drop valid entries")
    return out


# --- device transfer of the drawn bits (torch only moves the bytes) ---------

def to_dev(bits: np.ndarray):
    """bfloat16 bit patterns (uint16) -> a bfloat16 device tensor with those bits."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_dev_i32(x: np.ndarray):
    """int32 host array -> int32 device tensor."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def from_dev(t) -> np.ndarray:
    """bfloat16 device tensor -> its bit patterns (uint16) on the host."""
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
