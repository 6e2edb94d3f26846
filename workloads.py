"""Seeded synthetic inputs for one context-parallel rank's share of THD attention.

This module holds random draws, document-length recipes and bf16 rounding only.
It computes nothing of the method itself (no partitioning, no reordering, no
attention): both the CPU oracle's tests and the HIP path take their inputs from
here, and that is the only thing the two sides share.

Recipes (the pages fix none of the seeds or distributions; these follow the
workload descriptions of the five measured configurations):

* ``tiny_t28``  tiny: three documents of actual lengths 5, 12, 7 in padded slots
  ``[0, 8, 20, 28]`` (pads between documents), 2 q / 2 kv heads, head dim 16,
  all tensors N(0, 1).
* ``t8192_mha16``  T = 8192, lengths ``4 * round(U/4)`` with U uniform on
  [256, 2048], no pads, 16 q / 16 kv heads, head dim 128, Q/K/V ~ 0.5 N(0, 1).
* ``t32768_gqa32x8``  T = 32768, actual lengths log-normal (median 1024, sigma 1)
  clipped to [64, 8192], slots padded up to a multiple of 8, 32 q / 8 kv heads.
* ``t131072_gqa64x8``  T = 131072, lengths uniform integers on [1, 16384], no pads,
  64 q / 8 kv heads.
* ``dynamic_t``  16 micro-batches, active T = 64 * U with U uniform on [64, 1024],
  lengths as t32768_gqa32x8 but clipped to [32, 8192], on a 65536-token capacity.
* ``t1m_10k_docs`` T = 1,048,576 in 10,000 documents: 8 times a uniformly random
  composition of 131072 into 10,000 positive parts (partition indices only).

In every recipe the last document is trimmed so the padded lengths sum to T
(its actual length becomes ``min(actual, padded)``).

Tensor values are drawn block-wise: rows ``[b*4096, (b+1)*4096)`` of tensor
``tid`` (Q=1, K=2, V=3, dO=4) come from ``default_rng([*seed_key, tid, b])``,
so a subset of rows can be produced without materialising the whole tensor.
Values are float32 draws, scaled, then rounded to bf16 (round to nearest even);
Q, K, V and dO are all in physical token order ``[T, H, D]``.
"""
from __future__ import annotations

import math
import os
from dataclasses import dataclass, field

import numpy as np

TID_Q, TID_K, TID_V, TID_DO = 1, 2, 3, 4
ROW_BLOCK = 4096


# ----------------------------------------------------------------------------
# bf16 helpers (bit manipulation of IEEE float32, round to nearest even)
# ----------------------------------------------------------------------------
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # u + 0x7FFF + lsb stays below 2^32 for every finite value (the largest is 0x7F7FFFFF); NaNs are set below
    r = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    bits = (r >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        bits[nan] = np.uint16(0x7FC0)
    return bits


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values that are exactly representable in bf16."""
    return bf16_bits_to_f32(to_bf16_bits(x))


# ----------------------------------------------------------------------------
# document layouts
# ----------------------------------------------------------------------------
def _trim(padded: list[int], actual: list[int], total: int):
    """Trim the list of (padded, actual) lengths so the padded sum is exactly total."""
    out_p, out_a, run = [], [], 0
    for p, a in zip(padded, actual):
        if run + p >= total:
            p_last = total - run
            out_p.append(p_last)
            out_a.append(min(a, p_last))
            run = total
            break
        out_p.append(p)
        out_a.append(a)
        run += p
    assert run == total
    return out_p, out_a


def _cu(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def docs_uniform_mult4(rng, total, lo=256, hi=2048):
    padded = []
    while sum(padded) < total:
        u = int(rng.integers(lo, hi + 1))
        padded.append(4 * int(round(u / 4)))
    return _trim(padded, list(padded), total)


def docs_lognormal(rng, total, lo, hi, mult=8, median=1024.0, sigma=1.0):
    padded, actual = [], []
    while sum(padded) < total:
        a = int(np.clip(round(math.exp(rng.normal(math.log(median), sigma))), lo, hi))
        actual.append(a)
        padded.append(mult * ((a + mult - 1) // mult))
    return _trim(padded, actual, total)


def docs_uniform_any(rng, total, lo=1, hi=16384):
    padded = []
    while sum(padded) < total:
        padded.append(int(rng.integers(lo, hi + 1)))
    return _trim(padded, list(padded), total)


def docs_composition(rng, units, parts, unit_len):
    cuts = np.sort(rng.choice(np.arange(1, units), size=parts - 1, replace=False))
    sizes = np.diff(np.concatenate([[0], cuts, [units]])) * unit_len
    return [int(s) for s in sizes], [int(s) for s in sizes]


# ----------------------------------------------------------------------------
# tensor values
# ----------------------------------------------------------------------------
def normal_rows(seed_key, tid, n_rows, heads, dim, scale=1.0, rows=None, bf16=True):
    """Rows of an [n_rows, heads, dim] N(0,1)*scale tensor, drawn block-wise.

    ``rows`` (int array) selects physical rows; None means all of them.  Blocks
    are independent draws, so they are generated (and rounded) on a few threads.
    """
    key = list(seed_key) if isinstance(seed_key, (list, tuple)) else [int(seed_key)]
    whole = rows is None
    if whole:
        rows = np.arange(n_rows, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, heads, dim), dtype=np.float32)
    if rows.size == 0:
        return out
    order = np.argsort(rows // ROW_BLOCK, kind="stable")
    blk_of = rows[order] // ROW_BLOCK
    starts = np.searchsorted(blk_of, np.unique(blk_of))
    ends = list(starts[1:]) + [rows.size]

    def one(i):
        b = int(blk_of[starts[i]])
        lo = b * ROW_BLOCK
        nb = min(ROW_BLOCK, n_rows - lo)
        blk = np.random.default_rng(key + [tid, b]).standard_normal((nb, heads, dim), dtype=np.float32)
        if scale != 1.0:
            blk *= np.float32(scale)
        if bf16:
            blk = round_to_bf16(blk)
        if whole:
            out[lo:lo + nb] = blk
        else:
            sel = order[starts[i]:ends[i]]
            out[sel] = blk[rows[sel] - lo]

    n = len(starts)
    if n == 1 or rows.size * heads * dim < (1 << 22):
        for i in range(n):
            one(i)
    else:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1, n)) as ex:
            list(ex.map(one, range(n)))
    return out


@dataclass
class Workload:
    name: str
    seed_key: list
    T: int
    Hq: int
    Hkv: int
    D: int
    cu_padded: np.ndarray
    cu_actual: np.ndarray
    cp: int
    strategies: tuple
    ranks: tuple
    backward: bool
    qkv_scale: float = 0.5
    do_scale: float = 1.0
    bf16: bool = True
    capacity: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def num_docs(self) -> int:
        return int(self.cu_padded.size - 1)

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def q(self, rows=None):
        return normal_rows(self.seed_key, TID_Q, self.T, self.Hq, self.D, self.qkv_scale, rows, self.bf16)

    def k(self, rows=None):
        return normal_rows(self.seed_key, TID_K, self.T, self.Hkv, self.D, self.qkv_scale, rows, self.bf16)

    def v(self, rows=None):
        return normal_rows(self.seed_key, TID_V, self.T, self.Hkv, self.D, self.qkv_scale, rows, self.bf16)

    def do(self, rows=None):
        return normal_rows(self.seed_key, TID_DO, self.T, self.Hq, self.D, self.do_scale, rows, self.bf16)


DCS, CONTIG, PACKED = 0, 1, 2   # strategy codes as passed to both sides (enum values of the C ABI)


def tiny_t28(bf16=False) -> Workload:
    cu_p = np.array([0, 8, 20, 28], dtype=np.int32)
    cu_a = np.array([0, 5, 17, 24], dtype=np.int32)
    return Workload("tiny_t28", [0], 28, 2, 2, 16, cu_p, cu_a, 2, (DCS, CONTIG), (0, 1), True,
                    qkv_scale=1.0, do_scale=1.0, bf16=bf16)


def t8192_mha16() -> Workload:
    rng = np.random.default_rng(2)
    p, a = docs_uniform_mult4(rng, 8192)
    return Workload("t8192_mha16", [2], 8192, 16, 16, 128, _cu(p), _cu(a), 2, (DCS, CONTIG), (0, 1), False)


def t32768_gqa32x8() -> Workload:
    rng = np.random.default_rng(3)
    p, a = docs_lognormal(rng, 32768, 64, 8192)
    return Workload("t32768_gqa32x8", [3], 32768, 32, 8, 128, _cu(p), _cu(a), 4, (DCS, CONTIG), (0, 3), True)


def t131072_gqa64x8() -> Workload:
    rng = np.random.default_rng(4)
    p, a = docs_uniform_any(rng, 131072)
    return Workload("t131072_gqa64x8", [4], 131072, 64, 8, 128, _cu(p), _cu(a), 8, (CONTIG,), (0, 7), True)


DYNAMIC_T_CAPACITY = 65536
DYNAMIC_T_MICROBATCHES = 16


def dynamic_t(m: int) -> Workload:
    rng = np.random.default_rng([5, m])
    T = 64 * int(rng.integers(64, 1025))
    p, a = docs_lognormal(rng, T, 32, 8192)
    return Workload(f"dynamic_t.mb{m}", [5, m], T, 32, 8, 128, _cu(p), _cu(a), 4, (DCS, CONTIG), (0, 1, 2, 3),
                    True, capacity=DYNAMIC_T_CAPACITY)


def t1m_10k_docs():
    """Partition-only layout: 1,048,576 tokens in 10,000 documents (multiples of 8)."""
    rng = np.random.default_rng(55)
    p, a = docs_composition(rng, 131072, 10000, 8)
    return _cu(p), _cu(a)


def small_random(seed, cp, strategy, max_docs=5, max_len=32, Hq=2, Hkv=1, D=16, pads=True,
                 bf16=False, qkv_scale=1.0, do_scale=1.0) -> Workload:
    """A tiny random layout valid for the given strategy (for brute-force checks)."""
    rng = np.random.default_rng([1000, seed])
    nd = int(rng.integers(1, max_docs + 1))
    padded, actual = [], []
    for _ in range(nd):
        if strategy == DCS:
            L = 2 * cp * int(rng.integers(0, max(1, max_len // (2 * cp)) + 1))
        else:
            L = int(rng.integers(0, max_len + 1))
        a = int(rng.integers(0, L + 1)) if pads else L
        padded.append(L)
        actual.append(a)
    T = sum(padded)
    unit = {CONTIG: cp, PACKED: 2 * cp}.get(strategy, 1)
    if T % unit:
        extra = unit - T % unit
        padded[-1] += extra
        if not pads:
            actual[-1] += extra
        T += extra
    if T == 0:
        padded[-1] = 2 * cp
        actual[-1] = 2 * cp if not pads else int(rng.integers(0, 2 * cp + 1))
        T = 2 * cp
    return Workload(f"small{seed}", [1000, seed], T, Hq, Hkv, D, _cu(padded), _cu(actual), cp,
                    (strategy,), tuple(range(cp)), True, qkv_scale=qkv_scale, do_scale=do_scale, bf16=bf16)
