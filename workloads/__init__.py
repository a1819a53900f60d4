"""Seeded synthetic inputs for block-sparse paged attention.

This module draws inputs only. It holds none of the attention arithmetic and
none of the index construction: it is shared by the CPU oracle (``oracle/``)
and by the GPU library's tests and benchmark, which otherwise share no code.

Every array follows the layouts of the alice-llm ``sparse_attention`` pages:

* ``q``            float32 ``[Tq, Hq, d]`` packed queries (forward.rs,
                   ``kvouter_forward`` doc comment).
* ``k_pages``/``v_pages`` float32 ``[num_pages, Hkv, page_size, d]``
                   (forward.rs, ``kvouter_forward`` doc comment).
* ``selected``     int32 ``[Tq, Hkv, topk]`` row-major, ``-1`` = padding rank
                   (types.rs, ``SparseSelection``).
* ``block_tables`` int32 ``[B, max_pages]`` logical -> physical page, ``-1``
                   pads a row (types.rs, ``BlockTables``).
* ``cu_seqlens_q`` int64 ``[B+1]`` cumulative packed query lengths (types.rs,
                   ``CuSeqlensQ``).
* ``used_kv_lens`` int32 ``[B]`` or ``None`` (forward.rs, ``kvouter_forward``).

Generator: ``numpy.random.Generator(PCG64(seed))``. Draw order is fixed:
lengths -> used lengths -> page permutation -> selection -> q -> k -> v.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

CONFIG_NAMES = ("tiny", "decode", "prefill", "ragged", "skewed")
CONFIG_SEEDS = {name: i for i, name in enumerate(CONFIG_NAMES)}


@dataclasses.dataclass
class Workload:
    """One batch of synthetic inputs plus the scalars that describe it."""

    name: str
    q: np.ndarray
    k_pages: np.ndarray
    v_pages: np.ndarray
    selected: np.ndarray
    block_tables: np.ndarray
    cu_seqlens_q: np.ndarray
    used_kv_lens: Optional[np.ndarray]
    hq: int
    hkv: int
    head_dim: int
    block_size: int
    page_size: int
    topk: int
    softmax_scale: float
    causal: bool

    @property
    def tq(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def batch(self) -> int:
        return int(self.cu_seqlens_q.shape[0] - 1)

    @property
    def max_pages(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def num_pages(self) -> int:
        return int(self.k_pages.shape[0])

    def describe(self) -> dict:
        return {
            "workload": self.name,
            "B": self.batch,
            "Tq": self.tq,
            "Hq": self.hq,
            "Hkv": self.hkv,
            "head_dim": self.head_dim,
            "page_size": self.page_size,
            "block_size": self.block_size,
            "topk": self.topk,
            "max_pages": self.max_pages,
            "num_pages": self.num_pages,
            "causal": self.causal,
        }


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def _draw_qkv(rng, tq, hq, num_pages, hkv, ps, d, with_kv):
    """q, then k, then v (the last draws, so skipping K/V changes nothing else)."""
    qv = _normal(rng, (tq, hq, d))
    if not with_kv:
        # zero-stride placeholders: right shape, no memory, not real K/V
        empty = np.broadcast_to(np.float32(0.0), (num_pages, hkv, ps, d))
        return qv, empty, empty
    kp = _normal(rng, (num_pages, hkv, ps, d))
    vp = _normal(rng, (num_pages, hkv, ps, d))
    return qv, kp, vp


def _page_tables(rng, pages_per_seq, max_pages, num_pages):
    """Each row is a slice of one random permutation of the physical pages."""
    perm = rng.permutation(num_pages).astype(np.int32)
    tbl = np.full((len(pages_per_seq), max_pages), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(pages_per_seq):
        tbl[b, :n] = perm[pos:pos + n]
        pos += n
    return tbl


def _distinct_from(rng, lo, hi, k):
    """``k`` distinct integers drawn uniformly from ``[lo, hi)``."""
    return lo + rng.choice(hi - lo, size=k, replace=False)


def make_tiny(seed: int = 0, with_kv: bool = True) -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    B, qo, kv = 2, 4, 128
    hq, hkv, d = 4, 2, 32
    ps, bs, max_pages, num_pages, topk = 16, 32, 8, 16, 2
    msb = max_pages // (bs // ps)
    cu = np.arange(B + 1, dtype=np.int64) * qo
    tq = int(cu[-1])
    tbl = _page_tables(rng, [kv // ps] * B, max_pages, num_pages)
    sel = np.empty((tq, hkv, topk), dtype=np.int32)
    for q in range(tq):
        for h in range(hkv):
            ids = _distinct_from(rng, 0, msb, topk)
            pad = rng.random(topk) < 0.25
            sel[q, h] = np.where(pad, -1, ids)
    qv, kp, vp = _draw_qkv(rng, tq, hq, num_pages, hkv, ps, d, with_kv)
    return Workload("tiny", qv, kp, vp, sel, tbl, cu, None, hq, hkv, d, bs, ps,
                    topk, 1.0 / math.sqrt(d), False)


def make_decode(seed: int = 1, with_kv: bool = True) -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    B, qo, kv = 32, 1, 8192
    hq, hkv, d = 32, 8, 128
    ps, bs, topk = 16, 64, 16
    max_pages = kv // ps
    num_pages = B * max_pages
    msb = max_pages // (bs // ps)
    cu = np.arange(B + 1, dtype=np.int64) * qo
    tq = int(cu[-1])
    used = np.full(B, kv, dtype=np.int32)
    tbl = _page_tables(rng, [max_pages] * B, max_pages, num_pages)
    sel = np.empty((tq, hkv, topk), dtype=np.int32)
    for q in range(tq):
        for h in range(hkv):
            ids = np.concatenate([[msb - 1], _distinct_from(rng, 0, msb - 1, topk - 1)])
            sel[q, h] = rng.permutation(ids)
    qv, kp, vp = _draw_qkv(rng, tq, hq, num_pages, hkv, ps, d, with_kv)
    return Workload("decode", qv, kp, vp, sel, tbl, cu, used, hq, hkv, d, bs, ps,
                    topk, 1.0 / math.sqrt(d), True)


def make_prefill(seed: int = 2, with_kv: bool = True, head_dim: int = 128,
                 block_size: int = 128, name: str = "prefill") -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    B, qo, kv = 4, 1024, 16384
    hq, hkv, d = 64, 8, head_dim
    ps, bs, topk = min(64, block_size), block_size, 32
    max_pages = kv // ps
    num_pages = B * max_pages
    cu = np.arange(B + 1, dtype=np.int64) * qo
    tq = int(cu[-1])
    used = np.full(B, kv, dtype=np.int32)
    tbl = _page_tables(rng, [max_pages] * B, max_pages, num_pages)
    sel = np.empty((tq, hkv, topk), dtype=np.int32)
    for q in range(tq):
        q_local = q % qo
        recent_hi = (kv - qo + q_local) // bs          # block holding the query
        recent = np.arange(recent_hi - 7, recent_hi + 1)
        for h in range(hkv):
            rand = _distinct_from(rng, 1, recent_hi - 7, topk - 9)
            ids = np.concatenate([[0], recent, rand])
            sel[q, h] = rng.permutation(ids)
    qv, kp, vp = _draw_qkv(rng, tq, hq, num_pages, hkv, ps, d, with_kv)
    return Workload(name, qv, kp, vp, sel, tbl, cu, used, hq, hkv, d, bs, ps,
                    topk, 1.0 / math.sqrt(d), True)


def make_ragged(seed: int = 3, with_kv: bool = True) -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    B = 16
    hq, hkv, d = 16, 2, 128
    ps, bs, topk = 16, 64, 64
    kv = rng.integers(1024, 131072, size=B, endpoint=True)
    qo = rng.integers(1, 64, size=B, endpoint=True)
    used = (kv - rng.integers(0, 63, size=B, endpoint=True)).astype(np.int32)
    pages = [int(math.ceil(k / ps)) for k in kv]
    max_pages = (bs // ps) * int(math.ceil(int(kv.max()) / bs))
    num_pages = int(sum(pages))
    tbl = _page_tables(rng, pages, max_pages, num_pages)
    cu = np.concatenate([[0], np.cumsum(qo)]).astype(np.int64)
    tq = int(cu[-1])
    sel = np.empty((tq, hkv, topk), dtype=np.int32)
    for b in range(B):
        for q_local in range(int(qo[b])):
            q = int(cu[b]) + q_local
            # blocks at or before the query's right-aligned causal position
            n_visible = (int(used[b]) - int(qo[b]) + q_local) // bs + 1
            for h in range(hkv):
                pad = rng.random(topk) < 0.1
                n_real = min(int((~pad).sum()), n_visible)
                ids = _distinct_from(rng, 0, n_visible, n_real)
                row = np.full(topk, -1, dtype=np.int64)
                slots = np.flatnonzero(~pad)[:n_real]
                row[slots] = ids
                sel[q, h] = row
    qv, kp, vp = _draw_qkv(rng, tq, hq, num_pages, hkv, ps, d, with_kv)
    return Workload("ragged", qv, kp, vp, sel, tbl, cu, used, hq, hkv, d, bs, ps,
                    topk, 1.0 / math.sqrt(d), True)


def make_skewed(seed: int = 4, with_kv: bool = True) -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    B, qo, kv = 8, 256, 131072
    hq, hkv, d = 64, 4, 128
    ps, bs, topk = 32, 128, 128
    zipf_s = 1.1
    max_pages = kv // ps
    num_pages = B * max_pages
    msb = max_pages // (bs // ps)
    cu = np.arange(B + 1, dtype=np.int64) * qo
    tq = int(cu[-1])
    used = np.full(B, kv, dtype=np.int32)
    tbl = _page_tables(rng, [max_pages] * B, max_pages, num_pages)
    sel = np.empty((tq, hkv, topk), dtype=np.int32)
    log_w_rank = -zipf_s * np.log(np.arange(1, msb + 1, dtype=np.float64))
    for b in range(B):
        for h in range(hkv):
            perm = rng.permutation(msb)
            log_w = np.empty(msb)
            log_w[perm] = log_w_rank          # block perm[k] has weight (k+1)^-s
            gumbel = rng.gumbel(size=(qo, msb))
            keys = log_w[None, :] + gumbel      # Gumbel-top-k = sampling w/o replacement
            top = np.argpartition(-keys, topk - 1, axis=1)[:, :topk]
            for i in range(qo):
                sel[int(cu[b]) + i, h] = rng.permutation(top[i])
    qv, kp, vp = _draw_qkv(rng, tq, hq, num_pages, hkv, ps, d, with_kv)
    return Workload("skewed", qv, kp, vp, sel, tbl, cu, used, hq, hkv, d, bs, ps,
                    topk, 1.0 / math.sqrt(d), False)


_MAKERS = {
    "tiny": make_tiny,
    "decode": make_decode,
    "prefill": make_prefill,
    "ragged": make_ragged,
    "skewed": make_skewed,
}

# The prefill recipe at other head dims and block sizes (the chunked MFMA
# kernel's geometries): not among the five workloads, for measurement only.
VARIANT_NAMES = ("prefill_d64", "prefill_d256", "prefill_bs256")
_MAKERS.update({
    "prefill_d64": lambda seed, with_kv: make_prefill(seed, with_kv, 64, 128, "prefill_d64"),
    "prefill_d256": lambda seed, with_kv: make_prefill(seed, with_kv, 256, 64, "prefill_d256"),
    "prefill_bs256": lambda seed, with_kv: make_prefill(seed, with_kv, 128, 256, "prefill_bs256"),
})
CONFIG_SEEDS.update({name: CONFIG_SEEDS["prefill"] for name in VARIANT_NAMES})


def make_config(name: str, seed: Optional[int] = None, with_kv: bool = True) -> Workload:
    """Build one of the five named workloads (seed defaults to its index).

    ``with_kv=False`` skips the K/V draws (the last ones) and leaves
    zero-stride placeholders of the right shape in their place."""
    if seed is None:
        seed = CONFIG_SEEDS[name]
    return _MAKERS[name](seed, with_kv)


def encode_kv16(x: np.ndarray, fmt: str) -> np.ndarray:
    """Store float32 K/V values as 16-bit words (uint16), rounding to nearest
    even: ``fmt`` "bf16" keeps the top half of the binary32 pattern, "fp16"
    is IEEE binary16. Input generation only: the oracle decodes the words
    itself."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if fmt == "fp16":
        return x.astype(np.float16).view(np.uint16)
    if fmt != "bf16":
        raise ValueError(f"unknown 16-bit format {fmt!r}")
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16          # finite inputs (N(0,1) draws)
    return rounded.astype(np.uint16)


def make_random(seed: int, *, batch=2, qo_max=4, kv_max=24, hkv=1, qhead=2,
                head_dim=8, page_size=2, pages_per_block=2, topk=3,
                pad_prob=0.25, hole_prob=0.1, causal=None, with_used=None,
                extra_pages=2, allow_out_of_range=True) -> Workload:
    """Small random geometry for property tests.

    Sequence lengths may be zero; block-table rows may hold ``-1`` holes and
    unused columns; ``selected`` rows hold distinct ids (plus ``-1``); ranks
    may point past the used length so that the index must drop them.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    bs = page_size * pages_per_block
    qo = rng.integers(0, qo_max, size=batch, endpoint=True)
    if qo.sum() == 0:
        qo[0] = 1
    kv = rng.integers(1, kv_max, size=batch, endpoint=True)
    if with_used is None:
        with_used = bool(rng.integers(0, 2))
    if causal is None:
        causal = bool(rng.integers(0, 2))
    used = None
    if with_used:
        used = (kv - rng.integers(0, bs, size=batch, endpoint=True)).astype(np.int32)
        used = np.maximum(used, -1).astype(np.int32)
    max_blocks = int(math.ceil(int(kv.max()) / bs)) + 1
    max_pages = max_blocks * pages_per_block + int(rng.integers(0, pages_per_block))
    msb = max_pages // pages_per_block
    pages = [min(int(math.ceil(k / page_size)), max_pages) for k in kv]
    num_pages = int(sum(pages)) + extra_pages
    tbl = _page_tables(rng, pages, max_pages, num_pages)
    holes = rng.random(tbl.shape) < hole_prob
    tbl = np.where(holes, -1, tbl).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(qo)]).astype(np.int64)
    tq = int(cu[-1])
    hi = msb if allow_out_of_range else max(1, min(msb, int(math.ceil(int(kv.min()) / bs))))
    sel = np.empty((tq, hkv, topk), dtype=np.int32)
    for q in range(tq):
        for h in range(hkv):
            k = min(topk, hi)
            ids = np.full(topk, -1, dtype=np.int64)
            ids[:k] = _distinct_from(rng, 0, hi, k)
            ids = rng.permutation(ids)
            pad = rng.random(topk) < pad_prob
            sel[q, h] = np.where(pad, -1, ids)
    hq = hkv * qhead
    qv = _normal(rng, (tq, hq, head_dim))
    kp = _normal(rng, (num_pages, hkv, page_size, head_dim))
    vp = _normal(rng, (num_pages, hkv, page_size, head_dim))
    return Workload("random", qv, kp, vp, sel, tbl, cu, used, hq, hkv, head_dim, bs,
                    page_size, topk, 1.0 / math.sqrt(head_dim), causal)
