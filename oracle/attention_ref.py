"""Query-outer attention oracle (test infrastructure; only tests, the smoke
check and the benchmark's CPU-baseline leg may import it).

For each query ``q`` and KV head ``h`` it takes the *set* ``T`` of logical key
positions covered by the blocks that ``q`` selected under ``h`` and runs
plain softmax attention over ``T``, in float64, for each GQA lane.

What a position contributes follows ``process_work_unit`` on the alice-llm
2.0.0 ``forward.rs`` page:

* a kept block ``v`` covers ``[v*bs, min((v+1)*bs, lk_b))``, where ``lk_b`` is
  ``max(used[b], 0)`` or ``msb*bs`` without ``used`` (the KV-length resolution);
* a position whose page ``block_tables[b, t // ps]`` is negative is skipped;
  the others read ``k_pages[page, h, t % ps, :]`` and the same row of
  ``v_pages`` (the block gather);
* with ``causal``, a position is alive iff ``t <= lk_b - qo_len_b + q_local``,
  or ``t <= q_local`` when ``lk_b < qo_len_b`` (the causal limit);
* the score is ``dot(q, k) * softmax_scale``, the scale applied after the dot;
* GQA: KV head ``h`` serves query heads ``h*qhead .. h*qhead + qhead - 1``.

An empty ``T`` gives ``O = 0`` and ``lse = -inf``. Duplicate kept ids in one
``(q, h)`` row are outside this oracle's domain (the index would keep both
edges). With ``strict`` it raises ``ValueError``.

Argument checks run in this order: head counts -> block/page sizes and
head_dim -> the index build's length checks -> ``q`` length -> K/V page
stride -> the build's content checks (cu_seqlens content and total, selected
range, page ids). Checks that read only lengths come before checks that read
array contents.
"""
from __future__ import annotations

import numpy as np

from .errors import SparseAttentionError
from .index_ref import batch_of, resolve_kv_lens, validate_build_shapes, validate_cu_content


def check_forward_args(hq, hkv, head_dim, block_size, page_size):
    """The argument checks of ``kvouter_forward`` (forward.rs), in its order."""
    if hkv == 0 or hq == 0 or hq % hkv != 0:
        raise SparseAttentionError("HeadCountMismatch", None, hq, hkv)
    if head_dim == 0 or block_size <= 0 or page_size <= 0 or block_size % page_size != 0:
        raise SparseAttentionError("BlockPageMismatch", None, block_size, page_size)


def check_tensor_lengths(q, k_pages, v_pages, hq, hkv, head_dim, page_size, tq):
    """The ``q`` length and K/V page-stride checks of ``kvouter_forward``;
    returns ``num_pages``."""
    if np.asarray(q).size != tq * hq * head_dim:
        raise SparseAttentionError("ShapeMismatch", "q", tq * hq * head_dim, np.asarray(q).size)
    page_stride = hkv * page_size * head_dim
    kn, vn = np.asarray(k_pages).size, np.asarray(v_pages).size
    if kn % page_stride != 0 or vn != kn:
        raise SparseAttentionError("ShapeMismatch", "k_pages / v_pages page stride",
                                   page_stride, kn)
    return kn // page_stride


def causal_limit(lk, qo_len, q_local):
    """Right-aligned causal limit (inclusive) for one query."""
    return lk - qo_len + q_local if lk >= qo_len else q_local


def attention_qo_ref(q, k_pages, v_pages, selected, block_tables, cu_seqlens_q,
                     used_kv_lens, hq, hkv, head_dim, block_size, page_size,
                     softmax_scale, causal, topk=None, queries=None, strict=True):
    """Return ``(O, lse)`` in float64: ``O`` is ``[n, hq, d]`` and ``lse`` is
    ``[n, hq]`` for the packed queries in ``queries`` (all of them if None)."""
    check_forward_args(hq, hkv, head_dim, block_size, page_size)
    cu = np.asarray(cu_seqlens_q, dtype=np.int64).ravel()
    tbl_np = np.asarray(block_tables)
    batch = cu.shape[0] - 1 if tbl_np.ndim != 2 else tbl_np.shape[0]
    max_pages = tbl_np.shape[-1] if tbl_np.ndim == 2 else tbl_np.size // max(batch, 1)
    tq = int(cu[-1]) if cu.shape[0] >= 1 else 0
    sel_np = np.asarray(selected)
    if topk is None:
        topk = sel_np.shape[-1] if sel_np.ndim == 3 else sel_np.size // max(tq * hkv, 1)
    sel, tbl, cu = validate_build_shapes(selected, tq, hkv, topk, block_tables, batch,
                                         max_pages, cu_seqlens_q, used_kv_lens,
                                         block_size, page_size)
    num_pages = check_tensor_lengths(q, k_pages, v_pages, hq, hkv, head_dim, page_size, tq)
    validate_cu_content(cu, tq)

    ppb = block_size // page_size
    msb = max_pages // ppb
    bad = (sel < -1) | (sel >= msb)
    if bad.any():
        first = int(np.flatnonzero(bad)[0])
        raise SparseAttentionError("SelectedOutOfRange", None, msb, int(sel[first]))
    lk = resolve_kv_lens(used_kv_lens, batch, msb, block_size)
    sel3 = sel.reshape(tq, hkv, topk)
    tbl2 = tbl.reshape(batch, max_pages)
    qhead = hq // hkv
    qv = np.asarray(q, dtype=np.float32).reshape(tq, hq, head_dim)
    kp = np.asarray(k_pages, dtype=np.float32).reshape(num_pages, hkv, page_size, head_dim)
    vp = np.asarray(v_pages, dtype=np.float32).reshape(num_pages, hkv, page_size, head_dim)
    scale = float(np.float32(softmax_scale))

    # Page-id check over every page that a kept block touches (the forward's
    # "block_tables page id" error), first offender in block-table order.
    touched = np.zeros((batch, max_pages), dtype=bool)
    for qi in range(tq):
        b = int(batch_of(cu, qi))
        for v in sel3[qi].ravel().tolist():
            if v == -1 or v * block_size >= lk[b]:
                continue
            block_end = min((v + 1) * block_size, int(lk[b]))
            for pl in range(ppb):
                if v * block_size + pl * page_size < block_end:
                    touched[b, v * ppb + pl] = True
    over = touched & (tbl2 >= num_pages)
    if over.any():
        first = int(np.flatnonzero(over.ravel())[0])
        raise SparseAttentionError("ShapeMismatch", "block_tables page id", num_pages,
                                   int(tbl2.ravel()[first]))

    qlist = np.arange(tq) if queries is None else np.asarray(queries, dtype=np.int64)
    out = np.zeros((qlist.shape[0], hq, head_dim), dtype=np.float64)
    lse = np.full((qlist.shape[0], hq), -np.inf, dtype=np.float64)
    for n, qi in enumerate(qlist.tolist()):
        b = int(batch_of(cu, qi))
        lk_b = int(lk[b])
        qo_len = int(cu[b + 1] - cu[b])
        q_local = qi - int(cu[b])
        limit = causal_limit(lk_b, qo_len, q_local)
        for h in range(hkv):
            ids = [v for v in sel3[qi, h].tolist() if v != -1 and v * block_size < lk_b]
            if strict and len(set(ids)) != len(ids):
                raise ValueError(f"duplicate block id in selected[{qi}, {h}]")
            if not ids:
                continue
            spans = [np.arange(v * block_size, min((v + 1) * block_size, lk_b)) for v in ids]
            t = np.unique(np.concatenate(spans))               # the union T, ascending
            pages = tbl2[b, t // page_size]
            t, pages = t[pages >= 0], pages[pages >= 0]
            if causal:
                alive = t <= limit
                t, pages = t[alive], pages[alive]
            if t.shape[0] == 0:
                continue
            k = kp[pages, h, t % page_size, :].astype(np.float64)   # [|T|, d]
            v_rows = vp[pages, h, t % page_size, :].astype(np.float64)
            lanes = qv[qi, h * qhead:(h + 1) * qhead, :].astype(np.float64)  # [qhead, d]
            s = (lanes @ k.T) * scale                                       # [qhead, |T|]
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            l = p.sum(axis=1, keepdims=True)
            out[n, h * qhead:(h + 1) * qhead, :] = (p @ v_rows) / l
            lse[n, h * qhead:(h + 1) * qhead] = (m + np.log(l))[:, 0]
    return out, lse
