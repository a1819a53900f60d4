"""CSR inverted-index oracle (test infrastructure; only tests, the smoke check
and the benchmark's CPU-baseline leg may import it).

Follows the field docs of ``KvOuterIndex``, ``SparseSelection``,
``BlockTables`` and ``CuSeqlensQ`` on the alice-llm 2.0.0 ``types.rs`` page,
and the builder call ``build_kvouter_index(&sel, &tbl, &cu, Some(&used),
block_size, page_size)`` in the ``gpu.rs`` page's tests. The builder's body
is not on the pages, so each step below takes the plainest reading of the
index fields it must fill:

1. ``ppb = block_size / page_size`` (``pages_per_block``). ``msb = max_pages //
   ppb`` is the number of whole sparse blocks one block-table row can address.
   ``nbs = B * msb`` is the dense slot capacity per head.
2. ``lk_b = max(used[b], 0)``, or ``msb * block_size`` without ``used``
   (forward.rs, ``process_work_unit``, the KV-length resolution).
3. Every ``(q, h, r)`` with ``v = selected[q, h, r]``: ``v == -1`` is padding;
   ``v < -1`` or ``v >= msb`` is ``SelectedOutOfRange``; ``v * block_size >= lk_b``
   is dropped (the ``inv`` field doc: such ranks get ``-1``); anything else is an
   edge ``(q, r)`` of raw slot ``b * msb + v`` under head ``h``.
4. Per head: the nonempty raw slots in ascending order form the compact list
   ``sel_slots[h, :num_sel[h]]`` (the rest of the row is ``-1``).
   ``sel_offsets[h]`` holds the head-local CSR offsets and stays at ``E_h``
   after ``num_sel[h]`` (the field doc keeps the offsets flat there). Inside a slot, edges are in
   ascending ``(q, r)``.
5. ``edge_head_base`` is the exclusive prefix sum of ``E_h``.
   ``inv[h, q, r]`` is the head-local position of edge ``(q, r)``, or ``-1``.

Errors are raised in one fixed order (the pages fix the order only inside
``kvouter_forward``; for the builder it is this module's reading):
cu_seqlens too short -> block/page sizes -> ``selected`` length ->
``block_tables`` length -> block-table rows vs ``B = len(cu) - 1`` ->
``used_kv_lens`` length -> empty input ->
cu_seqlens content -> ``cu[B] != tq`` -> the first out-of-range id in memory
order -> the first referenced page id ``>= num_pages`` in block-table memory
order.
"""
from __future__ import annotations

import numpy as np

from .errors import SparseAttentionError


def batch_of(cu_seqlens_q, tq_idx):
    """Sequence id of packed query ``tq_idx``: the last ``b`` with
    ``cu[b] <= tq_idx`` (types.rs, ``CuSeqlensQ::batch_of``, right-open
    intervals; empty sequences are skipped)."""
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    idx = np.searchsorted(cu, np.asarray(tq_idx, dtype=np.int64), side="right")
    return np.maximum(idx - 1, 0)


def resolve_kv_lens(used_kv_lens, batch, msb, block_size):
    """``lk_b = max(used[b], 0)``; with no ``used`` it is ``msb * block_size``
    (forward.rs, ``process_work_unit``)."""
    if used_kv_lens is None:
        return np.full(batch, msb * block_size, dtype=np.int64)
    return np.maximum(np.asarray(used_kv_lens, dtype=np.int64), 0)


def validate_build_shapes(selected, tq, hkv, topk, block_tables, batch, max_pages,
                          cu_seqlens_q, used_kv_lens, block_size, page_size):
    """Checks that need only lengths and scalars, in the module doc's order.
    Returns flat int64 copies of ``selected``, ``block_tables``, ``cu``."""
    cu = np.asarray(cu_seqlens_q, dtype=np.int64).ravel()
    if cu.shape[0] < 2:
        raise SparseAttentionError("CuSeqlensInvalid")
    if block_size <= 0 or page_size <= 0 or block_size % page_size != 0:
        raise SparseAttentionError("BlockPageMismatch", None, block_size, page_size)
    sel = np.asarray(selected).astype(np.int64).ravel()
    if sel.shape[0] != tq * hkv * topk:
        raise SparseAttentionError("ShapeMismatch", "selected", tq * hkv * topk, sel.shape[0])
    tbl = np.asarray(block_tables).astype(np.int64).ravel()
    if tbl.shape[0] != batch * max_pages:
        raise SparseAttentionError("ShapeMismatch", "block_tables", batch * max_pages, tbl.shape[0])
    if cu.shape[0] - 1 != batch:
        raise SparseAttentionError("ShapeMismatch", "block_tables rows", cu.shape[0] - 1, batch)
    if used_kv_lens is not None and np.asarray(used_kv_lens).ravel().shape[0] != batch:
        raise SparseAttentionError("ShapeMismatch", "used_kv_lens", batch,
                                   np.asarray(used_kv_lens).ravel().shape[0])
    if tq == 0 or hkv == 0 or topk == 0:
        raise SparseAttentionError("EmptyInput")
    return sel, tbl, cu


def validate_cu_content(cu, tq):
    """``cu[0] == 0``, non-decreasing (types.rs ``CuSeqlensQ::new``), and
    ``cu[B] == tq``."""
    if cu[0] != 0 or np.any(cu[1:] < cu[:-1]):
        raise SparseAttentionError("CuSeqlensInvalid")
    if cu[-1] != tq:
        raise SparseAttentionError("ShapeMismatch", "cu_seqlens_q total", tq, int(cu[-1]))


def validate_build_inputs(selected, tq, hkv, topk, block_tables, batch, max_pages,
                          cu_seqlens_q, used_kv_lens, block_size, page_size):
    """All of the builder's checks except the id and page-id checks."""
    sel, tbl, cu = validate_build_shapes(selected, tq, hkv, topk, block_tables, batch,
                                         max_pages, cu_seqlens_q, used_kv_lens, block_size,
                                         page_size)
    validate_cu_content(cu, tq)
    return sel, tbl, cu


def build_index_ref(selected, tq, hkv, topk, block_tables, batch, max_pages,
                    cu_seqlens_q, used_kv_lens, block_size, page_size, num_pages=None):
    """Build the KV-outer CSR index. Returns a dict of numpy arrays:

    ``sel_slots`` int32 [hkv, nbs], ``sel_offsets`` int32 [hkv, nbs+1],
    ``num_sel`` int32 [hkv], ``edges`` int32 [E, 2] of ``(q, rank)``,
    ``edge_head_base`` int64 [hkv+1], ``inv`` int32 [hkv, tq, topk],
    plus the scalars ``msb``, ``nbs``, ``ppb`` and ``lk`` int64 [B].

    ``num_pages`` (optional) moves the forward's "block_tables page id" check
    (forward.rs, ``process_work_unit``) into the build: a page that a kept
    block's valid range touches must have an id below ``num_pages``.
    """
    sel, tbl, cu = validate_build_inputs(selected, tq, hkv, topk, block_tables, batch,
                                         max_pages, cu_seqlens_q, used_kv_lens,
                                         block_size, page_size)
    ppb = block_size // page_size
    msb = max_pages // ppb
    nbs = batch * msb
    lk = resolve_kv_lens(used_kv_lens, batch, msb, block_size)

    bad = (sel < -1) | (sel >= msb)
    if bad.any():
        first = int(np.flatnonzero(bad)[0])
        raise SparseAttentionError("SelectedOutOfRange", None, msb, int(sel[first]))

    sel3 = sel.reshape(tq, hkv, topk)
    b_of_q = batch_of(cu, np.arange(tq))                       # [tq]
    lk_q = lk[b_of_q][:, None, None]
    kept = (sel3 != -1) & (sel3 * block_size < lk_q)           # step 3
    raw = b_of_q[:, None, None] * msb + sel3                   # raw slot id

    if num_pages is not None:
        tbl2 = tbl.reshape(batch, max_pages)
        touched = np.zeros((batch, max_pages), dtype=bool)
        qs, hs, rs = np.nonzero(kept)
        for b, blk in set(zip(b_of_q[qs].tolist(), sel3[qs, hs, rs].tolist())):
            block_end = min((blk + 1) * block_size, int(lk[b]))
            for pl in range(ppb):
                if blk * block_size + pl * page_size < block_end:
                    touched[b, blk * ppb + pl] = True
        over = touched & (tbl2 >= num_pages)
        if over.any():
            first = int(np.flatnonzero(over.ravel())[0])
            raise SparseAttentionError("ShapeMismatch", "block_tables page id",
                                       int(num_pages), int(tbl[first]))

    sel_slots = np.full((hkv, nbs), -1, dtype=np.int32)
    sel_offsets = np.zeros((hkv, nbs + 1), dtype=np.int32)
    num_sel = np.zeros(hkv, dtype=np.int32)
    inv = np.full((hkv, tq, topk), -1, dtype=np.int32)
    edges_per_head = []
    for h in range(hkv):
        qs, rs = np.nonzero(kept[:, h, :])          # row-major: ascending (q, r)
        raws = raw[qs, h, rs]
        order = np.argsort(raws, kind="stable")     # stable: (q, r) order kept per slot
        qs, rs, raws = qs[order], rs[order], raws[order]
        slots, counts = np.unique(raws, return_counts=True)
        n = slots.shape[0]
        num_sel[h] = n
        sel_slots[h, :n] = slots
        sel_offsets[h, 1:n + 1] = np.cumsum(counts)
        sel_offsets[h, n + 1:] = qs.shape[0]        # plateau at E_h
        inv[h, qs, rs] = np.arange(qs.shape[0], dtype=np.int32)
        edges_per_head.append(np.stack([qs, rs], axis=1).astype(np.int32))

    counts = [e.shape[0] for e in edges_per_head]
    edge_head_base = np.zeros(hkv + 1, dtype=np.int64)
    edge_head_base[1:] = np.cumsum(counts)
    edges = (np.concatenate(edges_per_head, axis=0) if edges_per_head
             else np.zeros((0, 2), dtype=np.int32))
    return {
        "sel_slots": sel_slots,
        "sel_offsets": sel_offsets,
        "num_sel": num_sel,
        "edges": edges.reshape(-1, 2),
        "edge_head_base": edge_head_base,
        "inv": inv,
        "msb": msb,
        "nbs": nbs,
        "ppb": ppb,
        "lk": lk,
        "hkv": hkv,
        "tq": tq,
        "topk": topk,
        "batch": batch,
    }
