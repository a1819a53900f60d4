"""KV-outer partials and their log-sum-exp combine, in float64 (test
infrastructure; only tests, the smoke check and the benchmark's CPU-baseline
leg may import it).

``forward_partials_ref`` restates ``process_work_unit`` (alice-llm 2.0.0,
``forward.rs``) unit by unit, in its order, with one unit per compact slot:

1. decode the slot: ``raw = sel_slots[h, j]``, ``b = raw // msb``, ``blk = raw % msb``;
2. clamp the block to ``[blk*bs, min((blk+1)*bs, lk_b))``; an empty range
   leaves the slot's partials at their initial ``(o=0, m=-inf, l=0)``;
3. gather the block's rows page by page through ``block_tables[b, blk*ppb + pl]``,
   skipping negative pages; a page id ``>= num_pages`` is the
   ``ShapeMismatch("block_tables page id")`` error;
4. per edge ``(q, r)`` of the slot, and per GQA lane ``qh``: the score of each
   gathered row is ``dot(q, k) * scale`` if the row is causally alive, else
   ``-inf``; ``m`` is the max; all dead gives ``(0, -inf, 0)``; otherwise
   ``p = exp(s - m)``, ``l = sum p`` and ``o = sum p * v``.

Partial ``(e, qh)`` sits at row ``e * qhead + qh`` (``ForwardPartials::partial_index``).

``combine_ref`` is this module's reading of the combine pass, which the
pages name but do not show ("standard FlashAttention log-sum-exp update",
``forward.rs`` module doc). For ``(q, h, qh)`` it takes every rank with
``inv[h, q, r] >= 0``, at partial row ``(edge_head_base[h] + inv) * qhead + qh``,
and computes ``M = max m``, ``L = sum l * exp(m - M)`` and
``O = sum o * exp(m - M) / L``. With no finite ``m`` the result is ``O = 0``
and ``lse = -inf``; otherwise ``lse = M + log L``.
"""
from __future__ import annotations

import numpy as np

from .errors import SparseAttentionError
from .index_ref import batch_of


def forward_partials_ref(q, k_pages, v_pages, index, block_tables, cu_seqlens_q,
                         used_kv_lens, hq, hkv, head_dim, block_size, page_size,
                         softmax_scale, causal, only_edges=None):
    """Return ``(o [E*qhead, d], m [E*qhead], l [E*qhead])`` in float64.

    ``only_edges`` (a set of edge positions) restricts the work to those
    edges; the other rows keep their initial ``(0, -inf, 0)``."""
    qhead = hq // hkv
    ppb = block_size // page_size
    msb = index["msb"]
    cu = np.asarray(cu_seqlens_q, dtype=np.int64).ravel()
    batch = cu.shape[0] - 1
    tbl = np.asarray(block_tables, dtype=np.int64).reshape(batch, -1)
    tq = int(cu[-1])
    num_pages = np.asarray(k_pages).size // (hkv * page_size * head_dim)
    qv = np.asarray(q, dtype=np.float32).reshape(tq, hq, head_dim)
    kp = np.asarray(k_pages, dtype=np.float32).reshape(num_pages, hkv, page_size, head_dim)
    vp = np.asarray(v_pages, dtype=np.float32).reshape(num_pages, hkv, page_size, head_dim)
    scale = float(np.float32(softmax_scale))
    edges = index["edges"]
    n_edges = edges.shape[0]
    o = np.zeros((n_edges * qhead, head_dim), dtype=np.float64)
    m = np.full(n_edges * qhead, -np.inf, dtype=np.float64)
    l = np.zeros(n_edges * qhead, dtype=np.float64)

    for h in range(hkv):
        head_base = int(index["edge_head_base"][h])
        for j in range(int(index["num_sel"][h])):
            if only_edges is not None:
                lo = head_base + int(index["sel_offsets"][h, j])
                hi = head_base + int(index["sel_offsets"][h, j + 1])
                if not any(lo <= e < hi for e in only_edges):
                    continue
            raw = int(index["sel_slots"][h, j])
            b, blk = raw // msb, raw % msb
            lk = (msb * block_size if used_kv_lens is None
                  else max(int(np.asarray(used_kv_lens).ravel()[b]), 0))
            block_start = blk * block_size
            block_end = min((blk + 1) * block_size, lk)
            if block_end <= block_start:
                continue
            qo_len = int(cu[b + 1] - cu[b])
            k_rows, v_rows, positions = [], [], []
            for pl in range(ppb):
                page_seq_start = blk * block_size + pl * page_size
                lo = max(block_start, page_seq_start)
                hi = min(block_end, page_seq_start + page_size)
                if hi <= lo:
                    continue
                page = int(tbl[b, blk * ppb + pl])
                if page < 0:
                    continue
                if page >= num_pages:
                    raise SparseAttentionError("ShapeMismatch", "block_tables page id",
                                               num_pages, page)
                for pos in range(lo - page_seq_start, hi - page_seq_start):
                    k_rows.append(kp[page, h, pos])
                    v_rows.append(vp[page, h, pos])
                    positions.append(page_seq_start + pos)
            if not positions:
                continue
            kb = np.asarray(k_rows, dtype=np.float64)
            vb = np.asarray(v_rows, dtype=np.float64)
            pos_arr = np.asarray(positions)
            e0 = head_base + int(index["sel_offsets"][h, j])
            e1 = head_base + int(index["sel_offsets"][h, j + 1])
            for e in range(e0, e1):
                if only_edges is not None and e not in only_edges:
                    continue
                qi = int(edges[e, 0])
                alive = np.ones(pos_arr.shape[0], dtype=bool)
                if causal:
                    q_local = qi - int(cu[int(batch_of(cu, qi))])
                    limit = lk - qo_len + q_local if lk >= qo_len else q_local
                    alive = pos_arr <= limit
                for qh in range(qhead):
                    row = e * qhead + qh
                    qvec = qv[qi, h * qhead + qh].astype(np.float64)
                    s = np.where(alive, (kb @ qvec) * scale, -np.inf)
                    mx = s.max()
                    if not np.isfinite(mx):
                        continue                      # (o=0, m=-inf, l=0)
                    p = np.where(alive, np.exp(s - mx), 0.0)
                    m[row] = mx
                    l[row] = p.sum()
                    o[row] = p @ vb
    return o, m, l


def combine_ref(index, o_partial, m_partial, l_partial, hq, head_dim):
    """Log-sum-exp merge of the partials into ``(O [tq, hq, d], lse [tq, hq])``."""
    hkv = index["hkv"]
    tq = index["tq"]
    topk = index["topk"]
    qhead = hq // hkv
    inv = index["inv"]
    base = index["edge_head_base"]
    out = np.zeros((tq, hq, head_dim), dtype=np.float64)
    lse = np.full((tq, hq), -np.inf, dtype=np.float64)
    for qi in range(tq):
        for h in range(hkv):
            pos = [int(base[h]) + int(x) for x in inv[h, qi] if x >= 0]
            for qh in range(qhead):
                rows = [p * qhead + qh for p in pos]
                if not rows:
                    continue
                ms = np.asarray([m_partial[r] for r in rows], dtype=np.float64)
                big = ms.max()
                if not np.isfinite(big):
                    continue
                w = np.exp(ms - big)                  # exp(-inf) = 0 for empty partials
                ls = np.asarray([l_partial[r] for r in rows], dtype=np.float64)
                total = float((ls * w).sum())
                acc = np.zeros(head_dim, dtype=np.float64)
                for r, wr in zip(rows, w):
                    acc += np.asarray(o_partial[r], dtype=np.float64) * wr
                out[qi, h * qhead + qh] = acc / total
                lse[qi, h * qhead + qh] = big + np.log(total)
    return out, lse
