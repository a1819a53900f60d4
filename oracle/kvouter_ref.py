"""KV-outer partials and their log-sum-exp combine, in float64 (test
infrastructure: only the tests, the package smoke check and the benchmark's
CPU-baseline leg may import it; the GPU library never does).

The partial of one edge comes from what it stands for (alice-llm 2.0.0,
forward.rs: the ``ForwardPartials`` field docs, and what ``process_work_unit``
lets one key of a block contribute). It is written out per edge, with no
walk over slots, units or pages:

* edge ``(q, r)`` under KV head ``h`` names block ``v = selected[q, h, r]`` of
  the sequence ``b`` that holds query ``q``;
* the block's keys ``T`` are the logical positions ``t`` with
  ``v*bs <= t < min((v+1)*bs, lk_b)`` whose page ``block_tables[b, t // ps]``
  is not negative (``k_t = k_pages[page, h, t % ps]``, ``v_t`` likewise);
* with ``causal`` a key is alive only if ``t <= limit(q)``, the right-aligned
  limit the query-outer oracle uses;
* for GQA lane ``qh`` (query head ``h*qhead + qh``) the scores over the alive
  keys are ``s_t = dot(q, k_t) * scale``; then ``m = max s_t``,
  ``l = sum exp(s_t - m)`` and ``o = sum exp(s_t - m) v_t`` (not normalised).
  No alive key gives ``(o, m, l) = (0, -inf, 0)``.

Hence ``o / l`` is softmax attention over that block alone and ``m + log l``
its log-sum-exp. Row ``e * qhead + qh`` holds edge ``e``, lane ``qh``
(``ForwardPartials``: edges in CSR order, GQA lanes inner).

``combine_ref`` is this package's reading of the combine pass, which the
forward.rs module doc names but does not show: the log-sum-exp merge that
FlashAttention uses to join the softmax of separate key blocks. For
``(q, h, qh)`` it takes every rank with ``inv[h, q, r] >= 0``, at partial row
``(edge_head_base[h] + inv) * qhead + qh``, and computes ``M = max m``,
``L = sum l * exp(m - M)`` and ``O = sum o * exp(m - M) / L``. With no finite
``m`` the result is ``O = 0`` and ``lse = -inf``; otherwise ``lse = M + log L``.
"""
from __future__ import annotations

import numpy as np

from .attention_ref import causal_limit
from .index_ref import batch_of, resolve_kv_lens


def block_keys(tbl_row, v, lk_b, block_size, page_size):
    """Positions of block ``v`` below ``lk_b`` that sit on a page, with their
    pages: ``(t [n], page [n])``."""
    lo = v * block_size
    hi = min(lo + block_size, lk_b)
    t = np.arange(lo, hi) if hi > lo else np.zeros(0, dtype=np.int64)
    pages = tbl_row[t // page_size] if t.size else np.zeros(0, dtype=np.int64)
    keep = pages >= 0
    return t[keep], pages[keep]


def partial_over_keys(lanes, k, v, alive, scale):
    """``(o [qhead, d], m [qhead], l [qhead])`` over the keys where ``alive``:
    ``m`` the largest score, ``l`` and ``o`` the sums of ``exp(s - m)`` and of
    ``exp(s - m) v``."""
    qhead, d = lanes.shape
    if not alive.any():
        return np.zeros((qhead, d)), np.full(qhead, -np.inf), np.zeros(qhead)
    s = (lanes @ k[alive].T) * scale                     # [qhead, n_alive]
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    return p @ v[alive], m, p.sum(axis=1)


def forward_partials_ref(q, k_pages, v_pages, selected, index, block_tables, cu_seqlens_q,
                         used_kv_lens, hq, hkv, head_dim, block_size, page_size,
                         softmax_scale, causal, only_edges=None):
    """Partials of the index's edges, in float64.

    Returns ``(o [E*qhead, d], m [E*qhead], l [E*qhead])`` with row
    ``e*qhead + qh``. With ``only_edges`` (a sequence of edge positions) the
    rows are those edges' only, in the order given: ``[len*qhead, ...]``."""
    qhead = hq // hkv
    cu = np.asarray(cu_seqlens_q, dtype=np.int64).ravel()
    batch = cu.shape[0] - 1
    tbl = np.asarray(block_tables, dtype=np.int64).reshape(batch, -1)
    msb = tbl.shape[1] // (block_size // page_size)
    tq = int(cu[-1])
    topk = np.asarray(selected).size // max(tq * hkv, 1)
    sel = np.asarray(selected, dtype=np.int64).reshape(tq, hkv, topk)
    num_pages = np.asarray(k_pages).size // (hkv * page_size * head_dim)
    qv = np.asarray(q, dtype=np.float32).reshape(tq, hq, head_dim)
    kp = np.asarray(k_pages, dtype=np.float32).reshape(num_pages, hkv, page_size, head_dim)
    vp = np.asarray(v_pages, dtype=np.float32).reshape(num_pages, hkv, page_size, head_dim)
    scale = float(np.float32(softmax_scale))
    lk = resolve_kv_lens(used_kv_lens, batch, msb, block_size)
    edges = np.asarray(index["edges"])
    base = np.asarray(index["edge_head_base"], dtype=np.int64)
    n_edges = edges.shape[0]
    wanted = np.arange(n_edges) if only_edges is None else np.asarray(only_edges, dtype=np.int64)

    o = np.zeros((wanted.shape[0] * qhead, head_dim), dtype=np.float64)
    m = np.full(wanted.shape[0] * qhead, -np.inf, dtype=np.float64)
    l = np.zeros(wanted.shape[0] * qhead, dtype=np.float64)
    for n, e in enumerate(wanted.tolist()):
        h = int(np.searchsorted(base, e, side="right") - 1)     # head whose range holds e
        qi, r = int(edges[e, 0]), int(edges[e, 1])
        v = int(sel[qi, h, r])
        b = int(batch_of(cu, qi))
        t, pages = block_keys(tbl[b], v, int(lk[b]), block_size, page_size)
        alive = np.ones(t.shape[0], dtype=bool)
        if causal:
            qo_len = int(cu[b + 1] - cu[b])
            alive = t <= causal_limit(int(lk[b]), qo_len, qi - int(cu[b]))
        k_rows = kp[pages, h, t % page_size, :].astype(np.float64)
        v_rows = vp[pages, h, t % page_size, :].astype(np.float64)
        lanes = qv[qi, h * qhead:(h + 1) * qhead, :].astype(np.float64)
        oe, me, le = partial_over_keys(lanes, k_rows, v_rows, alive, scale)
        rows = slice(n * qhead, (n + 1) * qhead)
        o[rows], m[rows], l[rows] = oe, me, le
    return o, m, l


def combine_ref(index, o_partial, m_partial, l_partial, hq, head_dim):
    """Log-sum-exp merge of the partials into ``(O [tq, hq, d], lse [tq, hq])``."""
    hkv = index["hkv"]
    tq = index["tq"]
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
