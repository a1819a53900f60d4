"""Brute-force masked dense attention, float64 (test infrastructure; only
tests, the smoke check and the benchmark's CPU-baseline leg may import it).

It pins the query-outer oracle and is written independently of it: no union
gather, no per-block walk. For sequence ``b`` and KV head ``h`` it lays out
every logical position ``t in [0, msb*bs)`` as one dense key matrix, scores
every query of the sequence against all of them, and masks with

    alive(q, t) = (t // bs is a selected id of row (q, h))
                  and t < lk_b and block_tables[b, t // ps] >= 0
                  and (not causal or t <= limit(q)),

where ``lk_b`` and ``limit`` are as in ``process_work_unit`` (alice-llm 2.0.0,
``forward.rs``). A row with no alive position gives ``O = 0``, ``lse = -inf``.
"""
from __future__ import annotations

import numpy as np


def dense_masked_ref(q, k_pages, v_pages, selected, block_tables, cu_seqlens_q,
                     used_kv_lens, hq, hkv, head_dim, block_size, page_size,
                     softmax_scale, causal):
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    batch = cu.shape[0] - 1
    tq = int(cu[-1])
    tbl = np.asarray(block_tables, dtype=np.int64).reshape(batch, -1)
    max_pages = tbl.shape[1]
    ppb = block_size // page_size
    msb = max_pages // ppb
    n_pos = msb * block_size
    qhead = hq // hkv
    topk = np.asarray(selected).size // (tq * hkv)
    sel = np.asarray(selected, dtype=np.int64).reshape(tq, hkv, topk)
    num_pages = np.asarray(k_pages).size // (hkv * page_size * head_dim)
    kp = np.asarray(k_pages, dtype=np.float32).reshape(num_pages, hkv, page_size, head_dim)
    vp = np.asarray(v_pages, dtype=np.float32).reshape(num_pages, hkv, page_size, head_dim)
    qv = np.asarray(q, dtype=np.float32).reshape(tq, hq, head_dim).astype(np.float64)
    scale = float(np.float32(softmax_scale))

    out = np.zeros((tq, hq, head_dim), dtype=np.float64)
    lse = np.full((tq, hq), -np.inf, dtype=np.float64)
    t = np.arange(n_pos)
    for b in range(batch):
        q0, q1 = int(cu[b]), int(cu[b + 1])
        if q1 == q0:
            continue
        if used_kv_lens is None:
            lk = n_pos
        else:
            lk = max(int(np.asarray(used_kv_lens).ravel()[b]), 0)
        page_of_t = tbl[b, t // page_size] if n_pos else np.zeros(0, dtype=np.int64)
        page_ok = page_of_t >= 0
        qo_len = q1 - q0
        q_local = np.arange(qo_len)
        limit = (lk - qo_len + q_local) if lk >= qo_len else q_local       # [qo_len]
        for h in range(hkv):
            kd = np.zeros((n_pos, head_dim))
            vd = np.zeros((n_pos, head_dim))
            src = page_of_t[page_ok]
            kd[page_ok] = kp[src, h, t[page_ok] % page_size]
            vd[page_ok] = vp[src, h, t[page_ok] % page_size]
            member = (sel[q0:q1, h, :, None] == (t // block_size)[None, None, :]).any(axis=1)
            alive = member & (t < lk)[None, :] & page_ok[None, :]
            if causal:
                alive &= t[None, :] <= limit[:, None]
            for qh in range(qhead):
                hh = h * qhead + qh
                scores = (qv[q0:q1, hh, :] @ kd.T) * scale                  # [qo_len, n_pos]
                scores = np.where(alive, scores, -np.inf)
                for i in range(qo_len):
                    if not alive[i].any():
                        continue
                    mx = scores[i].max()
                    w = np.exp(scores[i] - mx)
                    out[q0 + i, hh] = (w @ vd) / w.sum()
                    lse[q0 + i, hh] = mx + np.log(w.sum())
    return out, lse
