"""Pins for the KV-outer partials oracle on their own (CPU only).

The combine is unchanged when one partial ``(o, m, l)`` becomes
``(c*o, m - ln c, c*l)``, so pins through the combine alone cannot fix the
reference point ``m``. These pin each partial directly (forward.rs, the
``ForwardPartials`` field docs: ``m`` is the row maximum of the scores,
``l`` the sum of ``exp(s - m)`` and ``o`` the ``exp(s - m)``-weighted sum of
value rows, not normalised):

* hand-computed cases whose scores are exact by construction: three keys of
  a block cut short by ``used_kv_lens``, a page hole, one alive key (``m`` is
  its score, ``l = 1``, ``o`` its value row), no alive key (``(0, -inf, 0)``);
* random tiny cases: ``m`` equals the largest alive score from a dense scoring
  of every logical position under an explicit mask (no block gather);
  ``1 <= l <= number of alive keys``; ``o / l`` and ``m + log l`` equal the
  query-outer oracle run with that one block selected;
* mutations: ``m`` over causally dead keys too, or the reference point moved by
  a constant, fails these pins.
"""
import math

import numpy as np
import pytest

import workloads as W
from oracle import attention_qo_ref, build_index_ref, forward_partials_ref, kvouter_ref


def _index(w):
    return build_index_ref(w.selected, w.tq, w.hkv, w.topk, w.block_tables, w.batch,
                           w.max_pages, w.cu_seqlens_q, w.used_kv_lens, w.block_size,
                           w.page_size, w.num_pages)


def _partials(w, idx, only_edges=None):
    return forward_partials_ref(w.q, w.k_pages, w.v_pages, w.selected, idx, w.block_tables,
                                w.cu_seqlens_q, w.used_kv_lens, w.hq, w.hkv, w.head_dim,
                                w.block_size, w.page_size, w.softmax_scale, w.causal,
                                only_edges=only_edges)


def _one_block_case(scores, values, *, used, causal=False, qo=1, table=None, ps=4, bs=4):
    """One sequence, hq = hkv = 1, d = 2, scale 0.5: query (2, 0) and key t =
    (scores[t], 0), so the score of key t is exactly scores[t]."""
    n = len(scores)
    npg = max(1, -(-n // ps))
    kp = np.zeros((npg, 1, ps, 2), dtype=np.float32)
    vp = np.zeros((npg, 1, ps, 2), dtype=np.float32)
    for t, (s, vv) in enumerate(zip(scores, values)):
        kp[t // ps, 0, t % ps] = (s, 0.0)
        vp[t // ps, 0, t % ps] = vv
    tbl = np.arange(npg, dtype=np.int32)[None] if table is None else np.asarray([table], np.int32)
    q = np.tile(np.asarray([[[2.0, 0.0]]], dtype=np.float32), (qo, 1, 1))
    sel = np.zeros((qo, 1, 1), dtype=np.int32)
    return W.Workload("hand", q, kp, vp, sel, tbl, np.asarray([0, qo], np.int64),
                      None if used is None else np.asarray([used], np.int32), 1, 1, 2, bs, ps,
                      1, 0.5, causal)


def test_hand_three_keys_cut_by_used_length():
    # key 3 (score 3.0, the largest) lies past used = 3 and must not count
    w = _one_block_case([1.0, 0.5, -0.25, 3.0], [(1, 2), (3, -1), (0.5, 0.5), (9, 9)], used=3)
    o, m, l = _partials(w, _index(w))
    e1, e2 = math.exp(-0.5), math.exp(-1.25)
    assert m[0] == pytest.approx(1.0, abs=1e-15)
    assert l[0] == pytest.approx(1 + e1 + e2, abs=1e-14)
    np.testing.assert_allclose(o[0], [1 + 3 * e1 + 0.5 * e2, 2 - e1 + 0.5 * e2], atol=1e-14)


def test_hand_page_hole_skips_its_keys():
    # page size 2, block of 4 keys; the block's second page is -1: keys 2, 3 skipped
    w = _one_block_case([0.0, 2.0, 5.0, 7.0], [(1, 0), (0, 1), (4, 4), (8, 8)], used=None,
                        ps=2, bs=4, table=[0, -1])
    o, m, l = _partials(w, _index(w))
    e = math.exp(-2.0)
    assert m[0] == pytest.approx(2.0, abs=1e-15)
    assert l[0] == pytest.approx(1 + e, abs=1e-15)
    np.testing.assert_allclose(o[0], [e, 1.0], atol=1e-15)


def test_hand_single_alive_key():
    # causal, used = 4, qo_len = 4: query 0's limit is position 0, so key 0
    # alone is alive although keys 1-3 score higher
    w = _one_block_case([0.75, 4.0, 5.0, 6.0], [(2, -3), (1, 1), (1, 1), (1, 1)], used=4,
                        causal=True, qo=4)
    idx = _index(w)
    o, m, l = _partials(w, idx)
    e0 = int(np.flatnonzero(idx["edges"][:, 0] == 0)[0])
    assert m[e0] == 0.75 and l[e0] == 1.0
    np.testing.assert_array_equal(o[e0], [2.0, -3.0])


def test_hand_no_alive_key():
    # causal, used = 8 and qo_len = 8 (two blocks of 4): query 0's limit is
    # position 0, so block 1 (keys 4..7) has no alive key, yet the index keeps
    # the edge; query 7's limit is 7 and all four keys count
    w = _one_block_case([1.0] * 8, [(1, 1)] * 8, used=8, causal=True, qo=8)
    w.selected[:] = 1
    idx = _index(w)
    o, m, l = _partials(w, idx)
    e0 = int(np.flatnonzero(idx["edges"][:, 0] == 0)[0])
    assert m[e0] == -np.inf and l[e0] == 0.0 and np.all(o[e0] == 0.0)
    e7 = int(np.flatnonzero(idx["edges"][:, 0] == 7)[0])
    assert m[e7] == pytest.approx(1.0) and l[e7] == pytest.approx(4.0)


def _dense_alive_max(w, idx):
    """Per partial row: the largest score over the alive keys of the edge's
    block, from all logical positions of the sequence scored at once and an
    explicit mask (no block gather)."""
    cu = w.cu_seqlens_q
    ppb = w.block_size // w.page_size
    msb = w.max_pages // ppb
    n_pos = msb * w.block_size
    qhead = w.hq // w.hkv
    t = np.arange(n_pos)
    out = np.full(idx["edges"].shape[0] * qhead, -np.inf)
    n_alive = np.zeros(idx["edges"].shape[0], dtype=np.int64)
    base = idx["edge_head_base"]
    for e, (qi, r) in enumerate(idx["edges"]):
        h = int(np.searchsorted(base, e, side="right") - 1)
        b = int(np.searchsorted(cu, qi, side="right") - 1)   # empty sequences skipped
        lk = n_pos if w.used_kv_lens is None else max(int(w.used_kv_lens[b]), 0)
        page = w.block_tables[b, t // w.page_size].astype(np.int64)
        kd = np.zeros((n_pos, w.head_dim))
        kd[page >= 0] = w.k_pages[page[page >= 0], h, t[page >= 0] % w.page_size]
        v = int(w.selected[qi, h, r])
        mask = (t // w.block_size == v) & (t < lk) & (page >= 0)
        if w.causal:
            qo_len, ql = int(cu[b + 1] - cu[b]), int(qi - cu[b])
            mask &= t <= ((lk - qo_len + ql) if lk >= qo_len else ql)
        n_alive[e] = int(mask.sum())
        for qh in range(qhead):
            s = (kd @ w.q[qi, h * qhead + qh].astype(np.float64)) * float(np.float32(w.softmax_scale))
            if mask.any():
                out[e * qhead + qh] = s[mask].max()
    return out, n_alive


def _check_random(w):
    idx = _index(w)
    o, m, l = _partials(w, idx)
    qhead = w.hq // w.hkv
    m_ref, n_alive = _dense_alive_max(w, idx)
    fin = np.isfinite(m_ref)
    assert np.array_equal(fin, np.isfinite(m))
    err_m = float(np.abs(m[fin] - m_ref[fin]).max()) if fin.any() else 0.0
    nal = np.repeat(n_alive, qhead)
    assert np.all(l[~fin] == 0) and np.all(o[~fin] == 0)
    assert np.all(l[fin] >= 1 - 1e-12) and np.all(l[fin] <= nal[fin] + 1e-12)
    # o / l and m + log l: the query-outer oracle with that one block selected
    base = idx["edge_head_base"]
    for r in range(w.topk):
        one = np.where(idx["inv"].transpose(1, 0, 2)[:, :, r:r + 1] >= 0,
                       w.selected[:, :, r:r + 1], -1).astype(np.int32)
        ref_o, ref_lse = attention_qo_ref(w.q, w.k_pages, w.v_pages, one, w.block_tables,
                                          w.cu_seqlens_q, w.used_kv_lens, w.hq, w.hkv,
                                          w.head_dim, w.block_size, w.page_size,
                                          w.softmax_scale, w.causal)
        for h in range(w.hkv):
            for qi in range(w.tq):
                p = int(idx["inv"][h, qi, r])
                if p < 0:
                    continue
                for qh in range(qhead):
                    row = (int(base[h]) + p) * qhead + qh
                    hq = h * qhead + qh
                    if not np.isfinite(m[row]):
                        assert ref_lse[qi, hq] == -np.inf
                        continue
                    np.testing.assert_allclose(o[row] / l[row], ref_o[qi, hq], atol=1e-12)
                    assert abs(m[row] + math.log(l[row]) - ref_lse[qi, hq]) < 1e-12
    return err_m


@pytest.mark.parametrize("seed", range(16))
def test_random_partials_pinned(seed):
    w = W.make_random(6000 + seed, batch=1 + seed % 3, hkv=1 + seed % 2, qhead=1 + seed % 3,
                      topk=1 + seed % 4, causal=bool(seed % 2) or None)
    assert _check_random(w) < 1e-12


def test_only_edges_rows_match_full():
    w = W.make_random(6100, batch=3, hkv=2, qhead=3, topk=4, qo_max=6, kv_max=40)
    idx = _index(w)
    o, m, l = _partials(w, idx)
    qhead = w.hq // w.hkv
    pick = [idx["edges"].shape[0] - 1, 0, 3]
    o2, m2, l2 = _partials(w, idx, only_edges=pick)
    rows = np.concatenate([np.arange(e * qhead, (e + 1) * qhead) for e in pick])
    np.testing.assert_array_equal(o2, o[rows])
    np.testing.assert_array_equal(m2, m[rows])
    np.testing.assert_array_equal(l2, l[rows])


def _max_over_all(real):
    """The planted mistake: m taken over every key of the block that has a
    page, causally dead ones included (o and l rescaled to match)."""
    def mutated(lanes, k, v, alive, scale):
        o, m, l = real(lanes, k, v, alive, scale)
        if not alive.any():
            return o, m, l
        m2 = ((lanes @ k.T) * scale).max(axis=1)
        c = np.exp(m - m2)
        return o * c[:, None], m2, l * c
    return mutated


def test_mutation_max_over_dead_keys_is_caught(monkeypatch):
    # hand case: query 5 of 8 (causal, used 8) sees keys 4, 5 of block 1 and
    # not the higher-scoring keys 6, 7
    w = _one_block_case([0, 0, 0, 0, 1.0, 0.5, 3.0, 4.0], [(1, 1)] * 8, used=8, causal=True,
                        qo=8)
    w.selected[:] = 1
    idx = _index(w)
    e5 = int(np.flatnonzero(idx["edges"][:, 0] == 5)[0])
    real = kvouter_ref.partial_over_keys
    o, m, l = _partials(w, idx)
    assert m[e5] == 1.0 and l[e5] == pytest.approx(1 + math.exp(-0.5))
    monkeypatch.setattr(kvouter_ref, "partial_over_keys", _max_over_all(real))
    o, m, l = _partials(w, idx)
    assert m[e5] == 4.0 and l[e5] < 1.0                 # what the pins below reject
    # random causal cases: wherever the mistake changes a partial, the pins
    # (the dense-mask maximum, or 1 <= l) reject it
    changed = 0
    for seed in range(6200, 6210):
        wr = W.make_random(seed, batch=2, hkv=1, qhead=2, topk=3, qo_max=6, kv_max=30,
                           causal=True, hole_prob=0.0)
        ir = _index(wr)
        with monkeypatch.context() as mp:
            mp.setattr(kvouter_ref, "partial_over_keys", real)
            _, m_true, _ = _partials(wr, ir)
        _, m_bad, _ = _partials(wr, ir)
        fin = np.isfinite(m_true)
        if not np.any(np.abs(m_bad[fin] - m_true[fin]) > 1e-9):
            continue
        changed += 1
        try:
            err = _check_random(wr)
        except AssertionError:
            continue                                   # a pin rejected it
        assert err > 1e-6                              # else the m pin must
    assert changed >= 2


def test_mutation_shifted_reference_point_is_caught(monkeypatch):
    # (c*o, m - ln c, c*l) leaves the combine unchanged; the direct pins catch it
    w = W.make_random(6050, batch=2, hkv=2, qhead=2, topk=3)
    real = kvouter_ref.partial_over_keys

    def shifted(lanes, k, v, alive, scale):
        o, m, l = real(lanes, k, v, alive, scale)
        return o * 2.0, m - math.log(2.0), l * 2.0
    monkeypatch.setattr(kvouter_ref, "partial_over_keys", shifted)
    with pytest.raises(AssertionError):
        _check_random(w)
