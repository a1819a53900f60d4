"""Pins for the attention oracles (CPU only).

* query-outer oracle == brute-force masked dense attention (tiny, fp64, 1e-12);
* KV-outer partials + LSE combine == query-outer oracle (1e-12);
* selecting every block == full attention from
  ``torch.nn.functional.scaled_dot_product_attention`` (float64, explicit mask),
  the "sparse full matches dense reference" test that gpu.rs names;
* right-aligned causal with qo_len == lk and every block == plain lower-triangular
  causal attention (``is_causal=True``);
* closed forms: one alive key gives its value row; constant keys give the mean
  of the alive values; a single block equals ``scipy.special.softmax`` attention;
* padding ranks and rank order change nothing; dropped and hole positions
  contribute nothing; an empty row gives O = 0 and lse = -inf;
* mutation checks: a planted mistake in the oracle (a wrong causal bound, a
  dropped scale, transposed lanes, a wrong combine weight) fails a pin.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import workloads as W
import oracle
from oracle import attention_ref, kvouter_ref
from oracle import (attention_qo_ref, build_index_ref, combine_ref, dense_masked_ref,
                    forward_partials_ref)


def qo(w, **kw):
    return attention_qo_ref(w.q, w.k_pages, w.v_pages, w.selected, w.block_tables,
                            w.cu_seqlens_q, w.used_kv_lens, w.hq, w.hkv, w.head_dim,
                            w.block_size, w.page_size, w.softmax_scale, w.causal, **kw)


def dense(w):
    return dense_masked_ref(w.q, w.k_pages, w.v_pages, w.selected, w.block_tables,
                            w.cu_seqlens_q, w.used_kv_lens, w.hq, w.hkv, w.head_dim,
                            w.block_size, w.page_size, w.softmax_scale, w.causal)


def ko(w):
    idx = build_index_ref(w.selected, w.tq, w.hkv, w.topk, w.block_tables, w.batch,
                          w.max_pages, w.cu_seqlens_q, w.used_kv_lens, w.block_size,
                          w.page_size, w.num_pages)
    o, m, l = forward_partials_ref(w.q, w.k_pages, w.v_pages, w.selected, idx, w.block_tables,
                                   w.cu_seqlens_q, w.used_kv_lens, w.hq, w.hkv,
                                   w.head_dim, w.block_size, w.page_size,
                                   w.softmax_scale, w.causal)
    return combine_ref(idx, o, m, l, w.hq, w.head_dim)


def max_err(a, b):
    a, b = np.asarray(a), np.asarray(b)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        d = np.where(both_inf, 0.0, np.abs(a - b))
    return float(np.nan_to_num(d, nan=np.inf).max()) if d.size else 0.0


def sdpa_full(w):
    """Full attention over the used, non-hole positions (plus the causal mask)
    of each sequence, via torch SDPA in float64."""
    cu = w.cu_seqlens_q
    ppb = w.block_size // w.page_size
    msb = w.max_pages // ppb
    n_pos = msb * w.block_size
    qhead = w.hq // w.hkv
    out = np.zeros((w.tq, w.hq, w.head_dim))
    t = np.arange(n_pos)
    for b in range(w.batch):
        q0, q1 = int(cu[b]), int(cu[b + 1])
        if q1 == q0:
            continue
        lk = n_pos if w.used_kv_lens is None else max(int(w.used_kv_lens[b]), 0)
        page = w.block_tables[b, t // w.page_size].astype(np.int64)
        ok = (page >= 0) & (t < lk)
        qo_len = q1 - q0
        ql = np.arange(qo_len)
        limit = (lk - qo_len + ql) if lk >= qo_len else ql
        mask = np.broadcast_to(ok, (qo_len, n_pos)).copy()
        if w.causal:
            mask &= t[None, :] <= limit[:, None]
        for h in range(w.hkv):
            kk = np.zeros((n_pos, w.head_dim))
            vv = np.zeros((n_pos, w.head_dim))
            kk[page >= 0] = w.k_pages[page[page >= 0], h, t[page >= 0] % w.page_size]
            vv[page >= 0] = w.v_pages[page[page >= 0], h, t[page >= 0] % w.page_size]
            qq = w.q[q0:q1, h * qhead:(h + 1) * qhead, :].astype(np.float64)
            qt = torch.from_numpy(np.ascontiguousarray(qq.transpose(1, 0, 2)))
            kt = torch.from_numpy(kk)[None].expand(qhead, -1, -1).contiguous()
            vt = torch.from_numpy(vv)[None].expand(qhead, -1, -1).contiguous()
            mt = torch.from_numpy(mask)[None].expand(qhead, -1, -1)
            o = torch.nn.functional.scaled_dot_product_attention(
                qt, kt, vt, attn_mask=mt, scale=float(np.float32(w.softmax_scale)))
            out[q0:q1, h * qhead:(h + 1) * qhead, :] = o.numpy().transpose(1, 0, 2)
    return out


def all_blocks(w):
    """Same inputs, every (q, h) row selecting all msb blocks (in shuffled order)."""
    ppb = w.block_size // w.page_size
    msb = w.max_pages // ppb
    rng = np.random.default_rng(0)
    sel = np.stack([rng.permutation(msb) for _ in range(w.tq * w.hkv)]).astype(np.int32)
    w2 = W.Workload(**{**w.__dict__})
    w2.selected = sel.reshape(w.tq, w.hkv, msb)
    w2.topk = msb
    return w2


# ---------------------------------------------------------------- cross pins

@pytest.mark.parametrize("seed", range(30))
def test_qo_matches_brute_force(seed):
    w = W.make_random(seed, batch=1 + seed % 3, hkv=1 + seed % 2, qhead=1 + seed % 3,
                      topk=1 + seed % 4, allow_out_of_range=bool(seed % 2))
    o1, l1 = qo(w)
    o2, l2 = dense(w)
    assert max_err(o1, o2) < 1e-12
    assert max_err(l1, l2) < 1e-12


@pytest.mark.parametrize("seed", range(30))
def test_kvouter_plus_combine_matches_qo(seed):
    w = W.make_random(1000 + seed, batch=1 + seed % 3, hkv=1 + seed % 2,
                      qhead=1 + seed % 3, topk=1 + seed % 4)
    o1, l1 = qo(w)
    o2, l2 = ko(w)
    assert max_err(o1, o2) < 1e-12
    assert max_err(l1, l2) < 1e-12


@pytest.mark.parametrize("seed", range(12))
def test_all_blocks_equals_full_attention_sdpa(seed):
    w = all_blocks(W.make_random(2000 + seed, batch=2, hkv=2, qhead=2, hole_prob=0.0,
                                 causal=bool(seed % 2), with_used=bool(seed % 3)))
    ref = sdpa_full(w)
    o, _ = qo(w)
    # rows whose mask is empty are NaN in SDPA; the oracle gives 0 there
    ok = ~np.isnan(ref)
    assert ok.any()
    assert max_err(o[ok], ref[ok]) < 1e-12


@pytest.mark.parametrize("seed", range(6))
def test_all_blocks_with_holes_equals_sdpa(seed):
    w = all_blocks(W.make_random(2100 + seed, batch=2, hkv=1, qhead=2, hole_prob=0.3,
                                 causal=False, with_used=True))
    ref = sdpa_full(w)
    o, _ = qo(w)
    ok = ~np.isnan(ref)
    assert max_err(o[ok], ref[ok]) < 1e-12


@pytest.mark.parametrize("seed", range(6))
def test_causal_square_is_lower_triangular(seed):
    # qo_len == lk and every block selected: right-aligned causal is plain causal.
    rng = np.random.default_rng(seed)
    bs, ps, d, hq, hkv = 4, 2, 8, 4, 2
    L = int(rng.integers(5, 13))
    msb = -(-L // bs)
    tbl = rng.permutation(msb * bs // ps + 3)[:msb * bs // ps].astype(np.int32)[None]
    num_pages = int(tbl.max()) + 1
    qv = rng.standard_normal((L, hq, d)).astype(np.float32)
    kp = rng.standard_normal((num_pages, hkv, ps, d)).astype(np.float32)
    vp = rng.standard_normal((num_pages, hkv, ps, d)).astype(np.float32)
    sel = np.tile(np.arange(msb, dtype=np.int32), (L, hkv, 1))
    o, _ = attention_qo_ref(qv, kp, vp, sel, tbl, np.asarray([0, L]), np.asarray([L], np.int32),
                            hq, hkv, d, bs, ps, 1 / math.sqrt(d), True)
    t = np.arange(L)
    qhead = hq // hkv
    for h in range(hkv):
        kk = kp[tbl[0, t // ps], h, t % ps].astype(np.float64)
        vv = vp[tbl[0, t // ps], h, t % ps].astype(np.float64)
        qq = torch.from_numpy(qv[:, h * qhead:(h + 1) * qhead].astype(np.float64).transpose(1, 0, 2).copy())
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq, torch.from_numpy(kk)[None].expand(qhead, -1, -1).contiguous(),
            torch.from_numpy(vv)[None].expand(qhead, -1, -1).contiguous(),
            is_causal=True, scale=float(np.float32(1 / math.sqrt(d))))
        assert max_err(o[:, h * qhead:(h + 1) * qhead], ref.numpy().transpose(1, 0, 2)) < 1e-12


# ---------------------------------------------------------------- closed forms

def _one_seq(rng, *, L, bs, ps, d, hq, hkv, used, sel, causal=False, kconst=False):
    msb = -(-L // bs)
    npg = msb * bs // ps
    tbl = rng.permutation(npg).astype(np.int32)[None]
    kp = rng.standard_normal((npg, hkv, ps, d)).astype(np.float32)
    if kconst:
        kp[:] = rng.standard_normal(d).astype(np.float32)
    vp = rng.standard_normal((npg, hkv, ps, d)).astype(np.float32)
    tq = sel.shape[0]
    qv = rng.standard_normal((tq, hq, d)).astype(np.float32)
    return qv, kp, vp, tbl


def test_single_alive_key_returns_its_value():
    rng = np.random.default_rng(1)
    bs, ps, d, hq, hkv = 4, 2, 8, 2, 1
    sel = np.asarray([[[2, -1]]], dtype=np.int32)          # block 2 only
    used = np.asarray([9], np.int32)                         # block 2 = [8, 9): one key
    qv, kp, vp, tbl = _one_seq(rng, L=12, bs=bs, ps=ps, d=d, hq=hq, hkv=hkv, used=used, sel=sel)
    o, lse = attention_qo_ref(qv, kp, vp, sel, tbl, np.asarray([0, 1]), used, hq, hkv, d,
                              bs, ps, 0.5, False)
    page = tbl[0, 8 // ps]
    for lane in range(hq):
        np.testing.assert_allclose(o[0, lane], vp[page, 0, 8 % ps].astype(np.float64), rtol=0, atol=1e-15)
        s = float(qv[0, lane].astype(np.float64) @ kp[page, 0, 8 % ps].astype(np.float64)) * 0.5
        assert abs(lse[0, lane] - s) < 1e-12                 # log(exp(s)) = s


def test_constant_keys_average_values():
    rng = np.random.default_rng(2)
    bs, ps, d, hq, hkv = 4, 2, 8, 2, 1
    sel = np.asarray([[[0, 2]]], dtype=np.int32)
    used = np.asarray([11], np.int32)
    qv, kp, vp, tbl = _one_seq(rng, L=12, bs=bs, ps=ps, d=d, hq=hq, hkv=hkv, used=used,
                               sel=sel, kconst=True)
    o, _ = attention_qo_ref(qv, kp, vp, sel, tbl, np.asarray([0, 1]), used, hq, hkv, d,
                            bs, ps, 0.3, False)
    t = np.concatenate([np.arange(0, 4), np.arange(8, 11)])
    mean_v = vp[tbl[0, t // ps], 0, t % ps].astype(np.float64).mean(axis=0)
    for lane in range(hq):
        np.testing.assert_allclose(o[0, lane], mean_v, rtol=0, atol=1e-14)


def test_single_block_is_textbook_softmax_attention():
    rng = np.random.default_rng(3)
    bs, ps, d, hq, hkv = 8, 4, 16, 3, 1
    sel = np.asarray([[[1]]], dtype=np.int32)
    qv, kp, vp, tbl = _one_seq(rng, L=16, bs=bs, ps=ps, d=d, hq=hq, hkv=hkv, used=None, sel=sel)
    scale = 0.25
    o, _ = attention_qo_ref(qv, kp, vp, sel, tbl, np.asarray([0, 1]), None, hq, hkv, d,
                            bs, ps, scale, False)
    t = np.arange(8, 16)
    K = kp[tbl[0, t // ps], 0, t % ps].astype(np.float64)
    V = vp[tbl[0, t // ps], 0, t % ps].astype(np.float64)
    Q = qv[0].astype(np.float64)
    ref = scipy.special.softmax(Q @ K.T * scale, axis=-1) @ V
    assert max_err(o[0], ref) < 1e-13


def test_empty_row_gives_zero_and_neg_inf():
    rng = np.random.default_rng(4)
    bs, ps, d, hq, hkv = 4, 2, 8, 2, 1
    sel = np.asarray([[[-1, -1]], [[3, -1]]], dtype=np.int32)   # q1's block is dropped
    used = np.asarray([10], np.int32)
    qv, kp, vp, tbl = _one_seq(rng, L=16, bs=bs, ps=ps, d=d, hq=hq, hkv=hkv, used=used, sel=sel)
    o, lse = attention_qo_ref(qv, kp, vp, sel, tbl, np.asarray([0, 2]), used, hq, hkv, d,
                              bs, ps, 0.3, False)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    o2, lse2 = ko(W.Workload("x", qv, kp, vp, sel, tbl, np.asarray([0, 2]), used, hq, hkv,
                             d, bs, ps, 2, 0.3, False))
    assert np.all(o2 == 0) and np.all(np.isneginf(lse2))


# ---------------------------------------------------------------- invariances

@pytest.mark.parametrize("seed", range(10))
def test_padding_ranks_are_inert(seed):
    w = W.make_random(3000 + seed, batch=2, hkv=2, qhead=2, topk=3, pad_prob=0.0)
    o1, _ = qo(w)
    rng = np.random.default_rng(seed)
    extra = np.full((w.tq, w.hkv, 2), -1, dtype=np.int32)
    sel = np.concatenate([w.selected, extra], axis=2)
    sel = np.stack([np.stack([rng.permutation(sel[q, h]) for h in range(w.hkv)])
                    for q in range(w.tq)]).astype(np.int32)
    w2 = W.Workload(**{**w.__dict__})
    w2.selected, w2.topk = sel, w.topk + 2
    o2, _ = qo(w2)
    o3, _ = ko(w2)
    assert max_err(o1, o2) < 1e-12 and max_err(o1, o3) < 1e-12


@pytest.mark.parametrize("seed", range(10))
def test_dropped_ranks_are_inert(seed):
    # a rank whose block starts at or past lk_b contributes nothing
    w = W.make_random(4000 + seed, batch=2, hkv=1, qhead=2, topk=4, with_used=True)
    ppb = w.block_size // w.page_size
    msb = w.max_pages // ppb
    lk = np.maximum(w.used_kv_lens.astype(np.int64), 0)
    sel = w.selected.copy()
    from oracle import batch_of
    for q in range(w.tq):
        b = int(batch_of(w.cu_seqlens_q, q))
        for h in range(w.hkv):
            for r in range(w.topk):
                if sel[q, h, r] >= 0 and sel[q, h, r] * w.block_size >= lk[b]:
                    sel[q, h, r] = -1
    w2 = W.Workload(**{**w.__dict__})
    w2.selected = sel
    assert max_err(qo(w)[0], qo(w2)[0]) == 0.0
    assert msb > 0


def test_causal_without_used_right_aligns_to_msb_blocks():
    # Reading: with no used_kv_lens the code path right-aligns to lk = msb*bs.
    rng = np.random.default_rng(5)
    bs, ps, d, hq, hkv = 4, 2, 8, 2, 1
    sel = np.asarray([[[0, 1]], [[0, 1]]], dtype=np.int32)
    qv, kp, vp, tbl = _one_seq(rng, L=8, bs=bs, ps=ps, d=d, hq=hq, hkv=hkv, used=None, sel=sel)
    o, _ = attention_qo_ref(qv, kp, vp, sel, tbl, np.asarray([0, 2]), None, hq, hkv, d,
                            bs, ps, 0.4, True)
    # lk = 8, qo_len = 2: query 0 sees t <= 6, query 1 sees t <= 7
    used = np.asarray([8], np.int32)
    o_used, _ = attention_qo_ref(qv, kp, vp, sel, tbl, np.asarray([0, 2]), used, hq, hkv,
                                 d, bs, ps, 0.4, True)
    assert max_err(o, o_used) == 0.0
    t = np.arange(7)
    K = kp[tbl[0, t // ps], 0, t % ps].astype(np.float64)
    V = vp[tbl[0, t // ps], 0, t % ps].astype(np.float64)
    ref = scipy.special.softmax(qv[0].astype(np.float64) @ K.T * float(np.float32(0.4)), axis=-1) @ V
    assert max_err(o[0], ref) < 1e-13


def test_short_kv_left_aligns():
    # lk_b < qo_len_b: the limit is q_local itself.
    rng = np.random.default_rng(6)
    bs, ps, d, hq, hkv = 4, 2, 8, 1, 1
    sel = np.asarray([[[0]], [[0]], [[0]]], dtype=np.int32)
    used = np.asarray([2], np.int32)
    qv, kp, vp, tbl = _one_seq(rng, L=4, bs=bs, ps=ps, d=d, hq=hq, hkv=hkv, used=used, sel=sel)
    o, _ = attention_qo_ref(qv, kp, vp, sel, tbl, np.asarray([0, 3]), used, hq, hkv, d,
                            bs, ps, 0.4, True)
    v0 = vp[tbl[0, 0], 0, 0].astype(np.float64)
    np.testing.assert_allclose(o[0, 0], v0, atol=1e-15)        # query 0 sees t = 0 only
    K = kp[tbl[0, 0], 0, :2].astype(np.float64)
    V = vp[tbl[0, 0], 0, :2].astype(np.float64)
    for qi in (1, 2):                                            # sees t = 0, 1 (lk = 2)
        ref = scipy.special.softmax(qv[qi, 0].astype(np.float64) @ K.T * float(np.float32(0.4))) @ V
        assert max_err(o[qi, 0], ref) < 1e-13


def test_pages_fixtures_regenerated():
    """The two closed-form fixtures of the gpu.rs tests, through QO, KO and SDPA."""
    # gpu_forward_matches_cpu_forward_small
    tq, hq, hkv, d, ps, bs, mp, npg = 2, 1, 1, 4, 2, 2, 3, 3
    qv = (np.arange(tq * hq * d, dtype=np.float32) * np.float32(0.11)).reshape(tq, hq, d)
    kp = np.sin(np.arange(npg * hkv * ps * d, dtype=np.float32) * np.float32(0.07)).reshape(npg, hkv, ps, d)
    vp = np.cos(np.arange(npg * hkv * ps * d, dtype=np.float32) * np.float32(0.13)).reshape(npg, hkv, ps, d)
    sel = np.tile(np.arange(mp, dtype=np.int32), (tq, hkv, 1))
    w = W.Workload("pages_small", qv, kp, vp, sel, np.asarray([[0, 1, 2]], np.int32),
                   np.asarray([0, 2]), np.asarray([6], np.int32), hq, hkv, d, bs, ps, mp,
                   1 / math.sqrt(d), False)
    ref = sdpa_full(w)
    assert max_err(qo(w)[0], ref) < 1e-12 and max_err(ko(w)[0], ref) < 1e-12
    # gpu_forward_gqa_multi_batch
    tq, hq, hkv, d, ps, bs, mp, npg = 3, 4, 2, 8, 4, 4, 3, 3
    qv = np.sin(np.arange(tq * hq * d, dtype=np.float32) * np.float32(0.05)).reshape(tq, hq, d)
    kp = np.cos(np.arange(npg * hkv * ps * d, dtype=np.float32) * np.float32(0.03)).reshape(npg, hkv, ps, d)
    vp = np.sin(np.arange(npg * hkv * ps * d, dtype=np.float32) * np.float32(0.09)).reshape(npg, hkv, ps, d)
    sel = np.tile(np.arange(mp, dtype=np.int32), (tq, hkv, 1))
    w = W.Workload("pages_gqa", qv, kp, vp, sel, np.asarray([[0, 1, 2], [0, 1, 2]], np.int32),
                   np.asarray([0, 2, 3]), np.asarray([12, 12], np.int32), hq, hkv, d, bs, ps,
                   mp, 1 / math.sqrt(d), False)
    ref = sdpa_full(w)
    assert max_err(qo(w)[0], ref) < 1e-12 and max_err(ko(w)[0], ref) < 1e-12


def test_errors_in_forward_order():
    w = W.make_random(9, batch=2, hkv=2, qhead=2, topk=2)
    with pytest.raises(oracle.SparseAttentionError) as ei:
        attention_qo_ref(w.q, w.k_pages, w.v_pages, w.selected, w.block_tables,
                         w.cu_seqlens_q, w.used_kv_lens, 3, 2, w.head_dim, 3, 2, 1.0, False)
    assert ei.value.kind == "HeadCountMismatch"
    with pytest.raises(oracle.SparseAttentionError) as ei:
        attention_qo_ref(w.q, w.k_pages, w.v_pages, w.selected, w.block_tables,
                         w.cu_seqlens_q, w.used_kv_lens, w.hq, w.hkv, 0, w.block_size,
                         w.page_size, 1.0, False)
    assert ei.value.kind == "BlockPageMismatch"
    with pytest.raises(oracle.SparseAttentionError) as ei:
        attention_qo_ref(w.q[:-1], w.k_pages, w.v_pages, w.selected, w.block_tables,
                         w.cu_seqlens_q, w.used_kv_lens, w.hq, w.hkv, w.head_dim,
                         w.block_size, w.page_size, 1.0, False)
    assert (ei.value.kind, ei.value.what) == ("ShapeMismatch", "q")
    with pytest.raises(oracle.SparseAttentionError) as ei:
        attention_qo_ref(w.q, w.k_pages, w.v_pages[:-1], w.selected, w.block_tables,
                         w.cu_seqlens_q, w.used_kv_lens, w.hq, w.hkv, w.head_dim,
                         w.block_size, w.page_size, 1.0, False)
    assert (ei.value.kind, ei.value.what) == ("ShapeMismatch", "k_pages / v_pages page stride")


# ---------------------------------------------------------------- mutation checks

def _sdpa_pin_error(seed=2003):
    w = all_blocks(W.make_random(seed, batch=2, hkv=2, qhead=2, hole_prob=0.0,
                                 causal=True, with_used=True))
    ref = sdpa_full(w)
    ok = ~np.isnan(ref)
    return max_err(qo(w)[0][ok], ref[ok])


def test_mutation_causal_bound_is_caught(monkeypatch):
    assert _sdpa_pin_error() < 1e-12
    monkeypatch.setattr(attention_ref, "causal_limit",
                        lambda lk, qo_len, ql: (lk - qo_len + ql - 1) if lk >= qo_len else ql)
    assert _sdpa_pin_error() > 1e-6


def test_mutation_dropped_scale_is_caught(monkeypatch):
    real = attention_ref.attention_qo_ref

    def no_scale(*a, **k):
        a = list(a)
        a[12] = 1.0
        return real(*a, **k)
    monkeypatch.setattr(oracle, "attention_qo_ref", no_scale)
    w = all_blocks(W.make_random(2001, batch=2, hkv=2, qhead=2, hole_prob=0.0))
    ref = sdpa_full(w)
    ok = ~np.isnan(ref)
    o = no_scale(w.q, w.k_pages, w.v_pages, w.selected, w.block_tables, w.cu_seqlens_q,
                 w.used_kv_lens, w.hq, w.hkv, w.head_dim, w.block_size, w.page_size,
                 w.softmax_scale, w.causal)[0]
    assert max_err(o[ok], ref[ok]) > 1e-6


def test_mutation_combine_weight_is_caught(monkeypatch):
    w = W.make_random(1005, batch=2, hkv=2, qhead=2, topk=3)
    good = max_err(ko(w)[0], qo(w)[0])
    assert good < 1e-12
    real_exp = np.exp

    class FakeNp:
        def __getattr__(self, k):
            return getattr(np, k)

        @staticmethod
        def exp(x):                       # forget the exp(m - M) rescale
            return np.ones_like(real_exp(x))
    monkeypatch.setattr(kvouter_ref, "np", FakeNp())
    bad = max_err(ko(w)[0], qo(w)[0])
    assert bad > 1e-6


def test_mutation_transposed_lanes_is_caught():
    # Serving KV head h with interleaved lanes (hq = qh*hkv + h) instead of the
    # contiguous groups of the pages would change the output.
    w = W.make_random(1007, batch=2, hkv=2, qhead=2, topk=3)
    o, _ = qo(w)
    w2 = W.Workload(**{**w.__dict__})
    qhead = w.hq // w.hkv
    perm = np.asarray([qh * w.hkv + h for h in range(w.hkv) for qh in range(qhead)])
    w2.q = w.q[:, perm, :]
    o2, _ = qo(w2)
    assert max_err(o, o2[:, np.argsort(perm), :]) > 1e-6
