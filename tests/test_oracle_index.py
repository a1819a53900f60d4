"""Pins for the index oracle (CPU only).

The index builder is absent from the pages, so the oracle's loop is the spec.
It is pinned to things other than itself:

* hand-derived indexes for the pages' two GPU-test fixtures (gpu.rs) and for a
  hand-built case with padding, drops, page holes and an empty sequence
  (``tests/golden/*.json``, each with its derivation);
* the accessor values printed by the types.rs tests;
* brute force on tiny random inputs: a per-entry dictionary construction
  written from the ``KvOuterIndex`` field docs, with no sort and no scan;
* invariants that hold at any size.
"""
import json
import os

import numpy as np
import pytest

import workloads as W
from oracle import SparseAttentionError, batch_of, build_index_ref


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _build_from_inputs(inp, num_pages=None):
    tbl = np.asarray(inp["block_tables"], dtype=np.int32)
    return build_index_ref(
        np.asarray(inp["selected"], dtype=np.int32), inp["tq"], inp["hkv"], inp["topk"],
        tbl, tbl.shape[0], tbl.shape[1], np.asarray(inp["cu_seqlens_q"], dtype=np.int64),
        None if inp.get("used_kv_lens") is None else np.asarray(inp["used_kv_lens"], np.int32),
        inp["block_size"], inp["page_size"],
        inp.get("num_pages") if num_pages is None else num_pages)


@pytest.mark.parametrize("name", ["pages_small_fixture_index.json",
                                  "pages_gqa_fixture_index.json",
                                  "handmade_index.json"])
def test_golden_index(golden_dir, name):
    g = _load(golden_dir, name)
    idx = _build_from_inputs(g["inputs"])
    exp = g["expected"]
    assert idx["msb"] == exp["msb"] and idx["nbs"] == exp["nbs"]
    for key in ("sel_slots", "sel_offsets", "num_sel", "edges", "edge_head_base", "inv"):
        np.testing.assert_array_equal(idx[key], np.asarray(exp[key]), err_msg=key)


def test_golden_page_error(golden_dir):
    g = _load(golden_dir, "handmade_index.json")
    case = g["page_error_case"]
    with pytest.raises(SparseAttentionError) as ei:
        _build_from_inputs(g["inputs"], num_pages=case["num_pages"])
    e = ei.value
    assert (e.kind, e.what, e.expected, e.got) == (case["kind"], case["what"],
                                                   case["expected"], case["got"])


def test_pages_types_cases(golden_dir):
    g = _load(golden_dir, "pages_types_cases.json")
    s = g["selection"]
    sel = np.asarray(s["flat"]).reshape(s["tq"], s["hkv"], s["topk"])
    for (q, h, r), val in s["get"]:
        assert sel[q, h, r] == val
    c = g["cu_seqlens"]
    for q, b in c["batch_of"]:
        assert batch_of(c["prefix"], q) == b
    # cu_seqlens validation: too short, prefix[0] != 0, non-monotone
    for bad in g["cu_seqlens_invalid"]:
        ntq = bad[-1] if bad else 0
        with pytest.raises(SparseAttentionError) as ei:
            build_index_ref(np.zeros(max(ntq, 0), np.int32), max(ntq, 0), 1, 1,
                            np.zeros((max(len(bad) - 1, 0), 1), np.int32),
                            max(len(bad) - 1, 0), 1, np.asarray(bad, np.int64), None, 1, 1)
        assert ei.value.kind == "CuSeqlensInvalid"


def _brute_index(w, num_pages=None):
    """Per-entry dictionary construction from the KvOuterIndex field docs."""
    ppb = w.block_size // w.page_size
    msb = w.max_pages // ppb
    nbs = w.batch * msb
    cu = [int(x) for x in w.cu_seqlens_q]
    buckets = [dict() for _ in range(w.hkv)]
    inv = -np.ones((w.hkv, w.tq, w.topk), dtype=np.int64)
    for h in range(w.hkv):
        for q in range(w.tq):
            b = max(i for i in range(w.batch) if cu[i] <= q and cu[i + 1] > q)
            lk = msb * w.block_size if w.used_kv_lens is None else max(int(w.used_kv_lens[b]), 0)
            for r in range(w.topk):
                v = int(w.selected[q, h, r])
                if v == -1 or v * w.block_size >= lk:
                    continue
                buckets[h].setdefault(b * msb + v, []).append((q, r))
    out_slots, out_offs, out_num, out_edges, bases = [], [], [], [], [0]
    for h in range(w.hkv):
        slots = sorted(buckets[h])
        row = slots + [-1] * (nbs - len(slots))
        offs, pos = [0], 0
        for s in slots:
            for (q, r) in buckets[h][s]:       # appended in (q, r) order
                inv[h, q, r] = pos
                out_edges.append((q, r))
                pos += 1
            offs.append(pos)
        offs += [pos] * (nbs + 1 - len(offs))
        out_slots.append(row)
        out_offs.append(offs)
        out_num.append(len(slots))
        bases.append(bases[-1] + pos)
    return {
        "sel_slots": np.asarray(out_slots).reshape(w.hkv, nbs),
        "sel_offsets": np.asarray(out_offs).reshape(w.hkv, nbs + 1),
        "num_sel": np.asarray(out_num),
        "edges": np.asarray(out_edges).reshape(-1, 2),
        "edge_head_base": np.asarray(bases),
        "inv": inv,
    }


def _build(w, num_pages=None):
    return build_index_ref(w.selected, w.tq, w.hkv, w.topk, w.block_tables, w.batch,
                           w.max_pages, w.cu_seqlens_q, w.used_kv_lens, w.block_size,
                           w.page_size, num_pages)


@pytest.mark.parametrize("seed", range(40))
def test_index_matches_brute_force(seed):
    w = W.make_random(seed, batch=1 + seed % 3, hkv=1 + seed % 2, topk=1 + seed % 4)
    idx = _build(w)
    ref = _brute_index(w)
    for key in ref:
        np.testing.assert_array_equal(idx[key], ref[key], err_msg=key)


def check_invariants(idx, selected, tq, hkv, topk):
    """Invariants of a CSR index that hold at any size."""
    E = idx["edges"].shape[0]
    base = idx["edge_head_base"]
    assert base[0] == 0 and base[-1] == E and np.all(np.diff(base) >= 0)
    nbs = idx["nbs"]
    for h in range(hkv):
        n = int(idx["num_sel"][h])
        slots = idx["sel_slots"][h]
        assert np.all(np.diff(slots[:n]) > 0)                    # ascending, distinct
        assert np.all(slots[n:] == -1)
        offs = idx["sel_offsets"][h]
        Eh = int(base[h + 1] - base[h])
        assert offs[0] == 0 and np.all(np.diff(offs) >= 0)
        assert np.all(np.diff(offs[:n + 1]) > 0)                 # nonempty slots
        assert np.all(offs[n:] == Eh)                            # plateau
        edges_h = idx["edges"][base[h]:base[h + 1]]
        for j in range(n):
            seg = edges_h[offs[j]:offs[j + 1]]
            key = seg[:, 0].astype(np.int64) * topk + seg[:, 1]
            assert np.all(np.diff(key) > 0)                      # ascending (q, r)
            assert np.all(selected[seg[:, 0], h, seg[:, 1]] >= 0)
        inv_h = idx["inv"][h]
        pos = inv_h[edges_h[:, 0], edges_h[:, 1]]
        np.testing.assert_array_equal(pos, np.arange(Eh))        # inv o edges = id
        assert (inv_h >= 0).sum() == Eh                          # each kept entry once
    assert nbs == idx["batch"] * idx["msb"]


@pytest.mark.parametrize("seed", range(20))
def test_index_invariants_random(seed):
    w = W.make_random(100 + seed, batch=3, qo_max=6, kv_max=40, hkv=2, topk=5)
    idx = _build(w)
    check_invariants(idx, w.selected, w.tq, w.hkv, w.topk)


@pytest.mark.parametrize("name", ["tiny", "decode", "ragged"])
def test_index_invariants_configs(name):
    w = W.make_config(name, with_kv=False)
    idx = _build(w, w.num_pages)
    check_invariants(idx, w.selected, w.tq, w.hkv, w.topk)
    if name == "decode":
        # qo_len 1: every edge is alone in its slot; nothing is dropped
        assert idx["edges"].shape[0] == w.tq * w.hkv * w.topk
        assert np.all(np.diff(idx["sel_offsets"][:, :int(idx["num_sel"][0]) + 1], axis=1) == 1)
    if name == "ragged":
        # every non-padding id is causally visible, so none is dropped
        assert idx["edges"].shape[0] == int((w.selected >= 0).sum())


def test_selected_out_of_range_first_in_memory_order():
    w = W.make_random(7, batch=2, hkv=2, topk=3)
    ppb = w.block_size // w.page_size
    msb = w.max_pages // ppb
    sel = w.selected.copy()
    flat = sel.reshape(-1)
    flat[5] = msb + 3
    flat[2] = -4
    with pytest.raises(SparseAttentionError) as ei:
        build_index_ref(sel, w.tq, w.hkv, w.topk, w.block_tables, w.batch, w.max_pages,
                        w.cu_seqlens_q, w.used_kv_lens, w.block_size, w.page_size)
    assert ei.value.kind == "SelectedOutOfRange"
    assert ei.value.got == -4 and ei.value.expected == msb


def test_error_order():
    w = W.make_random(3, batch=2, hkv=1, topk=2)
    args = dict(selected=w.selected, tq=w.tq, hkv=w.hkv, topk=w.topk,
                block_tables=w.block_tables, batch=w.batch, max_pages=w.max_pages,
                cu_seqlens_q=w.cu_seqlens_q, used_kv_lens=w.used_kv_lens,
                block_size=w.block_size, page_size=w.page_size)

    def kind(**over):
        a = dict(args, **over)
        with pytest.raises(SparseAttentionError) as ei:
            build_index_ref(**a)
        return ei.value.kind, ei.value.what

    # block/page before selected length
    assert kind(block_size=3, page_size=2, selected=w.selected[:1]) == ("BlockPageMismatch", None)
    assert kind(block_size=0)[0] == "BlockPageMismatch"
    assert kind(selected=w.selected.reshape(-1)[:-1]) == ("ShapeMismatch", "selected")
    assert kind(block_tables=w.block_tables.reshape(-1)[:-1]) == ("ShapeMismatch", "block_tables")
    assert kind(used_kv_lens=np.zeros(w.batch + 1, np.int32)) == ("ShapeMismatch", "used_kv_lens")
    assert kind(topk=0, selected=np.zeros(0, np.int32)) == ("EmptyInput", None)
    bad_cu = w.cu_seqlens_q.copy()
    bad_cu[0] = 1
    assert kind(cu_seqlens_q=bad_cu)[0] == "CuSeqlensInvalid"
    bad_cu = w.cu_seqlens_q.copy()
    bad_cu[-1] += 1
    sel_big = np.zeros((int(bad_cu[-1]), 1, w.topk), np.int32)
    assert kind(cu_seqlens_q=bad_cu) == ("ShapeMismatch", "cu_seqlens_q total")
    del sel_big


def test_negative_used_drops_everything():
    w = W.make_random(11, batch=2, hkv=1, topk=3, with_used=True)
    used = np.full(w.batch, -5, dtype=np.int32)
    idx = build_index_ref(w.selected, w.tq, w.hkv, w.topk, w.block_tables, w.batch,
                          w.max_pages, w.cu_seqlens_q, used, w.block_size, w.page_size)
    assert idx["edges"].shape[0] == 0
    assert np.all(idx["inv"] == -1)
    assert np.all(idx["sel_slots"] == -1)


def test_duplicate_ids_form_a_multiset():
    # Reading of the pages: the index keeps every (q, r) as its own edge.
    sel = np.asarray([[[1, 1, -1]]], dtype=np.int32)
    tbl = np.arange(4, dtype=np.int32).reshape(1, 4)
    idx = build_index_ref(sel, 1, 1, 3, tbl, 1, 4, np.asarray([0, 1]), None, 2, 2)
    np.testing.assert_array_equal(idx["edges"], [[0, 0], [0, 1]])
    np.testing.assert_array_equal(idx["sel_offsets"][0, :2], [0, 2])


def test_batch_of_skips_empty_sequences():
    cu = [0, 2, 2, 2, 5]
    assert [int(batch_of(cu, q)) for q in range(5)] == [0, 0, 3, 3, 3]
