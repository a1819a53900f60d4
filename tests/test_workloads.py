"""The seeded generators: determinism and the structure each workload claims."""
import numpy as np
import pytest

import workloads as W


@pytest.mark.parametrize("name", ["tiny", "decode", "ragged"])
def test_same_seed_same_bytes(name):
    a = W.make_config(name, with_kv=(name != "ragged"))
    b = W.make_config(name, with_kv=(name != "ragged"))
    for f in ("q", "k_pages", "v_pages", "selected", "block_tables", "cu_seqlens_q"):
        assert np.asarray(getattr(a, f)).tobytes() == np.asarray(getattr(b, f)).tobytes()
    c = W.make_config(name, seed=99, with_kv=False)
    assert c.selected.tobytes() != a.selected.tobytes() or c.q.tobytes() != a.q.tobytes()


def test_skipping_kv_changes_nothing_else():
    a = W.make_config("tiny")
    b = W.make_config("tiny", with_kv=False)
    for f in ("q", "selected", "block_tables", "cu_seqlens_q"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    assert b.k_pages.shape == a.k_pages.shape


@pytest.mark.parametrize("name", W.CONFIG_NAMES)
def test_rows_distinct_and_in_range(name):
    w = W.make_config(name, with_kv=False)
    ppb = w.block_size // w.page_size
    msb = w.max_pages // ppb
    sel = w.selected.reshape(-1, w.topk)
    assert sel.min() >= -1 and sel.max() < msb
    srt = np.sort(sel, axis=1)
    dup = (srt[:, 1:] == srt[:, :-1]) & (srt[:, 1:] >= 0)
    assert not dup.any()
    # each block-table row is a slice of one permutation: no physical page twice
    used = w.block_tables[w.block_tables >= 0]
    assert np.unique(used).size == used.size and used.max() < w.num_pages


def test_config_structure():
    d = W.make_config("decode", with_kv=False)
    assert (d.selected == 127).any(axis=2).all()              # last block in every row
    assert d.tq == 32 and d.topk == 16 and d.causal
    p = W.make_config("prefill", with_kv=False)
    assert (p.selected == 0).any(axis=2).all()
    q_local = np.arange(p.tq) % 1024
    hi = (16384 - 1024 + q_local) // 128
    for k in range(8):
        assert (p.selected == (hi - k)[:, None, None]).any(axis=2).all()
    t = W.make_config("tiny", with_kv=False)
    assert 0.05 < (t.selected == -1).mean() < 0.5
    r = W.make_config("ragged", with_kv=False)
    assert 0.05 < (r.selected == -1).mean() < 0.2
    assert r.used_kv_lens.min() >= 1024 - 63
    s = W.make_config("skewed", with_kv=False)
    assert (s.selected >= 0).all() and not s.causal
    # Zipf: a few blocks per (b, h) are shared by almost every query
    for b in range(2):
        rows = s.selected[b * 256:(b + 1) * 256, 0, :]
        counts = np.bincount(rows.ravel(), minlength=1024)
        assert counts.max() >= 240 and np.median(counts) < 64


def test_random_geometry_has_edge_cases():
    seen_empty = seen_hole = seen_drop = False
    for seed in range(60):
        w = W.make_random(seed)
        qo = np.diff(w.cu_seqlens_q)
        seen_empty |= bool((qo == 0).any())
        seen_hole |= bool((w.block_tables[:, :1] == -1).any() or (w.block_tables == -1).any())
        if w.used_kv_lens is not None:
            lk = np.maximum(w.used_kv_lens, 0)
            b = np.searchsorted(w.cu_seqlens_q, np.arange(w.tq), side="right") - 1
            seen_drop |= bool((w.selected * w.block_size >= lk[b][:, None, None]).any())
    assert seen_empty and seen_hole and seen_drop
