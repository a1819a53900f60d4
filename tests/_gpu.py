"""Helpers for the GPU tests: upload a workload, run the library, compare."""
import numpy as np
import torch

import block_sparse_paged_csr_amd as sa
import oracle


def dev_inputs(w, device="cuda"):
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dt)
    return {
        "q": t(w.q, torch.float32),
        "k": t(w.k_pages, torch.float32),
        "v": t(w.v_pages, torch.float32),
        "sel": t(w.selected, torch.int32),
        "bt": t(w.block_tables, torch.int32),
        "cu": t(w.cu_seqlens_q, torch.int64),
        "used": None if w.used_kv_lens is None else t(w.used_kv_lens, torch.int32),
    }


def run_index(w, d, num_pages=None):
    idx = sa.sa_index_plan(w.tq, w.hkv, w.topk, w.batch, w.max_pages, w.block_size,
                           w.page_size, w.hq, w.head_dim,
                           w.num_pages if num_pages is None else num_pages)
    idx.allocate(d["sel"].device)
    sa.sa_build_index(d["sel"], d["bt"], d["cu"], d["used"], idx)
    return idx


def run_attention(w, d, with_lse=True, return_index=False):
    return sa.sa_attention(d["q"], d["k"], d["v"], d["sel"], d["bt"], d["cu"], d["used"],
                           w.block_size, w.softmax_scale, w.causal, with_lse=with_lse,
                           return_index=return_index)


def oracle_index(w, num_pages=None):
    return oracle.build_index_ref(w.selected, w.tq, w.hkv, w.topk, w.block_tables, w.batch,
                                  w.max_pages, w.cu_seqlens_q, w.used_kv_lens, w.block_size,
                                  w.page_size, w.num_pages if num_pages is None else num_pages)


def assert_index_equal(idx, ref):
    info = sa.sa_index_status(idx)
    arrs = sa.index_arrays(idx, info)
    assert info["total_edges"] == ref["edges"].shape[0]
    for key in ("sel_slots", "sel_offsets", "num_sel", "edge_head_base", "inv", "edges"):
        got = arrs[key].cpu().numpy()
        np.testing.assert_array_equal(got, ref[key], err_msg=key)
    return info, arrs


def check_units(arrs, info, ref, cap_edges, w=None):
    """Units tile [0, E) exactly, each inside one slot, in CSR order per kind;
    each record's (b, blk, lk, delta) matches its slot."""
    E = info["total_edges"]
    units = np.concatenate([arrs["units_wave"].cpu().numpy(), arrs["units_mfma"].cpu().numpy()])
    cover = np.zeros(E, dtype=np.int64)
    for h, j, e0, e1, b, blk, lk, delta in units:
        assert 0 <= e0 < e1 <= E and e1 - e0 <= cap_edges
        base = ref["edge_head_base"][h]
        lo = base + ref["sel_offsets"][h, j]
        hi = base + ref["sel_offsets"][h, j + 1]
        assert lo <= e0 and e1 <= hi
        assert ref["sel_slots"][h, j] == b * ref["msb"] + blk
        assert lk == ref["lk"][b]
        if w is not None:
            q0, qo_len = int(w.cu_seqlens_q[b]), int(w.cu_seqlens_q[b + 1] - w.cu_seqlens_q[b])
            assert delta == (lk - qo_len if lk >= qo_len else 0) - q0
        cover[e0:e1] += 1
    assert np.all(cover == 1)
    for key in ("units_wave", "units_mfma"):
        u = arrs[key].cpu().numpy()
        if len(u) > 1:
            assert np.all(u[1:, 2] >= u[:-1, 3])       # CSR order within a kind


def max_rel_err(got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    scale = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (scale if scale > 0 else 1.0)), float(scale)


# ------------------------------------------------------------------ oracle in parallel
_POOL_W = None


def _qo_chunk(queries):
    w = _POOL_W
    return oracle.attention_qo_ref(w.q, w.k_pages, w.v_pages, w.selected, w.block_tables,
                                   w.cu_seqlens_q, w.used_kv_lens, w.hq, w.hkv, w.head_dim,
                                   w.block_size, w.page_size, w.softmax_scale, w.causal,
                                   queries=queries)


def qo_sampled(w, queries, workers=8, chunk=8):
    """The query-outer oracle on ``queries``, split over forked worker
    processes that share the workload's arrays (the workers run NumPy only and
    never touch the GPU)."""
    import multiprocessing as mp
    global _POOL_W
    queries = np.asarray(queries, dtype=np.int64)
    parts = [queries[i:i + chunk] for i in range(0, len(queries), chunk)]
    _POOL_W = w
    try:
        if workers <= 1 or len(parts) <= 1:
            res = [_qo_chunk(p) for p in parts]
        else:
            with mp.get_context("fork").Pool(min(workers, len(parts))) as pool:
                res = pool.map(_qo_chunk, parts)
    finally:
        _POOL_W = None
    return (np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res]))


# ------------------------------------------------------------------ partials
TOL_M = 1e-5          # partial max, absolute (natural-log units; scores are O(1))
TOL_OL = 1e-5         # partial o and l, relative to the largest magnitude compared


def sample_edges(ref, arrs, info, n_random=256, seed=0):
    """Edges to compare at full size: the first, middle and last edge of the
    hottest slot and of the smallest slot of every head, both ends of the
    first and last units of each kind, and n_random uniform draws."""
    rng = np.random.default_rng(seed)
    E = int(info["total_edges"])
    picks = set()
    for h in range(ref["hkv"]):
        n = int(ref["num_sel"][h])
        if n == 0:
            continue
        base = int(ref["edge_head_base"][h])
        sizes = np.diff(ref["sel_offsets"][h, :n + 1])
        for j in (int(np.argmax(sizes)), int(np.argmin(sizes))):
            lo = base + int(ref["sel_offsets"][h, j])
            hi = base + int(ref["sel_offsets"][h, j + 1])
            picks.update({lo, (lo + hi) // 2, hi - 1})
    for key in ("units_wave", "units_mfma"):
        u = arrs[key].cpu().numpy()
        for rec in (u[:2].tolist() + u[-2:].tolist()):
            picks.update({int(rec[2]), int(rec[3]) - 1})
    if E > 0:
        picks.update(rng.integers(0, E, size=min(n_random, E)).tolist())
    return np.asarray(sorted(p for p in picks if 0 <= p < E), dtype=np.int64)


def check_partials(w, d, idx, ref, only_edges=None, kv=None):
    """sa_forward's (o, m, l) against oracle.forward_partials_ref, on every
    edge or on ``only_edges``. ``kv`` = (k, v) device pages to use instead of
    d["k"], d["v"] (16-bit pages go through sa_forward_kv16)."""
    k, v = (d["k"], d["v"]) if kv is None else kv
    fwd = sa.sa_forward if k.dtype == torch.float32 else sa.sa_forward_kv16
    o, m, l = fwd(idx, d["q"], k, v, d["bt"], d["cu"], d["used"], w.hq, w.hkv, w.head_dim,
                  w.block_size, w.page_size, w.softmax_scale, w.causal)
    qhead = w.hq // w.hkv
    ro, rm, rl = oracle.forward_partials_ref(w.q, w.k_pages, w.v_pages, w.selected, ref,
                                             w.block_tables, w.cu_seqlens_q, w.used_kv_lens,
                                             w.hq, w.hkv, w.head_dim, w.block_size, w.page_size,
                                             w.softmax_scale, w.causal, only_edges=only_edges)
    if only_edges is None:
        rows = torch.arange(rm.shape[0], device=o.device)
    else:
        e = torch.as_tensor(np.asarray(only_edges), device=o.device)
        rows = (e[:, None] * qhead + torch.arange(qhead, device=o.device)[None, :]).reshape(-1)
    go = o[rows].cpu().numpy().astype(np.float64)
    gm = m[rows].cpu().numpy().astype(np.float64)
    gl = l[rows].cpu().numpy().astype(np.float64)
    fin = np.isfinite(rm)
    assert np.array_equal(fin, np.isfinite(gm)), "alive pattern of the partials"
    assert np.all(gl[~fin] == 0) and np.all(go[~fin] == 0), "empty partials must be (0, -inf, 0)"
    errs = {"m": 0.0, "l": 0.0, "o": 0.0, "rows": int(rm.shape[0])}
    if fin.any():
        errs["m"] = float(np.abs(gm[fin] - rm[fin]).max())
        errs["l"] = max_rel_err(gl, rl)[0]
        errs["o"] = max_rel_err(go, ro)[0]
        assert errs["m"] <= TOL_M, f"partial m abs err {errs['m']:.3e}"
        assert errs["l"] <= TOL_OL, f"partial l rel err {errs['l']:.3e}"
        assert errs["o"] <= TOL_OL, f"partial o rel err {errs['o']:.3e}"
    return errs
