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
