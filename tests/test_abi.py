"""The C ABI without a GPU: exports, planning, and the host-side checks.

Host-side checks return before anything touches the device, so they can run
here with null device pointers: every malformed call must report the same
error kind and detail as the oracle, in the same order.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import block_sparse_paged_csr_amd as sa
import oracle
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    with open(os.path.join(ROOT, "include", "sa.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^(?:sa_status|const char\*)\s+(sa_\w+)\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 9
    lib = sa.lib()
    for name in names:
        assert hasattr(lib, name), name
    # and the binding wraps the compute entry points under the same names
    for name in ("sa_index_plan", "sa_build_index", "sa_index_status", "sa_forward",
                 "sa_forward_kv16", "sa_combine", "sa_attention", "sa_attention_workspace_bytes"):
        assert callable(getattr(sa, name))


def test_struct_layout_matches_header():
    # the ctypes mirror must follow the header's field order
    with open(os.path.join(ROOT, "include", "sa.h")) as f:
        text = f.read()
    body = text[text.index("typedef struct sa_index {"):text.index("} sa_index;")]
    body = re.sub(r"/\*.*?\*/", "", body.split("{", 1)[1], flags=re.S)
    fields = re.findall(r"\b([a-z_]+)(?=[,;])", body)
    assert fields == [f for f, _ in sa.SaIndex._fields_]


@pytest.mark.parametrize("name", W.CONFIG_NAMES)
def test_plan_matches_oracle_geometry(name):
    w = W.make_config(name, with_kv=False)
    idx = sa.sa_index_plan(w.tq, w.hkv, w.topk, w.batch, w.max_pages, w.block_size,
                           w.page_size, w.hq, w.head_dim, w.num_pages)
    ppb = w.block_size // w.page_size
    assert idx.pages_per_block == ppb
    assert idx.msb == w.max_pages // ppb
    assert idx.nbs == w.batch * idx.msb
    assert idx.max_edges == w.tq * w.hkv * w.topk
    offs = [idx.off_header, idx.off_sel_slots, idx.off_sel_offsets, idx.off_num_sel,
            idx.off_edge_head_base, idx.off_edges, idx.off_inv, idx.off_units_wave,
            idx.off_units_mfma, idx.off_scratch]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert idx.index_bytes >= idx.off_scratch


def test_plan_errors():
    with pytest.raises(sa.SaError) as e:
        sa.sa_index_plan(4, 2, 2, 1, 8, 6, 4, 4, 32, 8)
    assert e.value.kind == "BlockPageMismatch"
    with pytest.raises(sa.SaError) as e:
        sa.sa_index_plan(4, 2, 2, 1, 8, 4, 4, 3, 32, 8)
    assert e.value.kind == "HeadCountMismatch"
    with pytest.raises(sa.SaError) as e:
        sa.sa_index_plan(0, 2, 2, 1, 8, 4, 4, 4, 32, 8)
    assert e.value.kind == "EmptyInput"
    with pytest.raises(sa.SaError) as e:
        sa.sa_index_plan(4, 2, 2, 1, 8, 4, 4, 4, 30, 8)
    assert e.value.kind == "Unsupported"


def _abi_attention_error(q_len, k_len, v_len, sel_len, tbl_len, cu_len, used_len, tq, hq, hkv,
                         d, topk, batch, max_pages, bs, ps, noalloc=False):
    """Call sa_attention (or sa_attention_noalloc) with null device pointers;
    only host checks can run."""
    lib = sa.lib()
    dummy = ctypes.c_void_p(0x1000)                 # never dereferenced by host checks
    used_ptr = None if used_len is None else dummy
    c = sa.SaIndex()
    if noalloc:
        st = lib.sa_attention_noalloc(dummy, q_len, dummy, k_len, dummy, v_len, dummy, sel_len,
                                      dummy, tbl_len, dummy, cu_len, used_ptr, used_len or 0, tq,
                                      hq, hkv, d, topk, batch, max_pages, bs, ps, 0.5, 1, dummy,
                                      None, ctypes.byref(c), None)
    else:
        st = lib.sa_attention(dummy, q_len, dummy, k_len, dummy, v_len, dummy, sel_len, dummy,
                              tbl_len, dummy, cu_len, used_ptr, used_len or 0, tq, hq, hkv, d,
                              topk, batch, max_pages, bs, ps, 0.5, 1, None, 0, dummy, None,
                              ctypes.byref(c), None)
    assert st != 0
    det = sa.SaErrorDetail()
    lib.sa_last_error(ctypes.byref(det))
    return sa.STATUS_NAMES[st], det.what.decode() or None, det.expected, det.got


def _cases():
    w = W.make_random(41, batch=2, qo_max=3, hkv=2, qhead=2, head_dim=8, topk=2,
                      with_used=True)
    base = dict(q=w.q, k=w.k_pages, v=w.v_pages, sel=w.selected, tbl=w.block_tables,
                cu=w.cu_seqlens_q, used=w.used_kv_lens, hq=w.hq, hkv=w.hkv, d=w.head_dim,
                bs=w.block_size, ps=w.page_size)
    cases = {
        "head_count": dict(hq=3),
        "hkv_zero": dict(hkv=0),
        "head_dim_zero": dict(d=0),
        "block_page": dict(bs=w.page_size * 2 + 1),
        "cu_short": dict(cu=w.cu_seqlens_q[:1]),
        "selected_len": dict(sel=w.selected.reshape(-1)[:-1]),
        "tbl_len": dict(tbl=w.block_tables.reshape(-1)[:-1].reshape(1, -1)),
        "tbl_rows": dict(tbl=w.block_tables[:1]),
        "used_len": dict(used=np.zeros(w.batch + 1, np.int32)),
        "q_len": dict(q=w.q.reshape(-1)[:-1]),
        "v_len": dict(v=w.v_pages.reshape(-1)[:-1]),
        "k_stride": dict(k=w.k_pages.reshape(-1)[:-1], v=w.v_pages.reshape(-1)[:-1]),
        "sel_and_q": dict(sel=w.selected.reshape(-1)[:-1], q=w.q.reshape(-1)[:-1]),
        "tbl_and_used": dict(tbl=w.block_tables[:1], used=np.zeros(7, np.int32)),
    }
    return w, base, cases


@pytest.mark.parametrize("noalloc", [False, True])
@pytest.mark.parametrize("case", list(_cases()[2].keys()))
def test_host_error_order_matches_oracle(case, noalloc):
    w, base, cases = _cases()
    a = dict(base, **cases[case])
    tq = int(np.asarray(a["cu"])[-1]) if np.asarray(a["cu"]).size else 0
    tbl = np.asarray(a["tbl"])
    batch, max_pages = (tbl.shape if tbl.ndim == 2 else (1, tbl.size))
    topk = w.topk
    with pytest.raises(oracle.SparseAttentionError) as ei:
        oracle.attention_qo_ref(a["q"], a["k"], a["v"], a["sel"], tbl, a["cu"], a["used"],
                                a["hq"], a["hkv"], a["d"], a["bs"], a["ps"], 0.5, True, topk=topk)
    ref = ei.value
    got = _abi_attention_error(np.asarray(a["q"]).size, np.asarray(a["k"]).size,
                               np.asarray(a["v"]).size, np.asarray(a["sel"]).size, tbl.size,
                               np.asarray(a["cu"]).size,
                               None if a["used"] is None else np.asarray(a["used"]).size,
                               tq, a["hq"], a["hkv"], a["d"], topk, batch, max_pages, a["bs"],
                               a["ps"], noalloc=noalloc)
    assert got[0] == ref.kind, (got, ref)
    if ref.kind == "ShapeMismatch":
        assert got[1:] == (ref.what, ref.expected, ref.got)
    if ref.kind in ("HeadCountMismatch", "BlockPageMismatch"):
        assert got[2:] == (ref.expected, ref.got)


def test_noalloc_rejects_problems_beyond_its_scratch():
    # decode-sized problems fit; prefill-sized ones need more than the
    # library's 32 MiB array and fail on the host, before any device call
    for name, fits in (("decode", True), ("prefill", False)):
        w = W.make_config(name, with_kv=False)
        need = sa.sa_attention_workspace_bytes(w.tq, w.hkv, w.topk, w.batch, w.max_pages,
                                               w.block_size, w.page_size, w.hq, w.head_dim)
        assert (need <= sa.SA_NOALLOC_SCRATCH_BYTES) == fits
    w = W.make_config("prefill", with_kv=False)
    page = w.hkv * w.page_size * w.head_dim
    got = _abi_attention_error(w.tq * w.hq * w.head_dim, page * 4, page * 4, w.selected.size,
                               w.block_tables.size, w.batch + 1, w.batch, w.tq, w.hq, w.hkv,
                               w.head_dim, w.topk, w.batch, w.max_pages, w.block_size,
                               w.page_size, noalloc=True)
    assert got[:3] == ("Unsupported", "workspace exceeds the no-alloc scratch",
                       sa.SA_NOALLOC_SCRATCH_BYTES)
    assert got[3] == need
    with open(os.path.join(ROOT, "include", "sa.h")) as f:
        assert "#define SA_NOALLOC_SCRATCH_BYTES (32u << 20)" in f.read()


def test_missing_gpu_tensors_fail_loudly():
    import torch
    t = torch.zeros(4)
    with pytest.raises(ValueError):
        sa._ptr(t, torch.float32, "q")


def _kv16_call(idx, d, bs, ps, hq, hkv, fmt):
    lib = sa.lib()
    n = 4 * hkv * ps * d
    return lib.sa_forward_kv16(ctypes.byref(idx.c), ctypes.c_void_p(16), idx.c.tq * hq * d,
                               ctypes.c_void_p(16), n, ctypes.c_void_p(16), n, fmt,
                               ctypes.c_void_p(16), ctypes.c_void_p(16), None, hq, hkv, d, bs,
                               ps, 0.1, 1, ctypes.c_void_p(16), ctypes.c_void_p(16),
                               ctypes.c_void_p(16), None)


@pytest.mark.parametrize("fmt,d,bs,qhead,what", [
    (3, 128, 64, 4, "kv_format"),                  # no such format
    (0, 128, 64, 4, "kv_format"),                  # fp32 goes through sa_forward
    (-1, 32, 128, 8, "kv_format"),
])
def test_kv16_host_checks(fmt, d, bs, qhead, what):
    # host checks return before any device access: a placeholder buffer suffices
    hkv, ps = 2, 16
    idx = sa.sa_index_plan(4, hkv, 2, 1, 16, bs, ps, hkv * qhead, d, 4)
    idx.c.buffer = 4096
    st = _kv16_call(idx, d, bs, ps, hkv * qhead, hkv, fmt)
    det = sa.SaErrorDetail()
    sa.lib().sa_last_error(ctypes.byref(det))
    assert sa.STATUS_NAMES[st] == "Unsupported"
    assert det.what.decode().startswith(what)


def test_kv16_shape_checks_come_first():
    # a wrong q length is reported before the format / geometry checks
    hkv, ps, d, bs, qhead = 2, 16, 128, 64, 4
    idx = sa.sa_index_plan(4, hkv, 2, 1, 16, bs, ps, hkv * qhead, d, 4)
    idx.c.buffer = 4096
    lib = sa.lib()
    n = 4 * hkv * ps * d
    st = lib.sa_forward_kv16(ctypes.byref(idx.c), ctypes.c_void_p(16), 5, ctypes.c_void_p(16), n,
                             ctypes.c_void_p(16), n, 3, ctypes.c_void_p(16), ctypes.c_void_p(16),
                             None, hkv * qhead, hkv, d, bs, ps, 0.1, 1, ctypes.c_void_p(16),
                             ctypes.c_void_p(16), ctypes.c_void_p(16), None)
    assert sa.STATUS_NAMES[st] == "ShapeMismatch"


def _fused_kv16_call(idx, sel_len, q_len, d, bs, ps, hq, hkv, fmt):
    lib = sa.lib()
    n = 4 * hkv * ps * d
    return lib.sa_forward_combine_kv16(
        ctypes.byref(idx.c), ctypes.c_void_p(16), sel_len, ctypes.c_void_p(16), q_len,
        ctypes.c_void_p(16), n, ctypes.c_void_p(16), n, fmt, ctypes.c_void_p(16),
        ctypes.c_void_p(16), None, hq, hkv, d, bs, ps, 0.1, 1, ctypes.c_void_p(16),
        ctypes.c_void_p(16), None)


@pytest.mark.parametrize("case", ["q", "kv_format"])
def test_fused_kv16_host_checks_in_order(case):
    # sa_forward's shape checks, then the format, before any device access
    # (the selections and the fused geometry come after the device check:
    # tested on the GPU)
    hkv, ps, d, qhead, topk, tq, bs = 2, 16, 128, 4, 2, 4, 64
    hq = hkv * qhead
    idx = sa.sa_index_plan(tq, hkv, topk, 1, 16, bs, ps, hq, d, 4)
    idx.c.buffer = 4096
    q_len = 5 if case == "q" else tq * hq * d
    fmt = 3 if case == "kv_format" else sa.SA_KV_BF16
    st = _fused_kv16_call(idx, tq * hkv * topk, q_len, d, bs, ps, hq, hkv, fmt)
    det = sa.SaErrorDetail()
    sa.lib().sa_last_error(ctypes.byref(det))
    want = {"q": ("ShapeMismatch", "q"), "kv_format": ("Unsupported", "kv_format")}
    assert sa.STATUS_NAMES[st] == want[case][0]
    assert det.what.decode().startswith(want[case][1])
