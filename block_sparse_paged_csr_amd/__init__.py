"""Python binding of ``libsa.so``, the KV-outer block-sparse paged attention
library for MI355X (gfx950).

This is argument marshalling only. Every step of the computation runs in
the HIP kernels behind the C ABI of ``include/sa.h``. The functions carry
the ABI's names (``sa_index_plan``, ``sa_build_index``, ``sa_index_status``,
``sa_forward``, ``sa_combine``, ``sa_attention``). They take torch tensors
that already live on the GPU and enqueue on torch's current stream. PyTorch
provides device memory and streams, nothing more.

If the library is not built, or a tensor is not on a GPU, the call fails
loudly. There is no CPU path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char, c_float, c_int32, c_int64, c_size_t, c_void_p

import torch

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libsa.so")

# sa_status codes (include/sa.h) and the names of the error kinds they stand for
STATUS_NAMES = {
    0: "ok",
    1: "HeadCountMismatch",
    2: "BlockPageMismatch",
    3: "CuSeqlensInvalid",
    4: "ShapeMismatch",
    5: "SelectedOutOfRange",
    6: "HeadDimMismatch",
    7: "EmptyInput",
    8: "GpuInitFailed",
    9: "GpuRuntimeError",
    10: "Unsupported",
}
SA_OK = 0
SA_ERR_HEAD_DIM = 6


class SaIndex(Structure):
    """Mirror of ``struct sa_index`` (include/sa.h)."""

    _fields_ = [
        ("buffer", c_void_p), ("index_bytes", c_size_t), ("tq", c_int64),
        ("hkv", c_int32), ("topk", c_int32), ("batch", c_int32), ("max_pages", c_int32),
        ("block_size", c_int32), ("page_size", c_int32), ("hq", c_int32), ("head_dim", c_int32),
        ("num_pages", c_int64), ("pages_per_block", c_int32), ("msb", c_int32),
        ("nbs", c_int64), ("max_edges", c_int64), ("max_units", c_int64),
        ("cap_edges", c_int32), ("wave_cap_edges", c_int32), ("mfma_min_rows", c_int32),
        ("off_header", c_size_t), ("off_sel_slots", c_size_t), ("off_sel_offsets", c_size_t),
        ("off_num_sel", c_size_t), ("off_edge_head_base", c_size_t), ("off_edges", c_size_t),
        ("off_inv", c_size_t), ("off_units_wave", c_size_t), ("off_units_mfma", c_size_t),
        ("off_scratch", c_size_t),
    ]


class SaIndexInfo(Structure):
    _fields_ = [("status", c_int32), ("what", c_char * 64), ("expected", c_int64),
                ("got", c_int64), ("total_edges", c_int64), ("num_units_wave", c_int32),
                ("num_units_mfma", c_int32), ("num_slots", c_int64)]


class SaErrorDetail(Structure):
    _fields_ = [("status", c_int32), ("what", c_char * 64), ("expected", c_int64),
                ("got", c_int64)]


class SaError(RuntimeError):
    """A non-zero ``sa_status``: ``kind`` is the error name, with the detail."""

    def __init__(self, status, what="", expected=0, got=0):
        self.status = int(status)
        self.kind = STATUS_NAMES.get(self.status, f"status{status}")
        self.what = what or None
        self.expected = int(expected)
        self.got = int(got)
        super().__init__(f"{self.kind}(what={self.what!r}, expected={self.expected}, got={self.got})")


_LIB = None


def _declare(lib):
    vp, i32, i64, sz = c_void_p, c_int32, c_int64, c_size_t
    idxp = POINTER(SaIndex)
    sig = {
        "sa_index_plan": [i64, i32, i32, i32, i32, i32, i32, i32, i32, i64, idxp],
        "sa_build_index": [vp, i64, vp, i64, vp, i64, vp, i64, idxp, vp],
        "sa_index_status": [idxp, POINTER(SaIndexInfo), vp],
        "sa_forward": [idxp, vp, i64, vp, i64, vp, i64, vp, vp, vp, i32, i32, i32, i32, i32,
                       c_float, i32, vp, vp, vp, vp],
        "sa_forward_kv16": [idxp, vp, i64, vp, i64, vp, i64, i32, vp, vp, vp, i32, i32, i32, i32,
                            i32, c_float, i32, vp, vp, vp, vp],
        "sa_combine": [idxp, vp, vp, vp, i32, i32, vp, vp, vp],
        "sa_forward_combine": [idxp, vp, i64, vp, i64, vp, i64, vp, i64, vp, vp, vp, i32, i32, i32,
                               i32, i32, c_float, i32, vp, vp, vp],
        "sa_forward_combine_kv16": [idxp, vp, i64, vp, i64, vp, i64, vp, i64, i32, vp, vp, vp, i32,
                                    i32, i32, i32, i32, c_float, i32, vp, vp, vp],
        "sa_attention_workspace_bytes": [i64, i32, i32, i32, i32, i32, i32, i32, i32,
                                         POINTER(c_size_t)],
        "sa_attention": [vp, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp, i64,
                         i64, i32, i32, i32, i32, i32, i32, i32, i32, c_float, i32,
                         vp, sz, vp, vp, idxp, vp],
        "sa_attention_noalloc": [vp, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp, i64,
                                 i64, i32, i32, i32, i32, i32, i32, i32, i32, c_float, i32,
                                 vp, vp, idxp, vp],
        "sa_last_error": [POINTER(SaErrorDetail)],
        "sa_status_string": [c_int32],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name == "sa_status_string" else c_int32


def lib():
    """Open the built ``libsa.so`` (never compiles; raises if it is missing)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "`python -m block_sparse_paged_csr_amd._build` first")
        _LIB = ctypes.CDLL(LIB_PATH)
        _declare(_LIB)
    return _LIB


def _raise_last(status):
    d = SaErrorDetail()
    lib().sa_last_error(ctypes.byref(d))
    raise SaError(status, d.what.decode(), d.expected, d.got)


def _check(status):
    if status != SA_OK:
        _raise_last(status)


def _stream(device=None):
    return c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t, dtype, name):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU (the library has no CPU path)")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return c_void_p(t.data_ptr())


class Index:
    """An index plan (``sa_index``) plus the device buffer that holds it."""

    def __init__(self, c: SaIndex, buffer: torch.Tensor | None = None):
        self.c = c
        self.buffer = buffer

    def allocate(self, device="cuda"):
        # 256 extra bytes so the data pointer can be rounded up to 256
        raw = torch.empty(self.c.index_bytes + 256, dtype=torch.uint8, device=device)
        off = (-raw.data_ptr()) % 256
        self.buffer = raw[off:off + self.c.index_bytes]
        self.c.buffer = self.buffer.data_ptr()
        return self

    def __getattr__(self, k):
        return getattr(self.__dict__["c"], k)


def sa_index_plan(tq, hkv, topk, batch, max_pages, block_size, page_size, hq, head_dim,
                  num_pages) -> Index:
    c = SaIndex()
    _check(lib().sa_index_plan(tq, hkv, topk, batch, max_pages, block_size, page_size, hq,
                               head_dim, num_pages, ctypes.byref(c)))
    return Index(c)


def sa_build_index(selected, block_tables, cu_seqlens_q, used_kv_lens, index: Index):
    """Enqueue the index build; device-side errors surface in sa_index_status."""
    if index.buffer is None:
        index.allocate(selected.device if isinstance(selected, torch.Tensor) else "cuda")
    st = lib().sa_build_index(
        _ptr(selected, torch.int32, "selected"), selected.numel(),
        _ptr(block_tables, torch.int32, "block_tables"), block_tables.numel(),
        _ptr(cu_seqlens_q, torch.int64, "cu_seqlens_q"), cu_seqlens_q.numel(),
        _ptr(used_kv_lens, torch.int32, "used_kv_lens"),
        0 if used_kv_lens is None else used_kv_lens.numel(),
        ctypes.byref(index.c), _stream(selected.device))
    _check(st)
    return index


def sa_index_status(index: Index, check=True, device=None) -> dict:
    """Wait for the stream and read the build's device header."""
    info = SaIndexInfo()
    st = lib().sa_index_status(ctypes.byref(index.c), ctypes.byref(info), _stream(device))
    out = {
        "status": int(info.status), "what": info.what.decode(), "expected": int(info.expected),
        "got": int(info.got), "total_edges": int(info.total_edges),
        "num_units_wave": int(info.num_units_wave), "num_units_mfma": int(info.num_units_mfma),
        "num_slots": int(info.num_slots),
    }
    if check and st != SA_OK:
        if info.status != SA_OK:
            raise SaError(info.status, out["what"], out["expected"], out["got"])
        _raise_last(st)
    return out


def _check_head_dims(q, k_pages, v_pages):
    if not (q.shape[-1] == k_pages.shape[-1] == v_pages.shape[-1]):
        raise SaError(SA_ERR_HEAD_DIM)


def sa_forward(index: Index, q, k_pages, v_pages, block_tables, cu_seqlens_q, used_kv_lens,
               hq, hkv, head_dim, block_size, page_size, softmax_scale, causal,
               o_partial=None, m_partial=None, l_partial=None):
    """Enqueue the KV-outer forward; returns (o_partial, m_partial, l_partial),
    each sized for the worst case of tq*hkv*topk edges."""
    _check_head_dims(q, k_pages, v_pages)
    rows = index.c.max_edges * (hq // hkv if hkv > 0 else 1)
    dev = q.device
    if o_partial is None:
        o_partial = torch.empty((rows, head_dim), dtype=torch.float32, device=dev)
    if m_partial is None:
        m_partial = torch.empty(rows, dtype=torch.float32, device=dev)
    if l_partial is None:
        l_partial = torch.empty(rows, dtype=torch.float32, device=dev)
    st = lib().sa_forward(
        ctypes.byref(index.c), _ptr(q, torch.float32, "q"), q.numel(),
        _ptr(k_pages, torch.float32, "k_pages"), k_pages.numel(),
        _ptr(v_pages, torch.float32, "v_pages"), v_pages.numel(),
        _ptr(block_tables, torch.int32, "block_tables"),
        _ptr(cu_seqlens_q, torch.int64, "cu_seqlens_q"),
        _ptr(used_kv_lens, torch.int32, "used_kv_lens"),
        hq, hkv, head_dim, block_size, page_size, float(softmax_scale), int(bool(causal)),
        _ptr(o_partial, torch.float32, "o_partial"), _ptr(m_partial, torch.float32, "m_partial"),
        _ptr(l_partial, torch.float32, "l_partial"), _stream(dev))
    _check(st)
    return o_partial, m_partial, l_partial


SA_KV_F32, SA_KV_BF16, SA_KV_F16 = 0, 1, 2
_KV16_FORMATS = {torch.bfloat16: SA_KV_BF16, torch.float16: SA_KV_F16}


def sa_forward_kv16(index: Index, q, k_pages, v_pages, block_tables, cu_seqlens_q, used_kv_lens,
                    hq, hkv, head_dim, block_size, page_size, softmax_scale, causal,
                    o_partial=None, m_partial=None, l_partial=None):
    """sa_forward with K/V pages stored as bfloat16 or float16 tensors (the
    format follows their dtype; both must match); returns the fp32 partials."""
    _check_head_dims(q, k_pages, v_pages)
    for name, t in (("k_pages", k_pages), ("v_pages", v_pages)):
        if not isinstance(t, torch.Tensor) or t.dtype not in _KV16_FORMATS:
            raise TypeError(f"{name} must be a bfloat16 or float16 tensor")
    if k_pages.dtype != v_pages.dtype:
        raise TypeError("k_pages and v_pages must share one dtype")
    fmt = _KV16_FORMATS[k_pages.dtype]
    rows = index.c.max_edges * (hq // hkv if hkv > 0 else 1)
    dev = q.device
    if o_partial is None:
        o_partial = torch.empty((rows, head_dim), dtype=torch.float32, device=dev)
    if m_partial is None:
        m_partial = torch.empty(rows, dtype=torch.float32, device=dev)
    if l_partial is None:
        l_partial = torch.empty(rows, dtype=torch.float32, device=dev)
    st = lib().sa_forward_kv16(
        ctypes.byref(index.c), _ptr(q, torch.float32, "q"), q.numel(),
        _ptr(k_pages, k_pages.dtype, "k_pages"), k_pages.numel(),
        _ptr(v_pages, v_pages.dtype, "v_pages"), v_pages.numel(), fmt,
        _ptr(block_tables, torch.int32, "block_tables"),
        _ptr(cu_seqlens_q, torch.int64, "cu_seqlens_q"),
        _ptr(used_kv_lens, torch.int32, "used_kv_lens"),
        hq, hkv, head_dim, block_size, page_size, float(softmax_scale), int(bool(causal)),
        _ptr(o_partial, torch.float32, "o_partial"), _ptr(m_partial, torch.float32, "m_partial"),
        _ptr(l_partial, torch.float32, "l_partial"), _stream(dev))
    _check(st)
    return o_partial, m_partial, l_partial


def sa_combine(index: Index, o_partial, m_partial, l_partial, hq, head_dim, out=None,
               lse=None, with_lse=True):
    dev = o_partial.device
    tq = index.c.tq
    if out is None:
        out = torch.empty((tq, hq, head_dim), dtype=torch.float32, device=dev)
    if lse is None and with_lse:
        lse = torch.empty((tq, hq), dtype=torch.float32, device=dev)
    st = lib().sa_combine(ctypes.byref(index.c), _ptr(o_partial, torch.float32, "o_partial"),
                          _ptr(m_partial, torch.float32, "m_partial"),
                          _ptr(l_partial, torch.float32, "l_partial"), hq, head_dim,
                          _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"),
                          _stream(dev))
    _check(st)
    return out, lse


def sa_forward_combine(index: Index, selected, q, k_pages, v_pages, block_tables, cu_seqlens_q,
                       used_kv_lens, hq, hkv, head_dim, block_size, page_size, softmax_scale,
                       causal, out=None, lse=None, with_lse=True):
    """Forward and combine in one launch (no partials): returns (out, lse)."""
    _check_head_dims(q, k_pages, v_pages)
    dev = q.device
    tq = index.c.tq
    if out is None:
        out = torch.empty((tq, hq, head_dim), dtype=torch.float32, device=dev)
    if lse is None and with_lse:
        lse = torch.empty((tq, hq), dtype=torch.float32, device=dev)
    st = lib().sa_forward_combine(
        ctypes.byref(index.c), _ptr(selected, torch.int32, "selected"), selected.numel(),
        _ptr(q, torch.float32, "q"), q.numel(),
        _ptr(k_pages, torch.float32, "k_pages"), k_pages.numel(),
        _ptr(v_pages, torch.float32, "v_pages"), v_pages.numel(),
        _ptr(block_tables, torch.int32, "block_tables"),
        _ptr(cu_seqlens_q, torch.int64, "cu_seqlens_q"),
        _ptr(used_kv_lens, torch.int32, "used_kv_lens"),
        hq, hkv, head_dim, block_size, page_size, float(softmax_scale), int(bool(causal)),
        _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"), _stream(dev))
    _check(st)
    return out, lse


def sa_forward_combine_kv16(index: Index, selected, q, k_pages, v_pages, block_tables,
                            cu_seqlens_q, used_kv_lens, hq, hkv, head_dim, block_size, page_size,
                            softmax_scale, causal, out=None, lse=None, with_lse=True):
    """sa_forward_combine with K/V pages stored as bfloat16 or float16 tensors
    (the format follows their dtype; both must match): returns (out, lse)."""
    _check_head_dims(q, k_pages, v_pages)
    for name, t in (("k_pages", k_pages), ("v_pages", v_pages)):
        if not isinstance(t, torch.Tensor) or t.dtype not in _KV16_FORMATS:
            raise TypeError(f"{name} must be a bfloat16 or float16 tensor")
    if k_pages.dtype != v_pages.dtype:
        raise TypeError("k_pages and v_pages must share one dtype")
    dev = q.device
    tq = index.c.tq
    if out is None:
        out = torch.empty((tq, hq, head_dim), dtype=torch.float32, device=dev)
    if lse is None and with_lse:
        lse = torch.empty((tq, hq), dtype=torch.float32, device=dev)
    st = lib().sa_forward_combine_kv16(
        ctypes.byref(index.c), _ptr(selected, torch.int32, "selected"), selected.numel(),
        _ptr(q, torch.float32, "q"), q.numel(),
        _ptr(k_pages, k_pages.dtype, "k_pages"), k_pages.numel(),
        _ptr(v_pages, v_pages.dtype, "v_pages"), v_pages.numel(), _KV16_FORMATS[k_pages.dtype],
        _ptr(block_tables, torch.int32, "block_tables"),
        _ptr(cu_seqlens_q, torch.int64, "cu_seqlens_q"),
        _ptr(used_kv_lens, torch.int32, "used_kv_lens"),
        hq, hkv, head_dim, block_size, page_size, float(softmax_scale), int(bool(causal)),
        _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"), _stream(dev))
    _check(st)
    return out, lse


def fused_fits(hq, hkv, head_dim, block_size, page_size, topk):
    """Whether sa_forward_combine takes this geometry (include/sa.h)."""
    return head_dim == 128 and block_size <= 64 and hq // hkv <= 16 and topk <= 512


def sa_attention_workspace_bytes(tq, hkv, topk, batch, max_pages, block_size, page_size, hq,
                                 head_dim) -> int:
    n = c_size_t(0)
    _check(lib().sa_attention_workspace_bytes(tq, hkv, topk, batch, max_pages, block_size,
                                              page_size, hq, head_dim, ctypes.byref(n)))
    return int(n.value)


class Workspace:
    """A 256-byte aligned device buffer reused across sa_attention calls."""

    def __init__(self, nbytes, device="cuda"):
        self.raw = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        off = (-self.raw.data_ptr()) % 256
        self.nbytes = nbytes
        self.ptr = self.raw.data_ptr() + off


def sa_attention(q, k_pages, v_pages, selected, block_tables, cu_seqlens_q, used_kv_lens,
                 block_size, softmax_scale, causal, *, tq=None,
                 workspace: Workspace | None = None,
                 out=None, lse=None, with_lse=True, return_index=False, check=True):
    """build -> forward -> combine on the current stream.

    Shapes: q [tq, hq, d]; k_pages/v_pages [num_pages, hkv, page_size, d];
    selected [tq, hkv, topk]; block_tables [batch, max_pages];
    cu_seqlens_q [batch+1] (int64); used_kv_lens [batch] (int32) or None.
    ``tq`` defaults to q.shape[0]. Errors the build finds on the device
    (cu_seqlens content, selected ids, page ids) fill ``out`` and ``lse`` with
    NaN; with ``check`` (the default) this call then waits for the stream,
    reads the build's status and raises ``SaError``. ``check=False`` leaves the
    call asynchronous; ``sa_index_status`` on the returned index reads the
    status later.
    """
    _check_head_dims(q, k_pages, v_pages)
    if tq is None:
        tq = q.shape[0]
    hq = q.shape[1] if q.dim() == 3 else 0
    hkv, page_size, head_dim = k_pages.shape[1], k_pages.shape[2], k_pages.shape[3]
    topk = selected.shape[-1]
    batch, max_pages = block_tables.shape if block_tables.dim() == 2 else (
        cu_seqlens_q.numel() - 1, block_tables.numel() // max(cu_seqlens_q.numel() - 1, 1))
    dev = q.device
    if workspace is None:
        nbytes = sa_attention_workspace_bytes(tq, hkv, topk, batch, max_pages, block_size,
                                              page_size, hq, head_dim)
        workspace = Workspace(nbytes, dev)
    if out is None:
        out = torch.empty((tq, hq, head_dim), dtype=torch.float32, device=dev)
    if lse is None and with_lse:
        lse = torch.empty((tq, hq), dtype=torch.float32, device=dev)
    c = SaIndex()
    st = lib().sa_attention(
        _ptr(q, torch.float32, "q"), q.numel(),
        _ptr(k_pages, torch.float32, "k_pages"), k_pages.numel(),
        _ptr(v_pages, torch.float32, "v_pages"), v_pages.numel(),
        _ptr(selected, torch.int32, "selected"), selected.numel(),
        _ptr(block_tables, torch.int32, "block_tables"), block_tables.numel(),
        _ptr(cu_seqlens_q, torch.int64, "cu_seqlens_q"), cu_seqlens_q.numel(),
        _ptr(used_kv_lens, torch.int32, "used_kv_lens"),
        0 if used_kv_lens is None else used_kv_lens.numel(),
        tq, hq, hkv, head_dim, topk, batch, max_pages, block_size, page_size,
        float(softmax_scale), int(bool(causal)), c_void_p(workspace.ptr), workspace.nbytes,
        _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"), ctypes.byref(c),
        _stream(dev))
    _check(st)
    index = Index(c, workspace.raw)
    if check:
        sa_index_status(index, check=True, device=dev)
    if return_index:
        return out, lse, index
    return out, lse


SA_NOALLOC_SCRATCH_BYTES = 32 << 20     # include/sa.h


def sa_attention_noalloc(q, k_pages, v_pages, selected, block_tables, cu_seqlens_q,
                         used_kv_lens, block_size, softmax_scale, causal, out, lse=None, *,
                         tq=None, check=False, return_index=False):
    """sa_attention with the library's own per-GPU workspace: the C call
    allocates nothing, and neither does this wrapper (``out`` is required and
    ``lse`` optional, both caller tensors). Calls on one GPU share the
    workspace and must not overlap. ``check`` reads the build's status
    (a host wait) and raises ``SaError`` on a device-side input error."""
    _check_head_dims(q, k_pages, v_pages)
    if tq is None:
        tq = q.shape[0]
    hq = q.shape[1] if q.dim() == 3 else 0
    hkv, page_size, head_dim = k_pages.shape[1], k_pages.shape[2], k_pages.shape[3]
    topk = selected.shape[-1]
    batch, max_pages = block_tables.shape
    c = SaIndex()
    st = lib().sa_attention_noalloc(
        _ptr(q, torch.float32, "q"), q.numel(),
        _ptr(k_pages, torch.float32, "k_pages"), k_pages.numel(),
        _ptr(v_pages, torch.float32, "v_pages"), v_pages.numel(),
        _ptr(selected, torch.int32, "selected"), selected.numel(),
        _ptr(block_tables, torch.int32, "block_tables"), block_tables.numel(),
        _ptr(cu_seqlens_q, torch.int64, "cu_seqlens_q"), cu_seqlens_q.numel(),
        _ptr(used_kv_lens, torch.int32, "used_kv_lens"),
        0 if used_kv_lens is None else used_kv_lens.numel(),
        tq, hq, hkv, head_dim, topk, batch, max_pages, block_size, page_size,
        float(softmax_scale), int(bool(causal)),
        _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"), ctypes.byref(c),
        _stream(q.device))
    _check(st)
    index = Index(c, None)
    if check:
        sa_index_status(index, check=True, device=q.device)
    return (out, lse, index) if return_index else (out, lse)


def index_arrays(index: Index, info: dict | None = None) -> dict:
    """Views of the index arrays inside its device buffer (for tests and
    external consumers). ``edges`` and ``units`` are trimmed to the device
    counts in ``info`` (from sa_index_status)."""
    c = index.c
    if c.buffer is None or index.buffer is None:
        raise ValueError("index has no buffer")
    base = c.buffer - index.buffer.data_ptr()
    buf = index.buffer

    def view(off, n, dtype, shape):
        itemsize = torch.empty((), dtype=dtype).element_size()
        start = base + off
        return buf[start:start + n * itemsize].view(dtype).reshape(shape)

    hkv, nbs, tq, topk = c.hkv, c.nbs, c.tq, c.topk
    if info is None:
        info = sa_index_status(index)
    E = info["total_edges"]
    out = {
        "sel_slots": view(c.off_sel_slots, hkv * nbs, torch.int32, (hkv, nbs)),
        "sel_offsets": view(c.off_sel_offsets, hkv * (nbs + 1), torch.int32, (hkv, nbs + 1)),
        "num_sel": view(c.off_num_sel, hkv, torch.int32, (hkv,)),
        "edge_head_base": view(c.off_edge_head_base, hkv + 1, torch.int64, (hkv + 1,)),
        "edges": view(c.off_edges, 2 * E, torch.int32, (E, 2)),
        "inv": view(c.off_inv, hkv * tq * topk, torch.int32, (hkv, tq, topk)),
        "units_wave": view(c.off_units_wave, 8 * info["num_units_wave"], torch.int32,
                           (info["num_units_wave"], 8)),
        "units_mfma": view(c.off_units_mfma, 8 * info["num_units_mfma"], torch.int32,
                           (info["num_units_mfma"], 8)),
    }
    return out


__all__ = [
    "SaError", "SaIndex", "Index", "Workspace", "lib", "sa_index_plan", "sa_build_index",
    "sa_index_status", "sa_forward", "sa_forward_kv16", "sa_combine", "sa_forward_combine",
    "sa_forward_combine_kv16",
    "fused_fits", "sa_attention",
    "SA_KV_F32", "SA_KV_BF16", "SA_KV_F16",
    "sa_attention_workspace_bytes", "sa_attention_noalloc", "SA_NOALLOC_SCRATCH_BYTES",
    "index_arrays", "STATUS_NAMES",
]
