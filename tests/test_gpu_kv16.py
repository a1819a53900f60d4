"""GPU parity of the forward on K/V pages stored as 16-bit words
(``sa_forward_kv16``, bfloat16 and IEEE fp16), on every forward kernel.

The words come from ``workloads.encode_kv16`` (round to nearest even). The
oracle decodes them itself (``oracle.decode_kv16``) and runs the fp32-input
query-outer attention on the decoded values, in float64. The bound is the
fp32 path's: ``max|O_gpu - O_ref| <= 1e-4 * max|O_ref|`` and lse to 1e-4.
On the same index, the 16-bit forward and the fp32 forward on the decoded
values give bitwise identical partials where the kernel converts each word
exactly to fp32 (same arithmetic on the same fp32 operands). The one-wave
and fused kernels (head_dim 128, blocks of at most 64 keys, at most 16
rows a unit) and the direct-to-LDS MFMA kernel (blocks of 65..128 keys)
instead run both formats on the 16-bit matrix cores: q as three terms of
the format (fp16: after a power-of-two row scale) and the probabilities p
as two. There the partials match the fp32 path's to
within the low part that p's split drops (below 2^-16 p a key), bounded
per row by 2^-16 * l * max|V|.
"""
import numpy as np
import pytest
import torch

import block_sparse_paged_csr_amd as sa
import oracle
import workloads as W
from _gpu import dev_inputs, max_rel_err, run_index

pytestmark = pytest.mark.gpu

TOL_O = 1e-4
TOL_LSE = 1e-4
TORCH16 = {"bf16": torch.bfloat16, "fp16": torch.float16}


def _pages16(w, fmt, device="cuda"):
    k = W.encode_kv16(w.k_pages, fmt)
    v = W.encode_kv16(w.v_pages, fmt)
    kt = torch.from_numpy(k.view(np.int16)).to(device).view(TORCH16[fmt])
    vt = torch.from_numpy(v.view(np.int16)).to(device).view(TORCH16[fmt])
    return k, v, kt, vt


def _assert_partials_match_fp32_path(fmt, rows, vdec, p16, p32, exact=False):
    """The 16-bit path's partials against the fp32 path's on the decoded
    pages: bitwise where every word converts exactly (`exact`); on the 16-bit
    matrix cores the scores carry q's 24 bits (three terms), so m and l agree
    to fp32 rounding, and o differs by at most the dropped part of p's
    two-term split, below 2^-16 p for each key: |o16 - o32| <= 2^-16 * l *
    max|V| on every row (4x for the scores' own rounding)."""
    o16, m16, l16 = (x[:rows] for x in p16)
    o32, m32, l32 = (x[:rows] for x in p32)
    if exact:
        assert torch.equal(o16, o32) and torch.equal(m16, m32) and torch.equal(l16, l32)
        return
    o16, m16, l16, o32, m32, l32 = (x.cpu().double() for x in (o16, m16, l16, o32, m32, l32))
    fin = torch.isfinite(m32)
    assert torch.equal(fin, torch.isfinite(m16))
    if fin.any():
        assert (m16[fin] - m32[fin]).abs().max().item() <= 1e-5 * max(1.0, m32[fin].abs().max().item())
    assert ((l16 - l32).abs() <= 1e-5 * l32.abs() + 1e-30).all()
    bound = 4 * 2.0 ** -16 * l32 * float(np.abs(vdec).max())
    assert ((o16 - o32).abs() <= bound[:, None] + 1e-30).all()


def _fwd_args(w, d):
    return (d["bt"], d["cu"], d["used"], w.hq, w.hkv, w.head_dim, w.block_size, w.page_size,
            w.softmax_scale, w.causal)


def _check(w, kdec, vdec, out, lse, queries=None):
    ref_o, ref_lse = oracle.attention_qo_ref(
        w.q, kdec, vdec, w.selected, w.block_tables, w.cu_seqlens_q, w.used_kv_lens, w.hq,
        w.hkv, w.head_dim, w.block_size, w.page_size, w.softmax_scale, w.causal,
        queries=queries)
    got_o = out.cpu().numpy().astype(np.float64)
    got_lse = lse.cpu().numpy().astype(np.float64)
    if queries is not None:
        got_o, got_lse = got_o[queries], got_lse[queries]
    err, _ = max_rel_err(got_o, ref_o)
    assert err <= TOL_O, err
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(got_lse))
    if fin.any():
        assert np.abs(got_lse[fin] - ref_lse[fin]).max() <= TOL_LSE
    return err


GEOM = [(4, 1), (2, 8), (8, 2), (16, 1), (4, 6), (8, 4), (16, 3), (16, 4)]


@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
@pytest.mark.parametrize("seed", range(8))
def test_random_kv16_matches_oracle(fmt, seed):
    ps, ppb = GEOM[seed % len(GEOM)]
    w = W.make_random(4100 + seed, batch=1 + seed % 4, qo_max=6, kv_max=260, hkv=1 + seed % 3,
                      qhead=[1, 2, 4, 8, 16][seed % 5], head_dim=128, page_size=ps,
                      pages_per_block=ppb, topk=1 + seed % 6)
    print(f"[gpu case] kv16 {fmt} seed={seed} tq={w.tq} bs={w.block_size}", flush=True)
    d = dev_inputs(w)
    k, v, kt, vt = _pages16(w, fmt)
    idx = run_index(w, d)
    o, m, l = sa.sa_forward_kv16(idx, d["q"], kt, vt, *_fwd_args(w, d))
    out, lse = sa.sa_combine(idx, o, m, l, w.hq, w.head_dim)
    _check(w, oracle.decode_kv16(k, fmt), oracle.decode_kv16(v, fmt), out, lse)


@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
@pytest.mark.parametrize("seed", range(3))
def test_kv16_partials_equal_fp32_path_on_decoded_pages(fmt, seed):
    w = W.make_random(4200 + seed, batch=2, qo_max=40, kv_max=300, hkv=2, qhead=4,
                      head_dim=128, page_size=16, pages_per_block=4, topk=6)
    print(f"[gpu case] kv16 bitwise {fmt} seed={seed}", flush=True)
    d = dev_inputs(w)
    k, v, kt, vt = _pages16(w, fmt)
    idx = run_index(w, d)
    o16, m16, l16 = sa.sa_forward_kv16(idx, d["q"], kt, vt, *_fwd_args(w, d))
    kd = torch.from_numpy(oracle.decode_kv16(k, fmt)).cuda()
    vd = torch.from_numpy(oracle.decode_kv16(v, fmt)).cuda()
    o32, m32, l32 = sa.sa_forward(idx, d["q"], kd, vd, *_fwd_args(w, d))
    rows = sa.sa_index_status(idx)["total_edges"] * (w.hq // w.hkv)
    _assert_partials_match_fp32_path(fmt, rows, oracle.decode_kv16(v, fmt), (o16, m16, l16),
                                     (o32, m32, l32))


@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
def test_decode_workload_kv16(fmt):
    w = W.make_config("decode")
    print(f"[gpu case] kv16 decode {fmt}", flush=True)
    d = dev_inputs(w)
    k, v, kt, vt = _pages16(w, fmt)
    idx = run_index(w, d)
    o, m, l = sa.sa_forward_kv16(idx, d["q"], kt, vt, *_fwd_args(w, d))
    out, lse = sa.sa_combine(idx, o, m, l, w.hq, w.head_dim)
    torch.cuda.synchronize()
    err = _check(w, oracle.decode_kv16(k, fmt), oracle.decode_kv16(v, fmt), out, lse)
    print(f"[gpu case] kv16 decode {fmt}: O rel err {err:.3e}", flush=True)


# The fused forward + combine on 16-bit pages (sa_forward_combine_kv16):
# decode-like batches (one or two queries a sequence, empty sequences) against
# the oracle on the decoded pages, the two-pass 16-bit path and the fused fp32
# path on the decoded values (1e-5).
@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
@pytest.mark.parametrize("seed", range(6))
def test_fused_forward_combine_kv16(fmt, seed):
    ps, ppb = [(16, 4), (16, 1), (8, 2), (4, 4), (16, 3), (32, 2)][seed]
    w = W.make_random(4600 + seed, batch=1 + seed % 7, qo_max=[1, 2][seed % 2], kv_max=400,
                      hkv=1 + seed % 3, qhead=[1, 2, 4, 8, 16][seed % 5], head_dim=128,
                      page_size=ps, pages_per_block=ppb, topk=1 + seed % 9,
                      causal=bool(seed % 3))
    print(f"[gpu case] fused kv16 {fmt} seed={seed} tq={w.tq} bs={w.block_size}", flush=True)
    d = dev_inputs(w)
    k, v, kt, vt = _pages16(w, fmt)
    idx = run_index(w, d)
    out, lse = sa.sa_forward_combine_kv16(idx, d["sel"], d["q"], kt, vt, *_fwd_args(w, d))
    kd, vd = oracle.decode_kv16(k, fmt), oracle.decode_kv16(v, fmt)
    _check(w, kd, vd, out, lse)
    o, m, l = sa.sa_forward_kv16(idx, d["q"], kt, vt, *_fwd_args(w, d))
    out2, lse2 = sa.sa_combine(idx, o, m, l, w.hq, w.head_dim)
    assert max_rel_err(out.cpu().numpy(), out2.cpu().numpy())[0] <= 1e-5
    fin = torch.isfinite(lse2)
    assert torch.equal(fin, torch.isfinite(lse))
    if fin.any():
        assert (lse[fin] - lse2[fin]).abs().max().item() <= 1e-5
    out3, lse3 = sa.sa_forward_combine(idx, d["sel"], d["q"], torch.from_numpy(kd).cuda(),
                                       torch.from_numpy(vd).cuda(), *_fwd_args(w, d))
    assert max_rel_err(out.cpu().numpy(), out3.cpu().numpy())[0] <= 1e-5
    fin = torch.isfinite(lse3)
    assert torch.equal(fin, torch.isfinite(lse))
    if fin.any():
        assert (lse[fin] - lse3[fin]).abs().max().item() <= 1e-5


def test_fused_kv16_rejects_geometry_and_selections():
    w = W.make_random(4650, batch=2, qo_max=1, kv_max=200, hkv=1, qhead=2, head_dim=64,
                      page_size=16, pages_per_block=2, topk=3)
    d = dev_inputs(w)
    k, v, kt, vt = _pages16(w, "bf16")
    idx = run_index(w, d)
    with pytest.raises(sa.SaError) as ei:
        sa.sa_forward_combine_kv16(idx, d["sel"], d["q"], kt, vt, *_fwd_args(w, d))
    assert ei.value.kind == "Unsupported"
    with pytest.raises(sa.SaError) as ei:
        sa.sa_forward_combine_kv16(idx, d["sel"][:-1], d["q"], kt, vt, *_fwd_args(w, d))
    assert (ei.value.kind, ei.value.what) == ("ShapeMismatch", "selected")


def test_decode_workload_fused_kv16_bf16():
    w = W.make_config("decode")
    print("[gpu case] fused kv16 decode bf16", flush=True)
    d = dev_inputs(w)
    k, v, kt, vt = _pages16(w, "bf16")
    idx = run_index(w, d)
    out, lse = sa.sa_forward_combine_kv16(idx, d["sel"], d["q"], kt, vt, *_fwd_args(w, d))
    torch.cuda.synchronize()
    err = _check(w, oracle.decode_kv16(k, "bf16"), oracle.decode_kv16(v, "bf16"), out, lse)
    print(f"[gpu case] fused kv16 decode bf16: O rel err {err:.3e}", flush=True)


# The 16-bit matrix-core paths split q into terms of the format; fp16 terms
# need q's rows scaled by a power of two first. q far above fp16's range
# (x 2e4: elements past 65504) and far below its normal range (x 1e-3:
# many elements under 2^-14), with K scaled the other way so that the
# scores stay of order one, against the oracle on the one-wave, fused and
# direct-to-LDS kernels.
@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
@pytest.mark.parametrize("scales", [(2e4, 5e-5), (1e-3, 1e3)])
@pytest.mark.parametrize("kernel", ["small", "fused", "mfma"])
def test_kv16_q_far_from_unit_range(fmt, scales, kernel):
    kernels = ["small", "fused", "mfma"]
    geo = {"small": dict(qo_max=12, page_size=16, pages_per_block=4, qhead=8),
           "fused": dict(qo_max=1, page_size=16, pages_per_block=2, qhead=4),
           "mfma": dict(qo_max=60, page_size=32, pages_per_block=4, qhead=8)}[kernel]
    q_scale, k_scale = scales
    w = W.make_random(4700 + 2 * kernels.index(kernel) + int(q_scale > 1), batch=3, kv_max=600,
                      hkv=2, head_dim=128, topk=4, causal=True, **geo)
    w.q = (w.q.astype(np.float64) * q_scale).astype(np.float32)
    w.k_pages = (w.k_pages.astype(np.float64) * k_scale).astype(np.float32)
    print(f"[gpu case] kv16 q range {fmt} q x{q_scale:g} k x{k_scale:g} {kernel} tq={w.tq} "
          f"bs={w.block_size}", flush=True)
    d = dev_inputs(w)
    k, v, kt, vt = _pages16(w, fmt)
    idx = run_index(w, d)
    n_mfma = sa.sa_index_status(idx)["num_units_mfma"]
    assert (n_mfma > 0) == (kernel == "mfma"), n_mfma
    if kernel == "fused":
        out, lse = sa.sa_forward_combine_kv16(idx, d["sel"], d["q"], kt, vt, *_fwd_args(w, d))
    else:
        o, m, l = sa.sa_forward_kv16(idx, d["q"], kt, vt, *_fwd_args(w, d))
        out, lse = sa.sa_combine(idx, o, m, l, w.hq, w.head_dim)
    _check(w, oracle.decode_kv16(k, fmt), oracle.decode_kv16(v, fmt), out, lse)


# Rows of one tile at very different scales (each q row times 10^u, u
# uniform in [-3, 4]): every row takes its own power of two on the fp16 path.
# Large rows give near-hard softmaxes with lse up to ~1e4, so lse is compared
# relative to its size; O to 1e-4 of max|O| as everywhere.
@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
@pytest.mark.parametrize("kernel", ["small", "fused", "mfma"])
def test_kv16_q_rows_of_mixed_scale(fmt, kernel):
    kernels = ["small", "fused", "mfma"]
    geo = {"small": dict(qo_max=12, page_size=16, pages_per_block=4, qhead=8),
           "fused": dict(qo_max=1, page_size=16, pages_per_block=2, qhead=4),
           "mfma": dict(qo_max=60, page_size=32, pages_per_block=4, qhead=8)}[kernel]
    w = W.make_random(4720 + kernels.index(kernel), batch=3, kv_max=600, hkv=2, head_dim=128,
                      topk=4, causal=True, **geo)
    rng = np.random.default_rng(4730 + kernels.index(kernel))
    row_scale = 10.0 ** rng.uniform(-3.0, 4.0, size=w.q.shape[:2])
    w.q = (w.q.astype(np.float64) * row_scale[:, :, None]).astype(np.float32)
    print(f"[gpu case] kv16 mixed row scales {fmt} {kernel} tq={w.tq} bs={w.block_size}", flush=True)
    d = dev_inputs(w)
    k, v, kt, vt = _pages16(w, fmt)
    idx = run_index(w, d)
    n_mfma = sa.sa_index_status(idx)["num_units_mfma"]
    assert (n_mfma > 0) == (kernel == "mfma"), n_mfma
    if kernel == "fused":
        out, lse = sa.sa_forward_combine_kv16(idx, d["sel"], d["q"], kt, vt, *_fwd_args(w, d))
    else:
        o, m, l = sa.sa_forward_kv16(idx, d["q"], kt, vt, *_fwd_args(w, d))
        out, lse = sa.sa_combine(idx, o, m, l, w.hq, w.head_dim)
    ref_o, ref_lse = oracle.attention_qo_ref(
        w.q, oracle.decode_kv16(k, fmt), oracle.decode_kv16(v, fmt), w.selected, w.block_tables,
        w.cu_seqlens_q, w.used_kv_lens, w.hq, w.hkv, w.head_dim, w.block_size, w.page_size,
        w.softmax_scale, w.causal)
    got_o = out.cpu().numpy().astype(np.float64)
    got_lse = lse.cpu().numpy().astype(np.float64)
    assert max_rel_err(got_o, ref_o)[0] <= TOL_O
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(got_lse))
    if fin.any():
        assert (np.abs(got_lse[fin] - ref_lse[fin]) <= TOL_LSE + 1e-6 * np.abs(ref_lse[fin])).all()


def test_ragged_workload_bf16_sampled():
    w = W.make_config("ragged")
    print("[gpu case] kv16 ragged bf16", flush=True)
    d = dev_inputs(w)
    k, v, kt, vt = _pages16(w, "bf16")
    idx = run_index(w, d)
    o, m, l = sa.sa_forward_kv16(idx, d["q"], kt, vt, *_fwd_args(w, d))
    out, lse = sa.sa_combine(idx, o, m, l, w.hq, w.head_dim)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    queries = np.sort(rng.choice(w.tq, size=24, replace=False))
    _check(w, oracle.decode_kv16(k, "bf16"), oracle.decode_kv16(v, "bf16"), out, lse, queries)


# Geometries of the other forward kernels: the wavefront kernel (head_dim
# other than 128), the 16-row MFMA kernel (blocks <= 64 keys, qhead > 16),
# the 32-row MFMA kernel (blocks of 96 / 128 keys) and the chunked MFMA
# kernel (head_dim 64 with 256-key blocks, 128 with 256, 256 with 128).
OTHER = [
    dict(head_dim=32, qhead=2, page_size=4, pages_per_block=2, qo_max=6, kv_max=120, topk=4),
    dict(head_dim=64, qhead=4, page_size=8, pages_per_block=4, qo_max=6, kv_max=300, topk=5),
    dict(head_dim=128, qhead=20, page_size=16, pages_per_block=4, qo_max=200, kv_max=600, topk=6),
    dict(head_dim=128, qhead=8, page_size=32, pages_per_block=4, qo_max=200, kv_max=1200, topk=6),
    dict(head_dim=128, qhead=4, page_size=32, pages_per_block=3, qo_max=150, kv_max=900, topk=5),
    dict(head_dim=64, qhead=8, page_size=32, pages_per_block=8, qo_max=80, kv_max=1500, topk=4),
    dict(head_dim=128, qhead=8, page_size=64, pages_per_block=4, qo_max=80, kv_max=1500, topk=4),
    dict(head_dim=256, qhead=8, page_size=16, pages_per_block=8, qo_max=50, kv_max=700, topk=4),
]


@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
@pytest.mark.parametrize("case", range(len(OTHER)))
def test_other_kernels_kv16(fmt, case):
    g = OTHER[case]
    w = W.make_random(4400 + case, batch=2, hkv=2, **g)
    print(f"[gpu case] kv16 other {fmt} case={case} tq={w.tq} d={w.head_dim} "
          f"bs={w.block_size} qhead={w.hq // w.hkv}", flush=True)
    d = dev_inputs(w)
    k, v, kt, vt = _pages16(w, fmt)
    idx = run_index(w, d)
    o, m, l = sa.sa_forward_kv16(idx, d["q"], kt, vt, *_fwd_args(w, d))
    out, lse = sa.sa_combine(idx, o, m, l, w.hq, w.head_dim)
    kd, vd = oracle.decode_kv16(k, fmt), oracle.decode_kv16(v, fmt)
    _check(w, kd, vd, out, lse)
    # and the fp32 path's partials on the decoded pages (bitwise where the
    # words are converted exactly)
    o32, m32, l32 = sa.sa_forward(idx, d["q"], torch.from_numpy(kd).cuda(),
                                  torch.from_numpy(vd).cuda(), *_fwd_args(w, d))
    rows = sa.sa_index_status(idx)["total_edges"] * (w.hq // w.hkv)
    # (fp16 words convert exactly in these kernels, but for the direct-to-LDS
    # MFMA kernel's: head_dim 128, blocks of 65..128 keys)
    exact = fmt == "fp16" and not (w.head_dim == 128 and 64 < w.block_size <= 128)
    _assert_partials_match_fp32_path(fmt, rows, vd, (o, m, l), (o32, m32, l32), exact=exact)


def test_prefill_workload_bf16_sampled():
    w = W.make_config("prefill")
    print("[gpu case] kv16 prefill bf16", flush=True)
    d = dev_inputs(w)
    k, v, kt, vt = _pages16(w, "bf16")
    idx = run_index(w, d)
    o, m, l = sa.sa_forward_kv16(idx, d["q"], kt, vt, *_fwd_args(w, d))
    out, lse = sa.sa_combine(idx, o, m, l, w.hq, w.head_dim)
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    queries = np.sort(rng.choice(w.tq, size=12, replace=False))
    _check(w, oracle.decode_kv16(k, "bf16"), oracle.decode_kv16(v, "bf16"), out, lse, queries)
