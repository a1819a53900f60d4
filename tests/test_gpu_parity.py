"""GPU parity: the HIP path through the C ABI against the CPU oracle.

* index: every array bit-exact against ``oracle.build_index_ref``;
* partials: per-edge (o, m, l) against ``oracle.forward_partials_ref`` (fp64);
* output: ``max|O_gpu - O_ref| <= 1e-4 * max|O_ref|`` against the query-outer
  oracle (fp64); lse to 1e-4 absolute.

Sizes: the tiny workload and random small geometries in full; the decode,
ragged, prefill and skewed workloads at full size in the launch configuration
the benchmark times, with the output compared on sampled queries (all queries
for decode) and the index compared in full.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_paged_csr_amd as sa
import oracle
import workloads as W
from _gpu import (assert_index_equal, check_partials, check_units, dev_inputs, max_rel_err,
                  oracle_index, qo_sampled, run_attention, run_index, sample_edges)

pytestmark = pytest.mark.gpu

TOL_O = 1e-4          # max|O_gpu - O_ref| / max|O_ref|
TOL_LSE = 1e-4        # absolute, natural-log units


def _qo(w, queries=None):
    return oracle.attention_qo_ref(w.q, w.k_pages, w.v_pages, w.selected, w.block_tables,
                                   w.cu_seqlens_q, w.used_kv_lens, w.hq, w.hkv, w.head_dim,
                                   w.block_size, w.page_size, w.softmax_scale, w.causal,
                                   queries=queries)


def _print_case(case, **kw):
    print(f"[gpu case] {case} {kw}", flush=True)


def _check_output(w, out, lse, queries=None, parallel=False):
    if parallel:
        qs = np.arange(w.tq) if queries is None else queries
        ref_o, ref_lse = qo_sampled(w, qs, workers=8)
    else:
        ref_o, ref_lse = _qo(w, queries)
    got_o = out.cpu().numpy().astype(np.float64)
    got_lse = lse.cpu().numpy().astype(np.float64)
    if queries is not None:
        got_o, got_lse = got_o[queries], got_lse[queries]
    err, scale = max_rel_err(got_o, ref_o)
    assert err <= TOL_O, f"O rel err {err:.3e} (max|O| {scale:.3e})"
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(got_lse))
    if fin.any():
        assert np.abs(got_lse[fin] - ref_lse[fin]).max() <= TOL_LSE
    assert np.all(got_o[~fin] == 0.0)            # nothing alive: O = 0
    return err


@pytest.fixture(params=["fused", "multi"])
def build_path(request, monkeypatch):
    """Small problems build in one fused kernel; SA_BUILD_MULTIKERNEL=1 keeps
    them on the multi-kernel build that large problems take."""
    if request.param == "multi":
        monkeypatch.setenv("SA_BUILD_MULTIKERNEL", "1")
    else:
        monkeypatch.delenv("SA_BUILD_MULTIKERNEL", raising=False)
    return request.param


# ------------------------------------------------------------------ small cases

@pytest.mark.parametrize("seed", range(24))
def test_random_small_end_to_end(seed):
    w = W.make_random(500 + seed, batch=1 + seed % 3, qo_max=5, kv_max=40,
                      hkv=1 + seed % 2, qhead=1 + seed % 4, head_dim=[8, 16, 32, 64][seed % 4],
                      page_size=[1, 2, 4][seed % 3], pages_per_block=1 + seed % 3,
                      topk=1 + seed % 5)
    _print_case("random_small", seed=seed, tq=w.tq, d=w.head_dim)
    d = dev_inputs(w)
    idx = run_index(w, d)
    ref = oracle_index(w)
    info, arrs = assert_index_equal(idx, ref)
    check_units(arrs, info, ref, idx.c.cap_edges, w)
    out, lse = run_attention(w, d)
    _check_output(w, out, lse)


@pytest.mark.parametrize("seed", range(8))
def test_random_small_index_multikernel(seed, monkeypatch):
    monkeypatch.setenv("SA_BUILD_MULTIKERNEL", "1")
    w = W.make_random(500 + seed, batch=1 + seed % 3, qo_max=5, kv_max=40,
                      hkv=1 + seed % 2, qhead=1 + seed % 4, head_dim=8,
                      page_size=[1, 2, 4][seed % 3], pages_per_block=1 + seed % 3,
                      topk=1 + seed % 5)
    _print_case("random_small_multikernel", seed=seed, tq=w.tq)
    d = dev_inputs(w)
    idx = run_index(w, d)
    ref = oracle_index(w)
    info, arrs = assert_index_equal(idx, ref)
    check_units(arrs, info, ref, idx.c.cap_edges, w)


# head_dim 128 with blocks of at most 64 keys: the one-wave-per-unit forward,
# with 1..4 pieces of 16 keys per block, partial pieces and up to 16 rows a unit
D128_GEOM = [(4, 1), (2, 8), (8, 2), (16, 1), (4, 6), (8, 4), (16, 3), (16, 4), (2, 3), (32, 2)]


@pytest.mark.parametrize("seed", range(20))
def test_random_d128_end_to_end(seed):
    ps, ppb = D128_GEOM[seed % len(D128_GEOM)]
    w = W.make_random(1300 + seed, batch=1 + seed % 4, qo_max=6, kv_max=260,
                      hkv=1 + seed % 3, qhead=[1, 2, 4, 8, 16][seed % 5], head_dim=128,
                      page_size=ps, pages_per_block=ppb, topk=1 + seed % 6)
    _print_case("random_d128", seed=seed, tq=w.tq, bs=w.block_size, qhead=w.hq // w.hkv)
    d = dev_inputs(w)
    idx = run_index(w, d)
    ref = oracle_index(w)
    info, arrs = assert_index_equal(idx, ref)
    check_units(arrs, info, ref, idx.c.cap_edges, w)
    out, lse = run_attention(w, d)
    _check_output(w, out, lse)


# Larger random batches (more than 4096 entries a head) on head_dim 128 and
# blocks of at most 64 keys: every slot stays on the one-wave kernel, a slot
# with more than 16 rows split into several 16-row units over the same block.
SPLIT_GEOM = [(4, 1), (8, 2), (16, 1), (16, 3), (16, 4), (32, 2), (2, 8), (8, 4)]
SPLIT_SEEDS = [0, 1, 3, 4, 5, 6, 7, 8, 9, 10, 11, 13]


@pytest.mark.parametrize("seed", SPLIT_SEEDS)
def test_random_d128_split_units(seed):
    ps, ppb = SPLIT_GEOM[seed % len(SPLIT_GEOM)]
    w = W.make_random(2100 + seed, batch=2 + seed % 2, qo_max=700, kv_max=900, hkv=1 + seed % 2,
                      qhead=[2, 4, 8, 16][seed % 4], head_dim=128, page_size=ps,
                      pages_per_block=ppb, topk=8)
    _print_case("random_d128_split", seed=seed, tq=w.tq, bs=w.block_size, qhead=w.hq // w.hkv)
    d = dev_inputs(w)
    idx = run_index(w, d)
    ref = oracle_index(w)
    info, arrs = assert_index_equal(idx, ref)
    assert info["num_units_mfma"] == 0
    assert info["num_units_wave"] > int(ref["num_sel"].sum())     # some slots were split
    check_units(arrs, info, ref, idx.c.wave_cap_edges, w)
    out, lse = run_attention(w, d)
    _check_output(w, out, lse)


# Head dims other than 64, 128 and 256 take the wavefront-reduction kernel
# only, built for head_dim/4 rounded up to a power of two (1 .. 64 float4
# columns): dims that are not a power of two mask the padded columns, and
# head_dim 256 with 16 GQA lanes is the largest qhead * head_dim the library
# takes (4096; its slots of 32 rows or more take the chunked MFMA kernel).
WAVE_DIMS = [(4, 3), (12, 5), (100, 2), (132, 3), (256, 16), (256, 1), (40, 7), (252, 4)]


@pytest.mark.parametrize("case", range(len(WAVE_DIMS)))
def test_random_head_dims_wave_kernel(case):
    d, qhead = WAVE_DIMS[case]
    w = W.make_random(7100 + case, batch=1 + case % 3, qo_max=5, kv_max=60, hkv=1 + case % 2,
                      qhead=qhead, head_dim=d, page_size=[2, 4, 8][case % 3],
                      pages_per_block=2 + case % 3, topk=2 + case % 4)
    _print_case("random_head_dims", idx=case, head_dim=d, qhead=qhead, tq=w.tq)
    d_in = dev_inputs(w)
    idx = run_index(w, d_in)
    ref = oracle_index(w)
    info, arrs = assert_index_equal(idx, ref)
    if d not in (64, 128, 256):
        assert info["num_units_mfma"] == 0
    check_units(arrs, info, ref, idx.c.cap_edges, w)
    out, lse = run_attention(w, d_in)
    _check_output(w, out, lse)


# Blocks of 96 and 128 keys on head_dim 128: slots of 32 rows or more take
# the MFMA kernel that stages the block in LDS (3 or 4 32-key column blocks),
# the rest the wavefront-reduction kernel; with page holes, ids past the used
# length, partial last blocks and either causal mode.
LARGE_BLOCK_GEOM = [(32, 3), (32, 4), (64, 2), (16, 8), (48, 2), (8, 12)]


@pytest.mark.parametrize("seed", range(8))
def test_random_large_blocks_mfma(seed):
    ps, ppb = LARGE_BLOCK_GEOM[seed % len(LARGE_BLOCK_GEOM)]
    w = W.make_random(7300 + seed, batch=1 + seed % 3, qo_max=40, kv_max=700, hkv=1 + seed % 2,
                      qhead=[4, 8, 16, 8][seed % 4], head_dim=128, page_size=ps,
                      pages_per_block=ppb, topk=3 + seed % 4, causal=seed % 2 == 1)
    _print_case("random_large_blocks", seed=seed, tq=w.tq, bs=w.block_size, qhead=w.hq // w.hkv)
    d_in = dev_inputs(w)
    idx = run_index(w, d_in)
    ref = oracle_index(w)
    info, arrs = assert_index_equal(idx, ref)
    assert info["num_units_mfma"] > 0
    check_units(arrs, info, ref, idx.c.cap_edges, w)
    out, lse = run_attention(w, d_in)
    _check_output(w, out, lse)


# More than 16 query heads per KV head on head_dim 128 and blocks of at most
# 64 keys: slots of 32 rows or more take the MFMA kernel for such blocks
# (16-row tiles staged through LDS), the rest the wavefront-reduction kernel.
WIDE_GEOM = [(16, 4), (8, 2), (16, 1), (4, 8), (32, 2), (16, 3)]


@pytest.mark.parametrize("seed", range(8))
def test_random_d128_wide_gqa_mfma_units(seed):
    ps, ppb = WIDE_GEOM[seed % len(WIDE_GEOM)]
    w = W.make_random(2300 + seed, batch=2, qo_max=300, kv_max=700, hkv=1 + seed % 2,
                      qhead=[17, 20, 24, 32][seed % 4], head_dim=128, page_size=ps,
                      pages_per_block=ppb, topk=6)
    _print_case("random_d128_wide_gqa", seed=seed, tq=w.tq, bs=w.block_size, qhead=w.hq // w.hkv)
    d = dev_inputs(w)
    idx = run_index(w, d)
    ref = oracle_index(w)
    info, arrs = assert_index_equal(idx, ref)
    assert info["num_units_mfma"] > 0
    check_units(arrs, info, ref, idx.c.cap_edges, w)
    out, lse = run_attention(w, d)
    _check_output(w, out, lse)


# The chunked MFMA kernel end to end: head_dim 64, 128 and 256 with blocks
# of one chunk, several chunks and a partial last chunk (block sizes that are
# not a multiple of the chunk), page holes, ids past the used length, GQA
# widths up to 16 lanes and either causal mode; units of multi-chunk blocks
# capped at one tile a wave. (head_dim, page_size, pages_per_block, qhead)
GENERAL_GEOM = [(64, 16, 4, 8), (64, 32, 8, 4), (64, 48, 4, 16), (128, 64, 3, 8), (128, 32, 8, 4),
                (256, 16, 2, 16), (256, 32, 2, 8), (256, 16, 6, 4), (128, 80, 2, 16), (64, 8, 4, 2)]


@pytest.mark.parametrize("case", range(len(GENERAL_GEOM)))
def test_random_general_mfma(case):
    d, ps, ppb, qhead = GENERAL_GEOM[case]
    w = W.make_random(7700 + case, batch=1 + case % 3, qo_max=40 if d == 256 else 70,
                      kv_max=ps * ppb * 6, hkv=1 + case % 2, qhead=qhead, head_dim=d,
                      page_size=ps, pages_per_block=ppb, topk=3 + case % 3, causal=case % 2 == 1)
    _print_case("random_general_mfma", idx=case, head_dim=d, bs=w.block_size, qhead=qhead, tq=w.tq)
    d_in = dev_inputs(w)
    idx = run_index(w, d_in)
    ref = oracle_index(w)
    info, arrs = assert_index_equal(idx, ref)
    assert info["num_units_mfma"] > 0
    check_units(arrs, info, ref, idx.c.cap_edges, w)
    out, lse = run_attention(w, d_in)
    _check_output(w, out, lse)


# Partial-level parity on every forward kernel: (o, m, l) per edge and lane
# against the oracle, so that the reference point m (which the combine cannot
# see) is checked on each of them.
#   wave:   head_dim 32, the wavefront-reduction kernel
#   small:  head_dim 128, blocks <= 64 keys, qhead <= 16: the one-wave kernel
#   mfma16: head_dim 128, blocks <= 64 keys, qhead > 16: 16-row MFMA tiles
#   mfma:   head_dim 128, blocks of 96 / 128 keys: 32-row MFMA tiles (slots
#           under 32 rows take the wavefront kernel)
#   gen64, gen128, gen256: the chunked MFMA kernel on head_dim 64 (blocks of
#           64, 128, 256 keys: one or two 128-key chunks), 128 (blocks of 192
#           and 256 keys) and 256 (blocks of 32, 64, 128 keys: 32- and 64-key
#           chunks), where a later chunk can raise a row's max
PARTIAL_KERNELS = {
    "wave": dict(head_dim=32, page_size=2, pages_per_block=(2, 3), qhead=(1, 2, 3),
                 qo_max=4, kv_max=48, topk=3),
    "small": dict(head_dim=128, page_size=16, pages_per_block=(1, 2, 4), qhead=(1, 4, 8, 16),
                  qo_max=12, kv_max=300, topk=4),
    "mfma16": dict(head_dim=128, page_size=16, pages_per_block=(2, 4), qhead=(20, 32),
                   qo_max=40, kv_max=260, topk=3),
    "mfma": dict(head_dim=128, page_size=32, pages_per_block=(3, 4), qhead=(4, 8, 16),
                 qo_max=60, kv_max=600, topk=3),
    "gen64": dict(head_dim=64, page_size=32, pages_per_block=(2, 4, 8), qhead=(4, 8, 16),
                  qo_max=60, kv_max=900, topk=3),
    "gen128": dict(head_dim=128, page_size=64, pages_per_block=(3, 4), qhead=(4, 8, 16),
                   qo_max=60, kv_max=900, topk=3),
    "gen256": dict(head_dim=256, page_size=16, pages_per_block=(2, 4, 8), qhead=(4, 8, 16),
                   qo_max=50, kv_max=500, topk=3),
}


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("kernel", list(PARTIAL_KERNELS))
def test_random_partials_match_kvouter_ref(kernel, seed):
    g = PARTIAL_KERNELS[kernel]
    w = W.make_random(700 + 37 * seed + 1000 * list(PARTIAL_KERNELS).index(kernel),
                      batch=1 + seed % 3, qo_max=g["qo_max"], kv_max=g["kv_max"],
                      hkv=1 + seed % 2, qhead=g["qhead"][seed % len(g["qhead"])],
                      head_dim=g["head_dim"], page_size=g["page_size"],
                      pages_per_block=g["pages_per_block"][seed % len(g["pages_per_block"])],
                      topk=g["topk"], causal=bool(seed % 2))
    _print_case("random_partials", kernel=kernel, seed=seed, tq=w.tq, bs=w.block_size,
                qhead=w.hq // w.hkv)
    d = dev_inputs(w)
    idx = run_index(w, d)
    ref = oracle_index(w)
    info, _ = assert_index_equal(idx, ref)
    if kernel in ("mfma16", "mfma") or kernel.startswith("gen"):
        assert info["num_units_mfma"] > 0, "no unit reached the MFMA kernel"
    else:
        assert info["num_units_mfma"] == 0
    check_partials(w, d, idx, ref)


# The fused forward + combine (sa_forward_combine; sa_attention takes it when
# tq == batch): one workgroup per (query, KV head) merges the query's kept
# blocks as it reads them. Exact for any batch, so it is checked on decode-like
# batches with empty sequences and sequences of two queries too (shared
# blocks, and the batch_of search instead of b = q), against the oracle and
# against the two-pass path (sa_forward + sa_combine).
FUSED_GEOM = [(16, 4), (16, 1), (8, 2), (4, 4), (16, 3), (32, 2), (2, 8)]


@pytest.mark.parametrize("seed", range(14))
def test_fused_forward_combine(seed):
    ps, ppb = FUSED_GEOM[seed % len(FUSED_GEOM)]
    w = W.make_random(8800 + seed, batch=1 + seed % 7, qo_max=[1, 2][seed % 2], kv_max=400,
                      hkv=1 + seed % 3, qhead=[1, 2, 4, 8, 16][seed % 5], head_dim=128,
                      page_size=ps, pages_per_block=ppb, topk=1 + seed % 9,
                      causal=bool(seed % 3))
    _print_case("fused_forward_combine", seed=seed, tq=w.tq, batch=w.batch, bs=w.block_size,
                qhead=w.hq // w.hkv, topk=w.topk)
    d = dev_inputs(w)
    idx = run_index(w, d)
    ref = oracle_index(w)
    assert_index_equal(idx, ref)
    out, lse = sa.sa_forward_combine(idx, d["sel"], d["q"], d["k"], d["v"], d["bt"], d["cu"],
                                     d["used"], w.hq, w.hkv, w.head_dim, w.block_size,
                                     w.page_size, w.softmax_scale, w.causal)
    _check_output(w, out, lse)
    o, m, l = sa.sa_forward(idx, d["q"], d["k"], d["v"], d["bt"], d["cu"], d["used"], w.hq,
                            w.hkv, w.head_dim, w.block_size, w.page_size, w.softmax_scale,
                            w.causal)
    out2, lse2 = sa.sa_combine(idx, o, m, l, w.hq, w.head_dim)
    assert max_rel_err(out.cpu().numpy(), out2.cpu().numpy())[0] <= 1e-5
    fin = torch.isfinite(lse2)
    assert torch.equal(fin, torch.isfinite(lse))
    if fin.any():
        assert (lse[fin] - lse2[fin]).abs().max().item() <= 1e-5
    if w.tq == w.batch:
        out3, lse3 = run_attention(w, d)              # sa_attention's own choice: fused
        assert torch.equal(out3, out) and torch.equal(lse3, lse)


def test_fused_rejects_geometry_outside_it():
    w = W.make_random(8850, batch=2, qo_max=1, kv_max=200, hkv=1, qhead=2, head_dim=64,
                      page_size=16, pages_per_block=2, topk=3)
    d = dev_inputs(w)
    idx = run_index(w, d)
    with pytest.raises(sa.SaError) as ei:
        sa.sa_forward_combine(idx, d["sel"], d["q"], d["k"], d["v"], d["bt"], d["cu"], d["used"],
                              w.hq, w.hkv, w.head_dim, w.block_size, w.page_size,
                              w.softmax_scale, w.causal)
    assert ei.value.kind == "Unsupported"
    with pytest.raises(sa.SaError) as ei:
        sa.sa_forward_combine(idx, d["sel"][:-1], d["q"], d["k"], d["v"], d["bt"], d["cu"],
                              d["used"], w.hq, w.hkv, w.head_dim, w.block_size, w.page_size,
                              w.softmax_scale, w.causal)
    assert (ei.value.kind, ei.value.what) == ("ShapeMismatch", "selected")


def test_tiny_workload():
    w = W.make_config("tiny")
    _print_case("tiny")
    d = dev_inputs(w)
    idx = run_index(w, d)
    ref = oracle_index(w)
    info, arrs = assert_index_equal(idx, ref)
    check_units(arrs, info, ref, idx.c.cap_edges, w)
    out, lse = run_attention(w, d)
    _check_output(w, out, lse)


@pytest.mark.parametrize("name", ["pages_small_fixture_index.json", "pages_gqa_fixture_index.json",
                                  "handmade_index.json"])
def test_golden_index_on_gpu(golden_dir, name, build_path):
    import json
    import os
    with open(os.path.join(golden_dir, name)) as f:
        g = json.load(f)
    inp = g["inputs"]
    tbl = np.asarray(inp["block_tables"], dtype=np.int32)
    tq, hkv, topk = inp["tq"], inp["hkv"], inp["topk"]
    idx = sa.sa_index_plan(tq, hkv, topk, tbl.shape[0], tbl.shape[1], inp["block_size"],
                           inp["page_size"], hkv, 4, inp["num_pages"])
    idx.allocate("cuda")
    t = lambda a, dt: torch.tensor(a, dtype=dt, device="cuda")
    used = None if inp.get("used_kv_lens") is None else t(inp["used_kv_lens"], torch.int32)
    sa.sa_build_index(t(inp["selected"], torch.int32), t(tbl, torch.int32),
                      t(inp["cu_seqlens_q"], torch.int64), used, idx)
    info = sa.sa_index_status(idx)
    arrs = sa.index_arrays(idx, info)
    for key in ("sel_slots", "sel_offsets", "num_sel", "edges", "edge_head_base", "inv"):
        np.testing.assert_array_equal(arrs[key].cpu().numpy(), np.asarray(g["expected"][key]),
                                      err_msg=key)


def test_determinism_bitwise():
    w = W.make_random(901, batch=3, qo_max=6, kv_max=64, hkv=2, qhead=4, head_dim=64, topk=4)
    d = dev_inputs(w)
    o1, l1 = run_attention(w, d)
    o2, l2 = run_attention(w, d)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ------------------------------------------------------------------ device errors

def _device_error(w, d, **over):
    dd = dict(d)
    dd.update(over)
    idx = run_index(w, dd)
    with pytest.raises(sa.SaError) as ei:
        sa.sa_index_status(idx)
    return ei.value


def _oracle_error(w, **over):
    import dataclasses
    w2 = dataclasses.replace(w, **over)
    with pytest.raises(oracle.SparseAttentionError) as ei:
        oracle_index(w2)
    return ei.value


def test_device_error_selected_out_of_range(build_path):
    w = W.make_random(31, batch=2, hkv=2, topk=3)
    msb = w.max_pages // (w.block_size // w.page_size)
    sel = w.selected.copy()
    sel.reshape(-1)[7] = msb + 5
    sel.reshape(-1)[4] = -3
    d = dev_inputs(w)
    got = _device_error(w, d, sel=torch.from_numpy(sel).cuda())
    ref = _oracle_error(w, selected=sel)
    assert got.kind == ref.kind == "SelectedOutOfRange"
    assert (got.got, got.expected) == (ref.got, ref.expected) == (-3, msb)


def test_device_error_cu_seqlens(build_path):
    w = W.make_random(32, batch=3, hkv=1, topk=2)
    d = dev_inputs(w)
    cu = w.cu_seqlens_q.copy()
    cu[1], cu[2] = cu[2] + 1, cu[1]               # decreasing pair
    got = _device_error(w, d, cu=torch.from_numpy(cu).cuda())
    assert got.kind == "CuSeqlensInvalid"
    cu = w.cu_seqlens_q.copy()
    cu[-1] = cu[-1] - 1 if cu[-1] > cu[-2] else cu[-1] + 1
    got = _device_error(w, d, cu=torch.from_numpy(cu).cuda())
    assert (got.kind, got.what, got.expected, got.got) == ("ShapeMismatch", "cu_seqlens_q total",
                                                           w.tq, int(cu[-1]))


def test_device_error_page_id(golden_dir, build_path):
    import json
    import os
    with open(os.path.join(golden_dir, "handmade_index.json")) as f:
        g = json.load(f)
    inp, case = g["inputs"], g["page_error_case"]
    tbl = np.asarray(inp["block_tables"], dtype=np.int32)
    idx = sa.sa_index_plan(inp["tq"], inp["hkv"], inp["topk"], tbl.shape[0], tbl.shape[1],
                           inp["block_size"], inp["page_size"], inp["hkv"], 4, case["num_pages"])
    idx.allocate("cuda")
    t = lambda a, dt: torch.tensor(a, dtype=dt, device="cuda")
    sa.sa_build_index(t(inp["selected"], torch.int32), t(tbl, torch.int32),
                      t(inp["cu_seqlens_q"], torch.int64), t(inp["used_kv_lens"], torch.int32), idx)
    with pytest.raises(sa.SaError) as ei:
        sa.sa_index_status(idx)
    e = ei.value
    assert (e.kind, e.what, e.expected, e.got) == (case["kind"], case["what"], case["expected"],
                                                   case["got"])


@pytest.mark.parametrize("head_dim", [32, 128])
def test_forward_skips_on_device_error(head_dim, build_path):
    """A build that finds an input error: sa_forward writes no partial,
    sa_combine fills out and lse with NaN, and sa_attention raises (or, with
    check=False, returns and leaves the status to sa_index_status)."""
    w = W.make_random(33, batch=2, hkv=1, topk=2, head_dim=head_dim)
    _print_case("device_error_outputs", d=head_dim, build=build_path)
    d = dev_inputs(w)
    sel = w.selected.copy()
    sel.reshape(-1)[0] = 10 ** 6
    d["sel"] = torch.from_numpy(sel).cuda()
    out = torch.full((w.tq, w.hq, w.head_dim), 7.0, device="cuda")
    lse = torch.full((w.tq, w.hq), 7.0, device="cuda")
    o, l_, idx = sa.sa_attention(d["q"], d["k"], d["v"], d["sel"], d["bt"], d["cu"], d["used"],
                                 w.block_size, w.softmax_scale, w.causal, out=out, lse=lse,
                                 return_index=True, check=False)
    with pytest.raises(sa.SaError) as ei:
        sa.sa_index_status(idx)
    assert ei.value.kind == "SelectedOutOfRange"
    assert torch.all(torch.isnan(out)) and torch.all(torch.isnan(lse))
    rows = idx.c.max_edges * (w.hq // w.hkv)
    o_p = torch.full((rows, w.head_dim), 5.0, device="cuda")
    m_p = torch.full((rows,), 5.0, device="cuda")
    l_p = torch.full((rows,), 5.0, device="cuda")
    sa.sa_forward(idx, d["q"], d["k"], d["v"], d["bt"], d["cu"], d["used"], w.hq, w.hkv,
                  w.head_dim, w.block_size, w.page_size, w.softmax_scale, w.causal, o_p, m_p, l_p)
    torch.cuda.synchronize()
    assert torch.all(o_p == 5.0) and torch.all(m_p == 5.0) and torch.all(l_p == 5.0)
    with pytest.raises(sa.SaError) as ei:
        sa.sa_attention(d["q"], d["k"], d["v"], d["sel"], d["bt"], d["cu"], d["used"],
                        w.block_size, w.softmax_scale, w.causal)
    assert ei.value.kind == "SelectedOutOfRange"


def test_rank_skipped_on_bad_cu_total(monkeypatch):
    """cu_seqlens_q whose total is below tq, on the multi-kernel build with a
    slot of 900 keys (the rank kernel's bitmap path): the status is the
    ShapeMismatch "cu_seqlens_q total", and the build writes inside its buffer
    only (a guard region after the index buffer stays untouched)."""
    monkeypatch.setenv("SA_BUILD_MULTIKERNEL", "1")
    batch, tq, topk, hkv, d = 2, 1000, 16, 1, 16
    ps, bs, max_pages = 16, 16, 64
    _print_case("rank_bad_cu_total", tq=tq, topk=topk)
    sel = torch.full((tq, hkv, topk), -1, dtype=torch.int32, device="cuda")
    sel[:, :, 0] = 0                                  # every query picks block 0
    bt = torch.arange(batch * max_pages, dtype=torch.int32, device="cuda").reshape(batch, max_pages)
    cu = torch.tensor([0, 100, 200], dtype=torch.int64, device="cuda")
    idx = sa.sa_index_plan(tq, hkv, topk, batch, max_pages, bs, ps, hkv, d, batch * max_pages)
    raw = torch.full((idx.c.index_bytes + 256 + 4096,), 0xAB, dtype=torch.uint8, device="cuda")
    off = (-raw.data_ptr()) % 256
    idx.buffer = raw[off:off + idx.c.index_bytes]
    idx.c.buffer = idx.buffer.data_ptr()
    sa.sa_build_index(sel, bt, cu, None, idx)
    with pytest.raises(sa.SaError) as ei:
        sa.sa_index_status(idx)
    e = ei.value
    assert (e.kind, e.what, e.expected, e.got) == ("ShapeMismatch", "cu_seqlens_q total", tq, 200)
    guard = raw[off + idx.c.index_bytes:]
    assert torch.all(guard == 0xAB)


# ------------------------------------------------------------------ empty inputs

@pytest.mark.parametrize("head_dim", [128, 32])
@pytest.mark.parametrize("table", ["full", "empty", "short"])
def test_nothing_selected(head_dim, table, build_path):
    """Every rank padded, with the block table as drawn, with no columns at
    all (max_pages = 0) and with fewer pages than one block (msb = 0): an
    empty index, O = 0 and lse = -inf, on the one-wave (d = 128) and the
    wavefront (d = 32) kernels."""
    w = W.make_random(5100, batch=2, qo_max=3, kv_max=80, hkv=2, qhead=2, head_dim=head_dim,
                      page_size=16, pages_per_block=2, topk=3)
    w.selected[...] = -1
    if table != "full":
        cols = 0 if table == "empty" else 1
        w.block_tables = np.ascontiguousarray(w.block_tables[:, :cols])
    _print_case("nothing_selected", d=head_dim, table=table, build=build_path)
    d = dev_inputs(w)
    idx = run_index(w, d)
    ref = oracle_index(w)
    info, _ = assert_index_equal(idx, ref)
    assert info["total_edges"] == 0
    out, lse = run_attention(w, d)
    assert torch.all(out == 0.0)
    assert torch.all(lse == -float("inf"))


# ------------------------------------------------------------------ full-size workloads

def _sample_queries(w, n, seed=0):
    rng = np.random.default_rng(seed)
    cu = w.cu_seqlens_q
    picks = set()
    for b in range(w.batch):
        if cu[b + 1] > cu[b]:
            picks.update({int(cu[b]), int(cu[b + 1] - 1)})
    picks.update(rng.choice(w.tq, size=min(n, w.tq), replace=False).tolist())
    return np.asarray(sorted(picks))


@pytest.mark.parametrize("name,n_sample", [("decode", None), ("ragged", 128),
                                           ("prefill", 128), ("skewed", 128)])
def test_full_size_workload(name, n_sample):
    """A full-size workload in the launch configuration the benchmark times:
    the index in full; the partials of sampled edges (the hottest and the
    smallest slot of each head, unit boundaries, random edges) against the
    oracle; the output on every query (decode) or on n_sample random queries
    plus the first and last query of each sequence, the oracle's rows computed
    in parallel worker processes."""
    _print_case("full_size", name=name)
    w = W.make_config(name)
    d = dev_inputs(w)
    idx = run_index(w, d)
    ref = oracle_index(w)
    info, arrs = assert_index_equal(idx, ref)
    check_units(arrs, info, ref, idx.c.cap_edges, w)
    edges = sample_edges(ref, arrs, info)
    perr = check_partials(w, d, idx, ref, only_edges=edges)
    print(f"[gpu case] {name}: partials of {len(edges)} edges: {perr}", flush=True)
    out, lse = run_attention(w, d)
    torch.cuda.synchronize()
    if w.tq == w.batch:
        # sa_attention took the fused forward + combine: the two-pass path agrees
        o, m, l = sa.sa_forward(idx, d["q"], d["k"], d["v"], d["bt"], d["cu"], d["used"], w.hq,
                                w.hkv, w.head_dim, w.block_size, w.page_size, w.softmax_scale,
                                w.causal)
        out2, _ = sa.sa_combine(idx, o, m, l, w.hq, w.head_dim)
        assert max_rel_err(out.cpu().numpy(), out2.cpu().numpy())[0] <= 1e-5
    queries = None if n_sample is None else _sample_queries(w, n_sample)
    err = _check_output(w, out, lse, queries, parallel=True)
    print(f"[gpu case] {name}: O rel err {err:.3e} over "
          f"{w.tq if queries is None else len(queries)} queries", flush=True)


# The one-kernel build at the edges of its own paths: the batch-of-query
# scan done by one wave (up to 256 queries) or by the workgroup (more), entry
# counts that straddle a wave's share of entries (1024 a slot), the slot scan
# of four slots a thread (4096 slots) against the general one (4095 and
# 5000), and many heads for the look-back. Built with and without the
# one-kernel path; index bit-exact, output against the oracle.
def _fused_case(seed, qo, batch, topk, msb, hkv, ps=4, ppb=2, qhead=2, d=16):
    rng = np.random.Generator(np.random.PCG64(seed))
    bs = ps * ppb
    max_pages = msb * ppb
    qo_b = np.full(batch, qo // batch, dtype=np.int64)
    qo_b[: qo % batch] += 1
    cu = np.concatenate([[0], np.cumsum(qo_b)]).astype(np.int64)
    tq = int(cu[-1])
    kv = rng.integers(bs, msb * bs + 1, size=batch)
    pages = [int(math.ceil(k / ps)) for k in kv]
    num_pages = int(sum(pages)) + 3
    perm = rng.permutation(num_pages)
    tbl = np.full((batch, max_pages), -1, dtype=np.int32)
    o = 0
    for b in range(batch):
        tbl[b, : pages[b]] = perm[o:o + pages[b]]
        o += pages[b]
    sel = np.full((tq, hkv, topk), -1, dtype=np.int32)
    for q in range(tq):
        b = int(np.searchsorted(cu, q, side="right") - 1)
        hi = max(1, int(math.ceil(kv[b] / bs)))
        for h in range(hkv):
            k = min(topk, hi)
            ids = rng.choice(hi, size=k, replace=False)
            row = np.full(topk, -1, dtype=np.int64)
            row[:k] = ids
            row[rng.random(topk) < 0.2] = -1
            sel[q, h] = rng.permutation(row)
    hq = hkv * qhead
    return W.Workload("fused_edge", rng.standard_normal((tq, hq, d), dtype=np.float32),
                      rng.standard_normal((num_pages, hkv, ps, d), dtype=np.float32),
                      rng.standard_normal((num_pages, hkv, ps, d), dtype=np.float32),
                      sel, tbl, cu, None, hq, hkv, d, bs, ps, topk, 1.0 / math.sqrt(d),
                      bool(seed % 2))


FUSED_EDGE = [
    # (qo, batch, topk, msb, hkv)
    (256, 4, 4, 1024, 1),    # 256 queries: one-wave scan; 4096 slots: four a thread
    (257, 5, 4, 819, 2),     # 257 queries: workgroup scan; 4095 slots
    (300, 3, 8, 1000, 1),    # 2400 entries; 3000 slots
    (1025, 7, 1, 600, 3),    # 1025 entries: a wave's share crosses 1024
    (683, 2, 6, 2500, 1),    # 4098 entries: past the one-kernel build's capacity
    (512, 8, 8, 625, 1),     # 4096 entries, 5000 slots: five slots a thread
    (32, 32, 16, 128, 40),   # 40 heads: the look-back folds 39 heads' totals
]


@pytest.mark.parametrize("case", range(len(FUSED_EDGE)))
def test_fused_build_edges(case, build_path):
    qo, batch, topk, msb, hkv = FUSED_EDGE[case]
    w = _fused_case(9000 + case, qo, batch, topk, msb, hkv)
    _print_case("fused_build_edges", idx=case, tq=w.tq, topk=topk, nbs=batch * msb, hkv=hkv,
                path=build_path)
    d_in = dev_inputs(w)
    idx = run_index(w, d_in)
    ref = oracle_index(w)
    info, arrs = assert_index_equal(idx, ref)
    check_units(arrs, info, ref, idx.c.cap_edges, w)
    out, lse = run_attention(w, d_in)
    _check_output(w, out, lse)


# The multi-kernel build's histogram and scatter count a chunk of 4096
# entries in LDS when one sequence's hkv*msb counters fit (8192 at most) and
# slots repeat, and take one global atomic an entry otherwise; SA_BUILD_AGG
# forces either kernel pair where the counters fit. Cases at that limit and
# past it, with hot slots (a few blocks shared by thousands of queries), and
# with chunks that span hundreds of short sequences (entries outside the
# chunk's first sequence take the global atomic). The last two reach the rank
# kernel's LDS bitmap over one sequence's keys and, past its 131072 keys, the
# pairwise ranks. Index bit-exact, output against the oracle.
AGG_EDGE = [
    # (qo, batch, topk, msb, hkv)
    (600, 2, 16, 4096, 2),   # 8192 counters: the LDS path; a chunk crosses sequences
    (600, 2, 16, 4097, 2),   # 8194 counters: one global atomic an entry
    (2000, 1, 8, 16, 2),     # 16 blocks for 2000 queries: ~1000 edges a slot
    (3000, 600, 2, 8, 1),    # 5-query sequences: ~400 of them in a chunk
    (4000, 4, 8, 16, 2),     # hot slots in 4 sequences: rank bitmaps over each one's keys
    (2100, 1, 64, 80, 1),    # 134400 keys in one sequence: past the rank bitmap (pairwise)
    (200, 2, 2, 8, 70),      # 70 heads: the multi-kernel build's per-head totals and look-backs
]


@pytest.mark.parametrize("agg", ["1", "0"])
@pytest.mark.parametrize("case", range(len(AGG_EDGE)))
def test_multikernel_build_aggregation(case, agg, monkeypatch):
    monkeypatch.setenv("SA_BUILD_MULTIKERNEL", "1")
    monkeypatch.setenv("SA_BUILD_AGG", agg)
    qo, batch, topk, msb, hkv = AGG_EDGE[case]
    w = _fused_case(9100 + case, qo, batch, topk, msb, hkv)
    _print_case("multikernel_build_aggregation", idx=case, tq=w.tq, topk=topk, nbs=batch * msb,
                hkv=hkv, agg=agg)
    d_in = dev_inputs(w)
    idx = run_index(w, d_in)
    ref = oracle_index(w)
    info, arrs = assert_index_equal(idx, ref)
    check_units(arrs, info, ref, idx.c.cap_edges, w)
    out, lse = run_attention(w, d_in)
    _check_output(w, out, lse)


# ------------------------------------------------------------------ decode-shaped builds
# Every sequence holds one query (cu[b] = b), as in decode batches: padding,
# repeated picks in a row (several edges in one slot), blocks past the used
# length, empty rows, one pick a row, 33 picks, 1024 rows, slots large enough
# for MFMA units, and a batch with tq == batch whose cu is not of that form.
# Index bit-exact, units checked, output against the oracle; both build paths.

def _decode_case(seed, batch, hkv, topk, msb, ppb=4, ps=4, qhead=2, d=16, dup=0.1, pad=0.2,
                 short=0.0, cu=None):
    rng = np.random.Generator(np.random.PCG64(seed))
    bs = ps * ppb
    max_pages = msb * ppb
    if cu is None:
        cu = np.arange(batch + 1, dtype=np.int64)
    tq = int(cu[-1])
    kv = rng.integers(1, msb * bs + 1, size=batch)
    used = np.where(rng.random(batch) < short, rng.integers(0, bs, size=batch), kv).astype(np.int32)
    pages = [int(math.ceil(k / ps)) for k in kv]
    num_pages = int(sum(pages)) + 2
    perm = rng.permutation(num_pages)
    tbl = np.full((batch, max_pages), -1, dtype=np.int32)
    o = 0
    for b in range(batch):
        tbl[b, : pages[b]] = perm[o:o + pages[b]]
        o += pages[b]
    sel = np.full((tq, hkv, topk), -1, dtype=np.int32)
    for q in range(tq):
        b = int(np.searchsorted(cu, q, side="right") - 1)
        hi = max(1, int(math.ceil(kv[b] / bs)))
        for h in range(hkv):
            k = min(topk, hi)
            row = np.full(topk, -1, dtype=np.int64)
            row[:k] = rng.choice(hi, size=k, replace=False)
            row = rng.permutation(row)
            if topk > 1 and dup > 0:
                dups = rng.random(topk) < dup
                row[dups] = row[0]
            row[rng.random(topk) < pad] = -1
            sel[q, h] = row
    hq = hkv * qhead
    return W.Workload("decode_edge", rng.standard_normal((tq, hq, d), dtype=np.float32),
                      rng.standard_normal((num_pages, hkv, ps, d), dtype=np.float32),
                      rng.standard_normal((num_pages, hkv, ps, d), dtype=np.float32),
                      sel, tbl, cu, used, hq, hkv, d, bs, ps, topk, 1.0 / math.sqrt(d),
                      bool(seed % 2))


DECODE_EDGE = [
    # (batch, hkv, topk, msb, ppb, ps, qhead, d, dup, pad, short)
    (32, 8, 16, 128, 4, 16, 4, 128, 0.1, 0.1, 0.1),   # the decode shape, kv shortened
    (7, 3, 5, 20, 2, 4, 2, 16, 0.3, 0.3, 0.2),        # 8 lanes a row
    (1, 1, 1, 3, 1, 4, 1, 8, 0.0, 0.0, 0.0),          # one pick
    (16, 4, 33, 40, 1, 8, 2, 16, 0.2, 0.2, 0.1),      # 64 lanes a row
    (64, 16, 4, 50, 2, 4, 2, 16, 0.2, 0.3, 0.3),      # 1024 rows
    (40, 2, 16, 30, 4, 4, 2, 16, 0.0, 0.5, 0.6),      # many blocks past lk, empty rows
    (24, 2, 8, 12, 4, 32, 16, 128, 0.5, 0.1, 0.0),    # 128-key blocks, duplicates: MFMA units
]


@pytest.mark.parametrize("case", range(len(DECODE_EDGE)))
def test_decode_shaped_build(case, build_path):
    batch, hkv, topk, msb, ppb, ps, qhead, d, dup, pad, short = DECODE_EDGE[case]
    w = _decode_case(9500 + case, batch, hkv, topk, msb, ppb, ps, qhead, d, dup, pad, short)
    _print_case("decode_shaped_build", idx=case, tq=w.tq, hkv=hkv, topk=topk, path=build_path)
    d_in = dev_inputs(w)
    idx = run_index(w, d_in)
    ref = oracle_index(w)
    info, arrs = assert_index_equal(idx, ref)
    check_units(arrs, info, ref, idx.c.cap_edges, w)
    # the output: the query-outer oracle attends over the union of a row's
    # blocks and so takes rows without repeated picks (the same draw, dup=0)
    w = _decode_case(9500 + case, batch, hkv, topk, msb, ppb, ps, qhead, d, 0.0, pad, short)
    out, lse = run_attention(w, dev_inputs(w))
    _check_output(w, out, lse)


def test_decode_shaped_build_falls_back_on_other_cu(build_path):
    # tq == batch, but one empty sequence and one with two queries
    cu = np.array([0, 1, 1, 3, 4, 5, 6, 7, 8], dtype=np.int64)
    w = _decode_case(9600, 8, 2, 6, 10, 2, 4, 2, 16, 0.2, 0.2, 0.0, cu=cu)
    _print_case("decode_shaped_fallback", tq=w.tq, path=build_path)
    d_in = dev_inputs(w)
    idx = run_index(w, d_in)
    ref = oracle_index(w)
    info, arrs = assert_index_equal(idx, ref)
    check_units(arrs, info, ref, idx.c.cap_edges, w)


@pytest.mark.parametrize("where", ["first", "last", "both"])
def test_decode_shaped_build_errors(where, build_path):
    w = _decode_case(9700, 12, 3, 8, 16, 4, 4, 2, 16, 0.1, 0.1, 0.0)
    msb = w.max_pages // (w.block_size // w.page_size)
    d = dev_inputs(w)
    _print_case("decode_shaped_errors", where=where, path=build_path)
    sel = w.selected.copy()
    flat = sel.reshape(-1)
    if where in ("first", "both"):
        flat[5] = msb
    if where in ("last", "both"):
        flat[-3] = -7
    got = _device_error(w, d, sel=torch.from_numpy(sel).cuda())
    ref = _oracle_error(w, selected=sel)
    assert (got.kind, got.expected, got.got) == (ref.kind, ref.expected, ref.got)
    # a page id past the pool in a touched page of a kept block (a later
    # head's entry, so that the last head's check must see it)
    tbl = w.block_tables.copy()
    q, h, r = 7, 2, int(np.nonzero(w.selected[7, 2] >= 0)[0][0])
    v = int(w.selected[q, h, r])
    ppb = w.block_size // w.page_size
    tbl[q, v * ppb] = w.k_pages.shape[0] + 5
    got = _device_error(w, d, bt=torch.from_numpy(tbl).cuda())
    ref = _oracle_error(w, block_tables=tbl)
    assert (got.kind, got.what, got.expected, got.got) == (ref.kind, ref.what, ref.expected, ref.got)
