#!/usr/bin/env python3
"""Benchmark of the KV-outer block-sparse paged attention hot path on one MI355X.

A step is one pass of the whole path over one batch: index build (histogram,
scan, scatter, rank, work units) -> KV-outer forward -> LSE combine. Inputs
are resident in HBM before the timed region. Steps rotate over ``--rotate``
independent selections and page tables that share one K/V cache. A step
therefore does not find its blocks in the 256 MB Infinity Cache from the
step before.

Prints ONE JSON line. ``value`` is kept edges per second of whole steps.
``roofline`` is for the forward pass (sa_forward), the dominant part of a
step. Its average duration is measured with HIP events recorded on the
stream it is launched on, right after the timed region: one event pair
around K back-to-back forward launches over the same rotated batches (an
event marker between kernels costs the GPU a few microseconds, so none sits
inside the timed region or between the launches timed); its algorithmic
bytes and flops are counted from the built index. For the MFMA-bound
workloads ``roofline.mfma_util`` is the matrix pipes' busy fraction that
rocprofv3 measured for the same kernel (profiles/<workload>_forward_mfma_util.md),
null once that kernel's sources have changed. ``cpu_baseline`` is the CPU
oracle timed on this host.

    python bench.py [--steps K] [--warmup W] [--config decode|tiny|prefill|ragged|skewed]
    python bench.py --copy-calibration   # plain copy kernel of known size, for PMC scaling
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "selected-block attention edges/s + effective TFLOP/s and HBM GB/s % of peak"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
FP32_MFMA_PEAK_TFLOPS = 157.3   # MI355X dense fp32 matrix
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 matrix
DEFAULT_CONFIG = "skewed"      # the largest workload that fits one GPU: skewed long-context


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default=DEFAULT_CONFIG,
                   choices=["tiny", "decode", "prefill", "ragged", "skewed",
                            "prefill_d64", "prefill_d256", "prefill_bs256"],
                   help="one of the five workloads, or the prefill recipe at head_dim 64 / 256 "
                        "or with 256-key blocks (the chunked MFMA kernel's geometries)")
    p.add_argument("--rotate", type=int, default=4, help="independent input batches cycled")
    p.add_argument("--kv-dtype", default="f32", choices=["f32", "bf16", "fp16"],
                   help="storage of the K/V pages (16-bit: sa_forward_kv16, or "
                        "sa_forward_combine_kv16 for decode-shaped batches)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target wall time of the oracle leg (all its worker processes)")
    p.add_argument("--copy-calibration", action="store_true")
    p.add_argument("--graph", action="store_true",
                   help="also time the step replayed from a captured HIP graph")
    p.add_argument("--two-pass", action="store_true",
                   help="decode-shaped batches: sa_forward + sa_combine instead of the fused "
                        "sa_forward_combine that sa_attention takes")
    return p.parse_args()


def copy_calibration():
    """A plain device copy of a known size (1 GiB read + 1 GiB written),
    for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = 1 << 28                                   # 2^28 floats = 1 GiB
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": 4 * n, "launches": 5}), flush=True)


def variants(name, rotate):
    """The base workload with K/V, plus rotate-1 more selections/page tables
    drawn with other seeds. They share one K/V cache, padded with seeded
    N(0,1) pages when a variant addresses more pages than the base."""
    import workloads as W
    base = W.make_config(name)
    out = [base]
    for r in range(1, rotate):
        out.append(W.make_config(name, seed=W.CONFIG_SEEDS[name] + 1000 * r, with_kv=False))
    pages = max(v.num_pages for v in out)
    k, v = base.k_pages, base.v_pages
    if pages > base.num_pages:
        rng = np.random.Generator(np.random.PCG64(W.CONFIG_SEEDS[name] + 99))
        extra = (pages - base.num_pages,) + k.shape[1:]
        k = np.concatenate([k, rng.standard_normal(extra, dtype=np.float32)])
        v = np.concatenate([v, rng.standard_normal(extra, dtype=np.float32)])
    return base, out, k, v


def algorithmic_work(w, arrs, info, kv_elem_bytes=4):
    """Bytes and flops the method must move/do for this batch, from the index.

    forward: K and V rows of every selected block once (valid positions with a
    page), Q once, partials (o, m, l) written.  combine: partials read once,
    inv read, O (and lse) written.  Flops: 4*d per (row, valid key)."""
    ppb = w.block_size // w.page_size
    msb = w.max_pages // ppb
    d = w.head_dim
    qhead = w.hq // w.hkv
    num_sel = arrs["num_sel"]
    offs = arrs["sel_offsets"]
    slots = arrs["sel_slots"]
    lk = (np.full(w.batch, msb * w.block_size, dtype=np.int64) if w.used_kv_lens is None
          else np.maximum(w.used_kv_lens.astype(np.int64), 0))
    kv_bytes = 0
    flops = 0
    for h in range(w.hkv):
        n = int(num_sel[h])
        raw = slots[h, :n].astype(np.int64)
        b, blk = raw // msb, raw % msb
        start = blk * w.block_size
        end = np.minimum(start + w.block_size, lk[b])
        # valid positions: inside [start, end) and on a page >= 0
        valid = np.zeros(n, dtype=np.int64)
        for pl in range(ppb):
            p0 = start + pl * w.page_size
            p1 = np.minimum(p0 + w.page_size, end)
            page = w.block_tables[b, blk * ppb + pl]
            valid += np.where((p1 > p0) & (page >= 0), p1 - p0, 0)
        edges_per_slot = np.diff(offs[h, :n + 1]).astype(np.int64)
        kv_bytes += int(2 * valid.sum() * d * kv_elem_bytes)
        flops += int((edges_per_slot * valid).sum() * qhead * 4 * d)
    E = info["total_edges"]
    rows = E * qhead
    q_bytes = w.tq * w.hq * d * 4
    part_bytes = rows * (d + 2) * 4
    meta_fwd = info["num_units_wave"] * 16 + info["num_units_mfma"] * 16 + E * 8
    fwd_bytes = kv_bytes + q_bytes + part_bytes + meta_fwd
    out_bytes = w.tq * w.hq * (d + 1) * 4
    comb_bytes = part_bytes + w.tq * w.hkv * w.topk * 4 + out_bytes
    # the fused forward + combine: K/V once, q once, inv and selected once, O and lse
    fused_bytes = kv_bytes + q_bytes + 2 * w.tq * w.hkv * w.topk * 4 + out_bytes
    return {"kv_bytes": kv_bytes, "fwd_bytes": fwd_bytes, "comb_bytes": comb_bytes,
            "total_bytes": fwd_bytes + comb_bytes, "fused_bytes": fused_bytes, "flops": flops,
            "edges": E, "rows": rows}


def cpu_workers():
    """Host cores for the oracle leg: the CPUs this process may run on, at
    most 16 (a one-GPU machine's share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


_CPU_W = None


def _cpu_init():
    from threadpoolctl import threadpool_limits
    global _CPU_LIMIT
    _CPU_LIMIT = threadpool_limits(limits=1)        # one BLAS thread per worker


def _cpu_chunk(queries):
    import oracle
    w = _CPU_W
    oracle.attention_qo_ref(w.q, w.k_pages, w.v_pages, w.selected, w.block_tables,
                            w.cu_seqlens_q, w.used_kv_lens, w.hq, w.hkv, w.head_dim,
                            w.block_size, w.page_size, w.softmax_scale, w.causal,
                            queries=queries)
    return len(queries)


def cpu_baseline(w, target_s, workers):
    """The oracle (index build + query-outer attention, float64 NumPy, as it
    stands) on the host: the attention over chunks of queries of this batch in
    `workers` forked processes with one BLAS thread each, in rounds of one
    chunk a worker, until ~target_s seconds of wall time; the index build is
    timed once and charged pro rata to the queries done."""
    import multiprocessing as mp
    import oracle
    from threadpoolctl import threadpool_limits
    global _CPU_W
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        idx = oracle.build_index_ref(w.selected, w.tq, w.hkv, w.topk, w.block_tables, w.batch,
                                     w.max_pages, w.cu_seqlens_q, w.used_kv_lens,
                                     w.block_size, w.page_size, w.num_pages)
        t_index = time.perf_counter() - t0
    kept = (idx["inv"] >= 0).sum(axis=(0, 2))          # kept edges per query
    chunk = max(1, min(32, w.tq // workers))
    order = np.random.default_rng(0).permutation(w.tq)
    _CPU_W = w
    done_q, edges_done = 0, 0
    with mp.get_context("fork").Pool(workers, initializer=_cpu_init) as pool:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < target_s:
            parts = []
            for _ in range(workers):
                at = (done_q + sum(len(p) for p in parts)) % w.tq
                parts.append(order[at:at + chunk] if at + chunk <= w.tq
                             else np.concatenate([order[at:], order[:at + chunk - w.tq]]))
            pool.map(_cpu_chunk, parts)
            for p in parts:
                done_q += len(p)
                edges_done += int(kept[p].sum())
        t_attn = time.perf_counter() - t0
    _CPU_W = None
    frac = done_q / w.tq
    secs = t_attn + t_index * frac                     # index build charged pro rata
    return {"value": edges_done / secs, "unit": "edges/s", "cores": workers,
            "blas_threads_per_core": 1, "kind": "oracle",
            "sample": f"{done_q} query rows ({frac:.2f} passes over the {w.tq} queries of "
                      f"the {w.name} batch, {edges_done} edges) in chunks of {chunk} over "
                      f"{workers} worker processes; index build ({t_index:.2f} s, one core) "
                      f"charged pro rata; float64 NumPy",
            "seconds": round(secs, 3)}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library runs on one GPU and has no "
              "multi-GPU path (no sharding, no collectives).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    base, vs, k_all, v_all = variants(args.config, max(1, args.rotate))
    # the oracle leg first: its worker processes fork before this process
    # touches the GPU
    cpu = None if args.no_cpu_baseline else cpu_baseline(base, args.cpu_seconds, cpu_workers())

    import torch
    import block_sparse_paged_csr_amd as sa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(device=dev, dtype=dt)
    k = t(k_all, torch.float32)
    v = t(v_all, torch.float32)
    kv16 = args.kv_dtype != "f32"
    if kv16:
        # 16-bit storage of the same draws (round to nearest even)
        dt16 = torch.bfloat16 if args.kv_dtype == "bf16" else torch.float16
        k, v = k.to(dt16), v.to(dt16)
        torch.cuda.empty_cache()
    num_pages = int(k_all.shape[0])
    del k_all, v_all
    sets = []
    for w in vs:
        idx = sa.sa_index_plan(w.tq, w.hkv, w.topk, w.batch, w.max_pages, w.block_size,
                               w.page_size, w.hq, w.head_dim, num_pages).allocate(dev)
        rows = idx.c.max_edges * (w.hq // w.hkv)
        sets.append({
            "w": w, "idx": idx,
            "q": t(w.q, torch.float32), "sel": t(w.selected, torch.int32),
            "bt": t(w.block_tables, torch.int32), "cu": t(w.cu_seqlens_q, torch.int64),
            "used": None if w.used_kv_lens is None else t(w.used_kv_lens, torch.int32),
            "o": torch.empty((rows, w.head_dim), dtype=torch.float32, device=dev),
            "m": torch.empty(rows, dtype=torch.float32, device=dev),
            "l": torch.empty(rows, dtype=torch.float32, device=dev),
            "out": torch.empty((w.tq, w.hq, w.head_dim), dtype=torch.float32, device=dev),
            "lse": torch.empty((w.tq, w.hq), dtype=torch.float32, device=dev),
        })

    def build(s):
        sa.sa_build_index(s["sel"], s["bt"], s["cu"], s["used"], s["idx"])

    def forward(s):
        w = s["w"]
        fwd = sa.sa_forward_kv16 if kv16 else sa.sa_forward
        fwd(s["idx"], s["q"], k, v, s["bt"], s["cu"], s["used"], w.hq, w.hkv, w.head_dim,
            w.block_size, w.page_size, w.softmax_scale, w.causal, s["o"], s["m"], s["l"])

    def combine(s):
        w = s["w"]
        sa.sa_combine(s["idx"], s["o"], s["m"], s["l"], w.hq, w.head_dim, s["out"], s["lse"])

    fused = (not args.two_pass and base.tq == base.batch and
             sa.fused_fits(base.hq, base.hkv, base.head_dim, base.block_size, base.page_size,
                           base.topk))

    def forward_combine(s):
        w = s["w"]
        fc = sa.sa_forward_combine_kv16 if kv16 else sa.sa_forward_combine
        fc(s["idx"], s["sel"], s["q"], k, v, s["bt"], s["cu"], s["used"], w.hq, w.hkv,
           w.head_dim, w.block_size, w.page_size, w.softmax_scale, w.causal, s["out"], s["lse"])

    def step(s):
        # what sa_attention runs: the build, then the fused forward + combine for
        # decode-shaped batches, else the forward and the combine
        build(s)
        if fused:
            forward_combine(s)
        else:
            forward(s)
            combine(s)

    # algorithmic work of each batch, counted from the built index
    work = []
    for s in sets:
        step(s)
        info = sa.sa_index_status(s["idx"])
        arrs = {kk: vv.cpu().numpy() for kk, vv in sa.index_arrays(s["idx"], info).items()}
        work.append(algorithmic_work(s["w"], arrs, info, 2 if kv16 else 4))

    for i in range(args.warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()

    # the timed region: K whole steps, nothing else on the stream
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for s in sets:                                  # device-side status of the last builds
        sa.sa_index_status(s["idx"])

    # per-call durations: one pair of HIP events on the launch stream around
    # K back-to-back launches of each call over the same rotated batches (a
    # timing marker between two kernels costs the GPU a few microseconds, so
    # none sits inside the timed region above or between the launches timed).
    # A spin kernel ahead of the first event keeps the GPU busy while the host
    # enqueues all K launches, so the pair times the GPU, not the host's launch
    # rate; the lead is doubled until the first event is still pending when
    # the last launch has been enqueued.
    def phase_ms(fn):
        lead_us = 40.0 * args.steps
        for _ in range(4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(int(lead_us * 2500))      # clock64 ticks, >= 1 per ns here
            e0.record()
            for i in range(args.steps):
                fn(sets[i % len(sets)])
            queued_ahead = not e0.query()
            e1.record()
            torch.cuda.synchronize()
            if queued_ahead:
                break
            lead_us *= 2
        return e0.elapsed_time(e1) / args.steps, queued_ahead

    if fused:
        (build_ms, ok_b), (fwd_ms, ok_f) = map(phase_ms, (build, forward_combine))
        comb_ms, ok_c = 0.0, True
    else:
        (build_ms, ok_b), (fwd_ms, ok_f), (comb_ms, ok_c) = map(phase_ms, (build, forward, combine))
    per = [work[i % len(sets)] for i in range(args.steps)]
    edges = sum(p["edges"] for p in per)
    fwd_bytes = np.mean([p["fwd_bytes"] for p in per])
    fwd_avg_s = fwd_ms / 1e3
    step_s = wall / args.steps
    total_bytes = np.mean([p["fused_bytes" if fused else "total_bytes"] for p in per])
    flops = np.mean([p["flops"] for p in per])
    fc_s = (fwd_ms + comb_ms) / 1e3
    if fused:
        fwd_bytes = total_bytes
    roofline = forward_roofline(base, fwd_bytes, flops, fwd_avg_s, args.kv_dtype, fused)

    result = {
        "metric": METRIC,
        "value": edges / wall,
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the matrix operands' type: fp32, or the pages' 16-bit format (q and
        # the probabilities as sums of its terms, fp32 accumulation)
        "dtype": "f32" if args.kv_dtype == "f32" else args.kv_dtype,
        "data": "synthetic",
        "config": {**base.describe(), "kv_dtype": args.kv_dtype,
                   "edges_per_batch": int(np.mean([p["edges"] for p in per])),
                   "rotated_batches": len(sets), "parallelism": "single-gpu"},
        "roofline": roofline,
        "forward_plus_combine": {
            "us": fc_s * 1e6,
            "edges_per_s": edges / args.steps / fc_s,
            "tflops": flops / fc_s / 1e12,
            "hbm_gbps": total_bytes / fc_s / 1e9,
            "hbm_frac": total_bytes / fc_s / 1e9 / HBM_PEAK_GBPS,
            "mfma_frac_fp32": flops / fc_s / 1e12 / FP32_MFMA_PEAK_TFLOPS,
        },
        "index_build_us": build_ms * 1e3,
        "per_call_gpu_bound": bool(ok_b and ok_f and ok_c),
        "combine_us": comb_ms * 1e3,
        "fused_forward_combine": bool(fused),
    }
    if args.graph:
        result["graph_step_us"] = graph_step_us(sets, step, args.steps)
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


def forward_kernels(w, fused=False, kv_dtype="f32"):
    """The kernels one sa_forward launches for this geometry: the one-wave
    kernel alone where it fits (head_dim 128, blocks <= 64 keys, qhead <= 16),
    else the wavefront-reduction kernel and an MFMA kernel (16-row tiles for
    head_dim 128 and blocks <= 64 keys; 32-row tiles with direct-to-LDS
    gathers for fp32 pages and blocks of 65..128 keys, with register gathers
    for 16-bit pages; the chunked kernel for head_dim 64 / 256 and larger
    blocks); with `fused`, the one kernel of sa_forward_combine."""
    qhead = w.hq // w.hkv
    nch = (w.block_size + 15) // 16
    if fused:
        return f"k_fwd_fused<{nch}>", None
    if w.head_dim == 128 and w.block_size <= 64 and qhead <= 16:
        return f"k_fwd_small<{nch}>", None
    if w.head_dim == 128 and w.block_size <= 64:
        return "k_fwd_wave", "k_fwd_mfma16"
    if w.head_dim == 128 and w.block_size <= 128:
        return "k_fwd_wave", "k_fwd_mfma_dma"
    if w.head_dim in (64, 128, 256):
        return "k_fwd_wave", "k_fwd_mfma_gen"
    return "k_fwd_wave", None


def forward_roofline(w, fwd_bytes, fwd_flops, fwd_s, kv_dtype="f32", fused=False):
    """Roofline of the forward pass (sa_forward: the one-wave kernel where
    it fits, else the wavefront kernel for units under 32 rows, then the MFMA
    kernel, which exits at once when the build made no such unit). Bound by HBM when the algorithmic intensity is
    below the fp32 MFMA ridge (157.3 TFLOP/s / 8 TB/s = 19.7 flop/B), else by
    fp32 MFMA. `traffic` comes from the committed FETCH_SIZE + WRITE_SIZE
    summary for this workload, and only while the kernel's source is the one
    the counters were taken on."""
    small, mfma = forward_kernels(w, fused, kv_dtype)
    if kv_dtype != "f32":
        small = small.replace(">", f", {kv_dtype}>")
    # 16-bit pages run their main tiles on the 16-bit matrix pipes (bf16 and
    # fp16 share one dense peak): that peak (and ridge), against the
    # algorithmic flops
    mfma_peak = BF16_MFMA_PEAK_TFLOPS if kv_dtype in ("bf16", "fp16") else FP32_MFMA_PEAK_TFLOPS
    ridge = mfma_peak * 1e12 / (HBM_PEAK_GBPS * 1e9)
    if fwd_flops / fwd_bytes < ridge:
        achieved, peak, unit, bound = fwd_bytes / fwd_s / 1e9, HBM_PEAK_GBPS, "GB/s", "hbm"
        kernels = small if mfma is None else f"{small} + {mfma}"
        # where an MFMA kernel runs, it takes nearly all of the forward's time
        dominant = small if mfma is None else mfma
    else:
        achieved, peak, unit, bound = fwd_flops / fwd_s / 1e12, mfma_peak, "TFLOP/s", "mfma"
        kernels = small if mfma is None else f"{mfma} + {small}"
        dominant = small if mfma is None else mfma
    return {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
            "frac": achieved / peak,
            "traffic": measured_traffic(w.name if kv_dtype == "f32" else f"{w.name}_{kv_dtype}",
                                        dominant),
            "mfma_util": measured_mfma_util(w.name) if bound == "mfma" and kv_dtype == "f32" else None,
            "kernel": f"{'sa_forward_combine' if fused else 'sa_forward'} ({kernels})",
            "alg_bytes_per_launch": int(fwd_bytes),
            "alg_flops_per_launch": int(fwd_flops), "avg_launch_us": fwd_s * 1e6}


def measured_traffic(workload, kernel):
    """HBM bytes per forward launch from profiles/<workload>_forward_traffic.md
    (rocprofv3 FETCH_SIZE and WRITE_SIZE runs scaled by a plain copy of known
    size), or None when there is no such summary or the forward sources have
    changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{workload}_forward_traffic.md")
    if not os.path.exists(path):
        return None
    rec = None
    with open(path) as f:
        for line in f:
            if line.startswith("TRAFFIC_JSON:"):
                rec = json.loads(line[len("TRAFFIC_JSON:"):])
    if rec is None or rec.get("kernel") != kernel:
        return None
    h = hashlib.sha256()
    for name in rec.get("sources", []):
        with open(os.path.join(ROOT, "block_sparse_paged_csr_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec.get("sources_sha256"):
        return None
    return rec["bytes_per_launch"]


def measured_mfma_util(workload):
    """MFMA utilisation of the MFMA forward kernel from
    profiles/<workload>_forward_mfma_util.md (rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES
    over GRBM_GUI_ACTIVE x SIMDs), or None when there is no such summary or the
    kernel's sources have changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{workload}_forward_mfma_util.md")
    if not os.path.exists(path):
        return None
    rec = None
    with open(path) as f:
        for line in f:
            if line.startswith("MFMA_JSON:"):
                rec = json.loads(line[len("MFMA_JSON:"):])
    if rec is None:
        return None
    h = hashlib.sha256()
    for name in rec.get("sources", []):
        with open(os.path.join(ROOT, "block_sparse_paged_csr_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec.get("sources_sha256"):
        return None
    return rec["mfma_util"]


def graph_step_us(sets, step, steps):
    """The same steps replayed from captured HIP graphs (one per batch)."""
    import torch
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for s in sets:
            step(s)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for s in sets:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(s)
        graphs.append(g)
    for i in range(len(graphs) * 2):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps * 1e6


if __name__ == "__main__":
    main()
