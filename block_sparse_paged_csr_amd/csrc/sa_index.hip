// Index build on the GPU: the KV-outer CSR index of types.rs (alice-llm
// 2.0.0, KvOuterIndex field docs) plus the work units that the forward walks.
//
//   k_index_init     zero the per-slot counters, reset the header, check
//                    cu_seqlens, and resolve (sequence, kv length) per query
//   k_index_hist     one thread per (q, h, r): drop padding / past-lk ranks,
//                    flag ids outside [-1, msb), check the block's touched
//                    page ids, count edges per (h, raw slot)
//   k_index_scan     a workgroup per chunk of 2048 slots of a head, chained by
//                    a decoupled look-back: exclusive scans of the counts,
//                    compaction of nonempty slots, unit counts per slot
//   k_index_scatter  one thread per kept (q, h, r): atomic cursor per slot,
//                    key q*topk + r into the slot's segment (unordered)
//                    (where one sequence's hkv*msb counters fit LDS, the
//                    histogram and the scatter run as *_agg variants that
//                    count a chunk of entries in LDS first)
//   k_index_rank     persistent over the nonempty slots of all heads: rank
//                    of each key inside its slot's segment; the plateau of
//                    sel_slots / sel_offsets past the nonempty slots
//                    (keys are unique) -> edges and inv in (q, r) order, then
//                    the slot's work units; workgroup 0 fills the header
//
// Small problems (a head's tq * topk entries and its slots fit one
// workgroup's LDS, as in decode) take one kernel instead, k_index_fused: a
// workgroup per head runs the same steps on LDS counters and member lists, and
// the heads' edge and unit bases come from a decoupled look-back over per-head
// totals that each workgroup publishes.
#include <cstddef>
#include <cstdlib>

#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kScanThreads = 256;
constexpr int kScanItems = kScanChunkSlots / kScanThreads;   // slots per thread
constexpr int kLookbackSpins = 1 << 22;              // then the build reports a runtime error
constexpr uint64_t kRankLookback = 5;                // error rank: a head's totals never appeared
constexpr int kAggThreads = 1024;                    // aggregating histogram / scatter
constexpr int kAggPer = 4;                           // entries per thread
constexpr int kAggItems = kAggThreads * kAggPer;     // entries per workgroup
constexpr int32_t kAggMaxSlots = 8192;               // hkv*msb LDS counters (32 KB)

__device__ inline int4 add4(int4 a, int4 b) {
  return make_int4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}
__device__ inline int4 sub4(int4 a, int4 b) {
  return make_int4(a.x - b.x, a.y - b.y, a.z - b.z, a.w - b.w);
}

__device__ inline int4 wave_sum4(int4 v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    v.x += __shfl_xor(v.x, off, 64);
    v.y += __shfl_xor(v.y, off, 64);
    v.z += __shfl_xor(v.z, off, 64);
    v.w += __shfl_xor(v.w, off, 64);
  }
  return v;
}

__device__ inline int4 wave_incl_scan4(int4 v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int4 t;
    t.x = __shfl_up(v.x, off, 64);
    t.y = __shfl_up(v.y, off, 64);
    t.z = __shfl_up(v.z, off, 64);
    t.w = __shfl_up(v.w, off, 64);
    if (lane >= off) v = add4(v, t);
  }
  return v;
}

__device__ inline int wave_incl_scan1(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  return v;
}

// Units of a slot with c edges. A slot with at least thr_e edges (rows >=
// the MFMA minimum) becomes ceil(c / cap) MFMA units; a smaller one becomes
// ceil(c / wave_cap) wavefront units. Part i of k spans
// [floor(i*c/k), floor((i+1)*c/k)), so the parts of a slot are near-equal.
__device__ inline void unit_split(int c, const BuildArgs& A, int thr_e, int* n_wave,
                                  int* n_mfma) {
  const bool is_m = c >= thr_e;
  const int cap = is_m ? A.cap_edges : A.wave_cap_edges;
  const uint32_t n = (uint32_t)(c + cap - 1);
  // the magic division is exact while n * cap < 2^40 (caps are <= 2048)
  const uint32_t k = n < (1u << 24) ? div_magic(n, is_m ? A.cap_magic : A.wave_cap_magic)
                                    : n / (uint32_t)cap;
  *n_wave = c > 0 && !is_m ? (int)k : 0;
  *n_mfma = c > 0 && is_m ? (int)k : 0;
}

__global__ __launch_bounds__(256) void k_index_init(IndexPtrs P, BuildArgs A) {
  const int64_t n = (int64_t)A.hkv * A.nbs;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) P.cnt[i] = 0;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < A.tq; q += stride) {
    const int32_t b = batch_of_dev(A.cu, A.batch, q);
    P.qinfo[q] = make_int2(b, (int32_t)kv_len_dev(A.used, b, A.msb, A.block_size));
  }
  if (blockIdx.x != 0) return;
  if (threadIdx.x == 0) {
    DevHeader* h = P.hdr;
    h->err_key = ~0ull;
    h->status = 0;
    h->what_code = kWhatNone;
    h->err_expected = 0;
    h->err_got = 0;
    h->total_edges = 0;
    h->num_units_wave = 0;
    h->num_units_mfma = 0;
    h->num_slots = 0;
    P.sort_hist[kSortHistCounter] = 0;           // the unit sort's counter
    h->geom[0] = (int32_t)A.tq;
    h->geom[1] = A.hkv;
    h->geom[2] = A.topk;
    h->geom[3] = A.batch;
    h->geom[4] = A.max_pages;
    h->geom[5] = A.block_size;
    h->geom[6] = A.page_size;
    h->geom[7] = A.qhead;
  }
  __syncthreads();
  // cu_seqlens content (types.rs CuSeqlensQ::new): cu[0] == 0, non-decreasing.
  for (int32_t b = threadIdx.x; b < A.batch; b += 256)
    if (A.cu[b + 1] < A.cu[b]) atomicMin(&P.hdr->err_key, err_key(kRankCuContent, b + 1));
  if (threadIdx.x == 0) {
    if (A.cu[0] != 0) atomicMin(&P.hdr->err_key, err_key(kRankCuContent, 0));
    if (A.cu[A.batch] != A.tq) atomicMin(&P.hdr->err_key, err_key(kRankCuTotal, 0));
  }
}

// Thread per entry of `selected`, in memory order idx = (q*hkv + h)*topk + r.
// One entry idx = (q*hkv + h)*topk + r of `selected`: sets inv to -1, flags
// an id outside [-1, msb) and missing page ids of the block's valid range; a
// kept entry (a valid id whose block starts below the sequence's kv length)
// returns true with its head h, sequence b and block v.
__device__ inline bool hist_entry(const IndexPtrs& P, const BuildArgs& A, int64_t idx, int32_t* hp,
                                  int32_t* bp, int32_t* vp) {
  const int32_t r = (int32_t)(idx % A.topk);
  const int64_t qh = idx / A.topk;
  const int32_t h = (int32_t)(qh % A.hkv);
  const int64_t q = qh / A.hkv;
  const int32_t v = A.selected[idx];
  const int2 qi = P.qinfo[q];
  P.inv[((int64_t)h * A.tq + q) * A.topk + r] = -1;
  if (v == -1) return false;
  if (v < -1 || v >= A.msb) {
    atomicMin(&P.hdr->err_key, err_key(kRankSelected, (uint64_t)idx));
    return false;
  }
  const int32_t b = qi.x;
  const int64_t lk = qi.y;
  const int64_t block_start = (int64_t)v * A.block_size;
  if (block_start >= lk) return false;
  if (A.num_pages >= 0) {
    // Pages that the kept block's valid range touches must exist (the
    // forward's "block_tables page id" check, moved into the build).
    const int64_t block_end = block_start + A.block_size < lk ? block_start + A.block_size : lk;
    const int64_t col0 = (int64_t)b * A.max_pages + (int64_t)v * A.ppb;
    int64_t bad = INT64_MAX;
    for (int32_t pl = 0; pl < A.ppb; ++pl) {
      const bool touched = block_start + (int64_t)pl * A.page_size < block_end;
      const int32_t page = touched ? A.block_tables[col0 + pl] : -1;
      if (page >= A.num_pages && col0 + pl < bad) bad = col0 + pl;
    }
    if (bad != INT64_MAX) atomicMin(&P.hdr->err_key, err_key(kRankPage, (uint64_t)bad));
  }
  *hp = h;
  *bp = b;
  *vp = v;
  return true;
}

__global__ __launch_bounds__(256) void k_index_hist(IndexPtrs P, BuildArgs A) {
  const int64_t total = A.tq * A.hkv * A.topk;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  int32_t h, b, v;
  if (hist_entry(P, A, idx, &h, &b, &v)) atomicAdd(&P.cnt[(int64_t)h * A.nbs + (int64_t)b * A.msb + v], 1);
}

// Aggregating variants of the histogram and the scatter: a workgroup takes
// kAggItems consecutive entries, which cover a run of consecutive queries and
// so mostly one sequence b0 (that of the chunk's first query). Its kept
// entries of b0 count into LDS counters over (h, v) (hkv*msb of them, dynamic
// LDS), and the workgroup then adds each nonzero count to the global counter
// with one atomic. Entries of another sequence take the global atomic
// directly. Selections concentrate on a few blocks per sequence (sinks, local
// windows, popular blocks), so this turns most same-address device atomics
// into LDS ones.
__global__ __launch_bounds__(kAggThreads) void k_index_hist_agg(IndexPtrs P, BuildArgs A) {
  extern __shared__ int32_t s_agg[];
  const int tid = threadIdx.x;
  const int64_t total = A.tq * A.hkv * A.topk;
  const int32_t nloc = A.hkv * A.msb;
  const int64_t c0 = (int64_t)blockIdx.x * kAggItems;
  for (int32_t j = tid; j < nloc; j += kAggThreads) s_agg[j] = 0;
  // the grid covers total > 0 entries, but guard the empty launch anyway
  const int32_t b0 = c0 < total ? P.qinfo[c0 / ((int64_t)A.hkv * A.topk)].x : -1;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kAggPer; ++k) {
    const int64_t idx = c0 + (int64_t)k * kAggThreads + tid;
    int32_t h, b, v;
    if (idx < total && hist_entry(P, A, idx, &h, &b, &v)) {
      if (b == b0) atomicAdd(&s_agg[h * A.msb + v], 1);
      else atomicAdd(&P.cnt[(int64_t)h * A.nbs + (int64_t)b * A.msb + v], 1);
    }
  }
  __syncthreads();
  for (int32_t j = tid; j < nloc; j += kAggThreads) {
    const int32_t c = s_agg[j];
    const int32_t h = j / A.msb;
    if (c > 0) atomicAdd(&P.cnt[(int64_t)h * A.nbs + (int64_t)b0 * A.msb + (j - h * A.msb)], c);
  }
}

// Workgroup (h, c) scans chunk c (kScanChunkSlots slots) of head h: its
// counts, loaded together, give the local sums; the chunk's offset within
// the head comes from a decoupled look-back over the chunks before it
// (chunk aggregates and inclusive sums tagged with the build call's epoch).
// Chunks of a head are dispatched in order, so every chunk waited on is
// already running or done; a spin limit turns a missing chunk into a
// runtime error instead of a hang. Outputs per nonempty slot: its compact
// position, CSR offset, unit offsets, and the scatter cursor. The last chunk
// writes the head totals and sel_offsets at the end of the compact list; the
// rank kernel fills the rest of the plateau.
__global__ __launch_bounds__(kScanThreads) void k_index_scan(IndexPtrs P, BuildArgs A) {
  const int64_t nbs = A.nbs;
  const int32_t nch = (int32_t)scan_chunks(nbs);
  const int32_t h = (int32_t)blockIdx.x / nch, ch = (int32_t)blockIdx.x - h * nch;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  constexpr int kWavesScan = kScanThreads / 64;
  __shared__ int4 s_wave[kWavesScan];
  __shared__ int4 s_excl;
  int32_t* cnt = P.cnt + (int64_t)h * nbs;
  const int thr_e = (int)(((int64_t)A.mfma_min_rows + A.qhead - 1) / A.qhead);
  const int64_t base = (int64_t)ch * kScanChunkSlots + (int64_t)tid * kScanItems;
  // clamped loads, none behind its own branch: all of them in flight together
  int c[kScanItems] = {};
  if (nbs > 0) {
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
      const int64_t raw = base + k;
      const int v = cnt[raw < nbs ? raw : nbs - 1];
      c[k] = raw < nbs ? v : 0;
    }
  }
  int nw[kScanItems], nm[kScanItems];
  int4 mine = make_int4(0, 0, 0, 0);        // edges, nonempty slots, wave units, mfma units
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    unit_split(c[k], A, thr_e, &nw[k], &nm[k]);
    mine = add4(mine, make_int4(c[k], c[k] > 0, nw[k], nm[k]));
  }
  const int4 incl = wave_incl_scan4(mine);
  if (lane == 63) s_wave[wid] = incl;
  __syncthreads();
  int4 pre = make_int4(0, 0, 0, 0), agg = make_int4(0, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < kWavesScan; ++i) {
    const int4 t = s_wave[i];
    if (i < wid) pre = add4(pre, t);
    agg = add4(agg, t);
  }
  if (wid == 0) {
    // Wave-parallel look-back: lane i reads chunk ch-1-i (64 predecessors per
    // round trip). The chunks up to the nearest one whose inclusive sum is
    // out contribute (their aggregates, that one its inclusive sum); if none
    // is, the whole window's aggregates count and the next window follows.
    ChunkAgg* my = P.chunk_agg + (int64_t)h * nch + ch;
    int4 excl = make_int4(0, 0, 0, 0);
    if (ch > 0) {
      if (lane == 0) {
        my->agg = agg;
        __hip_atomic_store(&my->flag, A.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      }
      for (int32_t top = ch - 1; top >= 0; top -= 64) {
        const int32_t p = top - lane;
        uint64_t f = 0;
        int4 val = make_int4(0, 0, 0, 0);
        if (p >= 0) {
          const ChunkAgg* pa = P.chunk_agg + (int64_t)h * nch + p;
          int spins = 0;
          while (true) {
            f = __hip_atomic_load(&pa->flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
            if (f == A.epoch || f == A.epoch + 1 || spins >= kLookbackSpins) break;
            __builtin_amdgcn_s_sleep(1);
            ++spins;
          }
          if (f == A.epoch + 1) val = pa->incl;
          else if (f == A.epoch) val = pa->agg;
        }
        const bool bad = p >= 0 && f != A.epoch && f != A.epoch + 1;
        if (__ballot(bad) != 0) {
          if (lane == 0) atomicMin(&P.hdr->err_key, err_key(kRankLookback, 0));
          break;
        }
        const uint64_t have_incl = __ballot(p >= 0 && f == A.epoch + 1);
        const int stop = have_incl != 0 ? __builtin_ctzll(have_incl) : 64;
        excl = add4(excl, wave_sum4(lane <= stop ? val : make_int4(0, 0, 0, 0)));
        if (have_incl != 0) break;
      }
    }
    if (lane == 0) {
      my->incl = add4(excl, agg);
      __hip_atomic_store(&my->flag, A.epoch + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      s_excl = excl;
      if (ch == nch - 1) {
        const int4 tot = add4(excl, agg);
        P.num_sel[h] = tot.y;
        P.head_e[h] = tot.x;
        P.head_uw[h] = tot.z;
        P.head_um[h] = tot.w;
        P.sel_offsets[(int64_t)h * (nbs + 1) + tot.y] = tot.x;
      }
    }
  }
  __syncthreads();
  int4 run = add4(add4(s_excl, pre), sub4(incl, mine));
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    const int64_t raw = base + k;
    if (c[k] > 0) {
      const int64_t j = run.y;
      P.sel_slots[(int64_t)h * nbs + j] = (int32_t)raw;
      P.sel_offsets[(int64_t)h * (nbs + 1) + j] = run.x;
      P.slot_uw[(int64_t)h * nbs + j] = run.z;
      P.slot_um[(int64_t)h * nbs + j] = run.w;
      cnt[raw] = run.x;                               // scatter cursor
    }
    run = add4(run, make_int4(c[k], c[k] > 0, nw[k], nm[k]));
  }
}

__device__ inline int64_t head_edge_base(const IndexPtrs& P, int32_t h) {
  int64_t s = 0;
  for (int32_t i = 0; i < h; ++i) s += P.head_e[i];
  return s;
}

__global__ __launch_bounds__(256) void k_index_scatter(IndexPtrs P, BuildArgs A) {
  const int64_t total = A.tq * A.hkv * A.topk;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int32_t r = (int32_t)(idx % A.topk);
  const int64_t qh = idx / A.topk;
  const int32_t h = (int32_t)(qh % A.hkv);
  const int64_t q = qh / A.hkv;
  const int32_t v = A.selected[idx];
  const int2 qi = P.qinfo[q];
  const int64_t hb = head_edge_base(P, h);
  if (v < 0 || v >= A.msb) return;
  if ((int64_t)v * A.block_size >= qi.y) return;
  const int32_t pos = atomicAdd(&P.cnt[(int64_t)h * A.nbs + (int64_t)qi.x * A.msb + v], 1);
  P.keys[hb + pos] = (int32_t)(q * A.topk + r);
}

// The scatter's aggregating variant (see k_index_hist_agg): LDS cursors hand
// out offsets inside the chunk's share of each (h, v) slot of b0, and one
// global atomic per nonzero slot reserves that share.
__global__ __launch_bounds__(kAggThreads) void k_index_scatter_agg(IndexPtrs P, BuildArgs A) {
  extern __shared__ int32_t s_agg[];
  const int tid = threadIdx.x;
  const int64_t total = A.tq * A.hkv * A.topk;
  const int32_t nloc = A.hkv * A.msb;
  const int64_t c0 = (int64_t)blockIdx.x * kAggItems;
  for (int32_t j = tid; j < nloc; j += kAggThreads) s_agg[j] = 0;
  // the grid covers total > 0 entries, but guard the empty launch anyway
  const int32_t b0 = c0 < total ? P.qinfo[c0 / ((int64_t)A.hkv * A.topk)].x : -1;
  __syncthreads();
  int32_t loc[kAggPer], li[kAggPer], key[kAggPer], hh[kAggPer];
#pragma unroll
  for (int k = 0; k < kAggPer; ++k) {
    loc[k] = -1;
    const int64_t idx = c0 + (int64_t)k * kAggThreads + tid;
    if (idx >= total) continue;
    const int32_t r = (int32_t)(idx % A.topk);
    const int64_t qh = idx / A.topk;
    const int32_t h = (int32_t)(qh % A.hkv);
    const int64_t q = qh / A.hkv;
    const int32_t v = A.selected[idx];
    const int2 qi = P.qinfo[q];
    if (v < 0 || v >= A.msb || (int64_t)v * A.block_size >= qi.y) continue;
    key[k] = (int32_t)(q * A.topk + r);
    hh[k] = h;
    if (qi.x == b0) {
      loc[k] = h * A.msb + v;
      li[k] = atomicAdd(&s_agg[loc[k]], 1);
    } else {
      const int32_t pos = atomicAdd(&P.cnt[(int64_t)h * A.nbs + (int64_t)qi.x * A.msb + v], 1);
      P.keys[head_edge_base(P, h) + pos] = key[k];
    }
  }
  __syncthreads();
  for (int32_t j = tid; j < nloc; j += kAggThreads) {
    const int32_t c = s_agg[j];
    const int32_t h = j / A.msb;
    if (c > 0) s_agg[j] = atomicAdd(&P.cnt[(int64_t)h * A.nbs + (int64_t)b0 * A.msb + (j - h * A.msb)], c);
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kAggPer; ++k)
    if (loc[k] >= 0) P.keys[head_edge_base(P, hh[k]) + s_agg[loc[k]] + li[k]] = key[k];
}

// Status and error details from the smallest error key (~0ull: none).
__device__ void set_status(DevHeader* hd, const BuildArgs& A, unsigned long long key) {
  if (key == ~0ull) { hd->status = SA_OK; return; }
  const uint64_t rank = key >> 56;
  const int64_t pos = (int64_t)(key & ((1ull << 56) - 1));
  if (rank == kRankCuContent) {
    hd->status = SA_ERR_CU_SEQLENS;
  } else if (rank == kRankCuTotal) {
    hd->status = SA_ERR_SHAPE;
    hd->what_code = kWhatCuTotal;
    hd->err_expected = A.tq;
    hd->err_got = A.cu[A.batch];
  } else if (rank == kRankSelected) {
    hd->status = SA_ERR_SELECTED_RANGE;
    hd->err_expected = A.msb;
    hd->err_got = A.selected[pos];
  } else if (rank == kRankPage) {
    hd->status = SA_ERR_SHAPE;
    hd->what_code = kWhatPageId;
    hd->err_expected = A.num_pages;
    hd->err_got = A.block_tables[pos];
  } else {
    hd->status = SA_ERR_GPU_RUNTIME;
  }
}

__device__ void finalize_header(const IndexPtrs& P, const BuildArgs& A) {
  int64_t e = 0, ns = 0;
  int32_t uw = 0, um = 0;
  for (int32_t h = 0; h < A.hkv; ++h) {
    P.edge_head_base[h] = e;
    e += P.head_e[h];
    uw += P.head_uw[h];
    um += P.head_um[h];
    ns += P.num_sel[h];
  }
  P.edge_head_base[A.hkv] = e;
  DevHeader* hd = P.hdr;
  hd->total_edges = e;
  hd->num_units_wave = uw;
  hd->num_units_mfma = um;
  hd->num_slots = ns;
  set_status(hd, A, hd->err_key);
}

constexpr int kRankChunk = 2048;   // keys staged in LDS per pass
constexpr int kRankKeys = 4;       // keys held per thread per pass
constexpr int kRankBitmapMaxWords = 4096;   // 16 KB (a sequence of up to 131072 keys): a
                                            // larger bitmap costs the small slots occupancy
constexpr int kRankBitmapMinKeys = 128;     // smaller slots: pairwise counting is cheaper

__device__ inline void write_edge(const IndexPtrs& P, const BuildArgs& A, int32_t h,
                                  int64_t head_base, int32_t off0, int32_t key, int32_t rank) {
  const int32_t q = key / A.topk, r = key % A.topk;
  const int64_t e = head_base + off0 + rank;
  *reinterpret_cast<int2*>(P.edges + 2 * e) = make_int2(q, r);
  P.inv[((int64_t)h * A.tq + q) * A.topk + r] = off0 + rank;
}

struct SlotInfo {
  int32_t n, h, j, off0, uw, um, b, blk, lk, delta;
  int32_t kb, nw;   // the sequence's key range [kb, kb + 32*nw) covers the slot's keys
  int64_t base;
};

// Persistent over the nonempty slots of all heads, numbered densely head by
// head (g = sum of num_sel over heads before h, plus j): each pass of a
// workgroup takes 4 consecutive ids g = 4*gg + wave. Slots with <= 64 keys
// are ranked by their wave with lane shuffles. If any of the 4 has more, the
// whole workgroup ranks them one after another through LDS.
__global__ __launch_bounds__(256) void k_index_rank(IndexPtrs P, BuildArgs A) {
  if (blockIdx.x == 0 && threadIdx.x == 0) finalize_header(P, A);
  if (A.nbs == 0) return;                          // no slots at all (msb == 0)
  // Every device error is final once the histogram has run. A failed build
  // leaves edges, inv and the units unused, so the ranking is skipped; with
  // bad cu_seqlens a slot's keys need not lie in its sequence's key range,
  // which the bitmap below relies on.
  if (__hip_atomic_load(&P.hdr->err_key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != ~0ull)
    return;
  extern __shared__ uint32_t s_bits[];              // [rank_bitmap_words] (dynamic)
  __shared__ SlotInfo s_slot[4];
  __shared__ __align__(16) int32_t s_keys[kRankChunk];
  __shared__ int64_t s_total;
  __shared__ int s_wsum[4];
  __shared__ int s_runpre[256];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid == 0) {
    int64_t t = 0;
    for (int32_t h = 0; h < A.hkv; ++h) t += P.num_sel[h];
    s_total = t;
  }
  // plateau past each head's nonempty slots: sel_slots -1, sel_offsets E_h
  // (the scan wrote sel_offsets at num_sel itself)
  {
    const int64_t gsz = (int64_t)gridDim.x * 256, gid = (int64_t)blockIdx.x * 256 + tid;
    for (int32_t h = 0; h < A.hkv; ++h) {
      const int32_t ns = P.num_sel[h];
      const int32_t eh = P.head_e[h];
      for (int64_t j = ns + gid; j < A.nbs; j += gsz) P.sel_slots[(int64_t)h * A.nbs + j] = -1;
      for (int64_t j = ns + 1 + gid; j <= A.nbs; j += gsz)
        P.sel_offsets[(int64_t)h * (A.nbs + 1) + j] = eh;
    }
  }
  __syncthreads();
  const int64_t total = s_total;
  const int32_t thr_e = (int32_t)(((int64_t)A.mfma_min_rows + A.qhead - 1) / A.qhead);
  for (int64_t gg = blockIdx.x; 4 * gg < total; gg += gridDim.x) {
    const int64_t g = 4 * gg + w;
    if (lane == 0) {
      SlotInfo si{};
      if (g < total) {
        // head of dense id g and the totals of the heads before it
        int64_t j = g, hb = 0;
        int32_t h = 0, uw = 0, um = 0;
        for (; h < A.hkv; ++h) {
          const int32_t ns = P.num_sel[h];
          if (j < ns) break;
          j -= ns;
          hb += P.head_e[h];
          uw += P.head_uw[h];
          um += P.head_um[h];
        }
        const int32_t o0 = P.sel_offsets[(int64_t)h * (A.nbs + 1) + j];
        const int32_t o1 = P.sel_offsets[(int64_t)h * (A.nbs + 1) + j + 1];
        const int32_t raw = P.sel_slots[(int64_t)h * A.nbs + j];
        si.n = o1 - o0;
        si.off0 = o0;
        si.base = hb;
        si.uw = uw + P.slot_uw[(int64_t)h * A.nbs + j];
        si.um = um + P.slot_um[(int64_t)h * A.nbs + j];
        si.b = raw / A.msb;
        si.blk = raw % A.msb;
        const int64_t q0 = A.cu[si.b], qo_len = A.cu[si.b + 1] - q0;
        const int64_t lk = kv_len_dev(A.used, si.b, A.msb, A.block_size);
        si.lk = (int32_t)lk;
        si.delta = (int32_t)((lk >= qo_len ? lk - qo_len : 0) - q0);
        si.kb = (int32_t)(q0 * A.topk);
        si.nw = (int32_t)((qo_len * A.topk + 31) / 32);
        si.h = h;
        si.j = (int32_t)j;
      }
      s_slot[w] = si;
    }
    __syncthreads();
    const bool block_mode =
        s_slot[0].n > 64 || s_slot[1].n > 64 || s_slot[2].n > 64 || s_slot[3].n > 64;
    if (!block_mode) {
      const int32_t n = s_slot[w].n;
      if (n > 0) {
        const int32_t* seg = P.keys + s_slot[w].base + s_slot[w].off0;
        const int32_t key = lane < n ? seg[lane] : INT32_MAX;
        int32_t rank = 0;
        for (int32_t x = 0; x < n; ++x) rank += __shfl(key, x, 64) < key;
        if (lane < n) write_edge(P, A, s_slot[w].h, s_slot[w].base, s_slot[w].off0, key, rank);
      }
    } else {
      for (int s = 0; s < 4; ++s) {
        const int32_t n = s_slot[s].n;
        if (n == 0) continue;
        const int32_t* seg = P.keys + s_slot[s].base + s_slot[s].off0;
        if (s_slot[s].nw <= A.rank_bitmap_words && n >= kRankBitmapMinKeys) {
          // The slot's keys as bits of a bitmap over its sequence's key
          // range (the slot's queries are that sequence's); a key's rank is
          // the number of set bits before it: a prefix count per thread's
          // run of words, then within the run.
          const int32_t W = s_slot[s].nw, kb = s_slot[s].kb;
          const int32_t C = (W + 255) / 256;                 // words per thread
          for (int32_t x = tid; x < W; x += 256) s_bits[x] = 0u;
          __syncthreads();
          const uint32_t nbits = 32u * (uint32_t)W;
          for (int32_t i = tid; i < n; i += 256) {
            const int32_t bit = seg[i] - kb;
            if ((uint32_t)bit < nbits) atomicOr(&s_bits[bit >> 5], 1u << (bit & 31));
          }
          __syncthreads();
          int cntw = 0;
          for (int32_t x = 0; x < C; ++x) {
            const int32_t wd = tid * C + x;
            cntw += wd < W ? __popc(s_bits[wd]) : 0;
          }
          const int incl = wave_incl_scan1(cntw);
          if (lane == 63) s_wsum[w] = incl;
          __syncthreads();
          int pre = incl - cntw;
#pragma unroll
          for (int i = 0; i < 4; ++i) pre += i < w ? s_wsum[i] : 0;
          s_runpre[tid] = pre;
          __syncthreads();
          for (int32_t i = tid; i < n; i += 256) {
            const int32_t key = seg[i], bit = key - kb;
            if ((uint32_t)bit >= nbits) continue;      // not reached with valid cu_seqlens
            const int32_t wd = bit >> 5, run = wd / C;
            int32_t rank = s_runpre[run];
            for (int32_t x = run * C; x < wd; ++x) rank += __popc(s_bits[x]);
            rank += __popc(s_bits[wd] & ((1u << (bit & 31)) - 1u));
            write_edge(P, A, s_slot[s].h, s_slot[s].base, s_slot[s].off0, key,
                       rank < n ? rank : n - 1);
          }
          __syncthreads();                           // the bitmap is reused
          continue;
        }
        for (int32_t pass = 0; pass < n; pass += 256 * kRankKeys) {
          int32_t mine[kRankKeys], rank[kRankKeys];
#pragma unroll
          for (int k = 0; k < kRankKeys; ++k) {
            const int32_t i = pass + tid + 256 * k;
            mine[k] = i < n ? seg[i] : INT32_MAX;
            rank[k] = 0;
          }
          for (int32_t c0 = 0; c0 < n; c0 += kRankChunk) {
            const int32_t m = n - c0 < kRankChunk ? n - c0 : kRankChunk;
            const int32_t m4 = (m + 3) & ~3;
            __syncthreads();
            for (int32_t x = tid; x < m4; x += 256) s_keys[x] = x < m ? seg[c0 + x] : INT32_MAX;
            __syncthreads();
            for (int32_t x = 0; x < m4; x += 4) {
              const int4 kk = *reinterpret_cast<const int4*>(&s_keys[x]);
#pragma unroll
              for (int k = 0; k < kRankKeys; ++k)
                rank[k] += (kk.x < mine[k]) + (kk.y < mine[k]) + (kk.z < mine[k]) + (kk.w < mine[k]);
            }
          }
#pragma unroll
          for (int k = 0; k < kRankKeys; ++k) {
            const int32_t i = pass + tid + 256 * k;
            if (i < n)
              write_edge(P, A, s_slot[s].h, s_slot[s].base, s_slot[s].off0, mine[k], rank[k]);
          }
        }
      }
    }
    // Work units of this wave's slot, in CSR order within each kind.
    const SlotInfo si = s_slot[w];
    if (si.n > 0) {
      const bool is_m = si.n >= thr_e;
      const int32_t cap = is_m ? A.cap_edges : A.wave_cap_edges;
      const int32_t k_units = (si.n + cap - 1) / cap;
      Unit* dst = is_m ? P.units_mfma + si.um : P.units_wave + si.uw;
      const int64_t e_base = si.base + si.off0;
      for (int32_t i = lane; i < k_units; i += 64) {
        const int32_t s0 = (int32_t)(((int64_t)i * si.n) / k_units);
        const int32_t s1 = (int32_t)(((int64_t)(i + 1) * si.n) / k_units);
        dst[i] = Unit{si.h, si.j, (int32_t)(e_base + s0), (int32_t)(e_base + s1),
                      si.b, si.blk, si.lk, si.delta};
      }
    }
    __syncthreads();                               // s_slot and s_keys are reused
  }
}

// ------------------------------------------------------------ fused build
constexpr int kFusedThreads = 1024;
constexpr int kFusedItems = 4;                       // entries per thread and head
constexpr int64_t kFusedMaxSlots = 16384;
constexpr int64_t kFusedMaxQ = 2048;
constexpr int32_t kFusedMaxBatch = 2048;
constexpr size_t kFusedMaxLds = 150 * 1024;            // dynamic LDS of the fused build
// Inclusive wave64 scans on DPP: row_shr 1, 2, 4, 8 inside each row of 16
// lanes, then row_bcast 15 and 31 carry row totals across rows (rows the
// broadcast does not write keep the identity).
__device__ inline uint32_t wave_incl_sum(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);
  return v;
}
__device__ inline int wave_incl_max(int v) {
  int t;
  t = __builtin_amdgcn_update_dpp(-1, v, 0x111, 0xf, 0xf, false); v = v > t ? v : t;
  t = __builtin_amdgcn_update_dpp(-1, v, 0x112, 0xf, 0xf, false); v = v > t ? v : t;
  t = __builtin_amdgcn_update_dpp(-1, v, 0x114, 0xf, 0xf, false); v = v > t ? v : t;
  t = __builtin_amdgcn_update_dpp(-1, v, 0x118, 0xf, 0xf, false); v = v > t ? v : t;
  t = __builtin_amdgcn_update_dpp(-1, v, 0x142, 0xa, 0xf, false); v = v > t ? v : t;
  t = __builtin_amdgcn_update_dpp(-1, v, 0x143, 0xc, 0xf, false); v = v > t ? v : t;
  return v;
}

// Exclusive scan of two packed sums over the workgroup (kFusedThreads);
// *ta / *tb get the totals.
__device__ uint2 block_excl_scan2(uint32_t a, uint32_t b, uint2* s_w, uint32_t* ta, uint32_t* tb) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t ia = wave_incl_sum(a), ib = wave_incl_sum(b);
  if (lane == 63) s_w[wid] = make_uint2(ia, ib);
  __syncthreads();
  if (wid == 0) {
    const uint2 w = lane < kFusedThreads / 64 ? s_w[lane] : make_uint2(0u, 0u);
    const uint32_t wa = wave_incl_sum(w.x), wb = wave_incl_sum(w.y);
    if (lane < kFusedThreads / 64) s_w[lane] = make_uint2(wa, wb);
  }
  __syncthreads();
  uint2 ex = make_uint2(ia - a, ib - b);
  if (wid > 0) {
    ex.x += s_w[wid - 1].x;
    ex.y += s_w[wid - 1].y;
  }
  *ta = s_w[kFusedThreads / 64 - 1].x;
  *tb = s_w[kFusedThreads / 64 - 1].y;
  __syncthreads();
  return ex;
}

// Max over the values of lower threads (-1 if none).
__device__ int block_excl_max(int v, int* s_w) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int incl = wave_incl_max(v);
  if (lane == 63) s_w[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    int w = lane < kFusedThreads / 64 ? s_w[lane] : -1;
    w = wave_incl_max(w);
    if (lane < kFusedThreads / 64) s_w[lane] = w;
  }
  __syncthreads();
  int ex = __builtin_amdgcn_update_dpp(-1, incl, 0x138, 0xf, 0xf, false);   // wave_shr:1
  if (wid > 0) ex = ex > s_w[wid - 1] ? ex : s_w[wid - 1];
  __syncthreads();
  return ex;
}

// Packed per-slot sums for the fused scans: (edges | nonempty << 16) and
// (wavefront units | MFMA units << 16); a head has at most 4096 entries, so
// no field carries into the next.
__device__ inline uint2 slot_sums(int c, const BuildArgs& A, int thr_e) {
  if (c <= 0) return make_uint2(0u, 0u);
  const bool is_m = c >= thr_e;
  const uint32_t n = is_m ? div_magic((uint32_t)(c + A.cap_edges - 1), A.cap_magic)
                          : div_magic((uint32_t)(c + A.wave_cap_edges - 1), A.wave_cap_magic);
  return make_uint2((uint32_t)c | (1u << 16), is_m ? n << 16 : n);
}

// Per (h, raw slot) counts of kept entries, their exclusive offsets, the
// member list of each slot and each entry's rank in it, the compact slot list
// and the slot's units, all for head h = blockIdx.x. Entry i = q * topk + r
// of the head is handled by thread i % 1024. Dynamic LDS (int32): counts, then
// offsets [nbs]; member lists [tq*topk]; compact slot list and unit offsets
// [min(nbs, tq*topk)] each; batch of each query [tq]; lk and causal delta per
// sequence [batch] each.
__global__ __launch_bounds__(kFusedThreads) void k_index_fused(IndexPtrs P, BuildArgs A) {
  extern __shared__ __align__(16) int32_t s_dyn[];
  __shared__ uint2 s_w2[kFusedThreads / 64];
  __shared__ int s_w1[kFusedThreads / 64];
  __shared__ unsigned long long s_err;
  __shared__ unsigned long long s_base_e, s_base_ns;
  __shared__ int32_t s_base_uw, s_base_um;

  const int32_t h = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t nbs = A.nbs;
  const int32_t tq = (int32_t)A.tq, topk = A.topk, hkv = A.hkv, batch = A.batch;
  const int32_t items = tq * topk;
  const int32_t nslots = (int32_t)nbs;          // nbs <= kFusedMaxSlots
  const int32_t nlist = nslots < items ? nslots : items;   // nonempty slots <= both
  int32_t* s_cnt = s_dyn;                       // [nbs]   counts, then offsets
  int32_t* s_mem = s_cnt + nslots;              // [items] member lists
  int32_t* s_list = s_mem + items;              // [nlist] raw slot of compact slot j
  uint32_t* s_uoff = reinterpret_cast<uint32_t*>(s_list + nlist);  // [nlist] unit offsets
  int32_t* s_qb = reinterpret_cast<int32_t*>(s_uoff + nlist);      // [tq]
  int32_t* s_lkb = s_qb + tq;                   // [batch]
  int32_t* s_dlb = s_lkb + batch;               // [batch]

  // Entry slots k (entries tid + kFusedThreads k) that hold an entry for some
  // lane of this wave; the loops over entries skip the others as a whole
  // wave (with tq * topk below the workgroup's capacity, most waves have
  // one slot or none).
  const int32_t tid0 = tid - (tid & 63);
  const int32_t nk_wave = tid0 < items ? (items - tid0 + kFusedThreads - 1) / kFusedThreads : 0;

  // this thread's entries of `selected`, loaded first so that their latency
  // overlaps the per-sequence setup
  int32_t v_k[kFusedItems];
#pragma unroll
  for (int k = 0; k < kFusedItems; ++k) {
    v_k[k] = -1;
    if (k >= nk_wave) continue;
    const int32_t i = tid + kFusedThreads * k;
    const int32_t q = i / topk, r = i - q * topk;
    v_k[k] = i < items ? A.selected[((int64_t)q * hkv + h) * topk + r] : -1;
  }

  // this thread's sequences (b = tid + kFusedThreads k): cu bounds and used
  // length, also loaded before the LDS setup (clamped, no load behind a branch)
  constexpr int kSeqPerThread = (kFusedMaxBatch + kFusedThreads - 1) / kFusedThreads;
  int64_t c0_k[kSeqPerThread], c1_k[kSeqPerThread];
  int32_t used_k[kSeqPerThread];
  // (sequence slots with no sequence for any lane of the wave read nothing)
  const int32_t nb_wave = tid0 < batch ? (batch - tid0 + kFusedThreads - 1) / kFusedThreads : 0;
#pragma unroll
  for (int k = 0; k < kSeqPerThread; ++k) {
    c0_k[k] = c1_k[k] = 0;
    used_k[k] = 0;
    if (k >= nb_wave) continue;
    const int32_t b = tid + kFusedThreads * k;
    const int32_t bb = b < batch ? b : 0;
    c0_k[k] = A.cu[bb];
    c1_k[k] = A.cu[bb + 1];
    used_k[k] = A.used != nullptr ? A.used[bb] : 0;
  }
  // cu[0] and cu[batch] for head 0's checks, loaded here with the rest (cu
  // has batch + 1 entries): behind the check's branches they were two
  // serial round trips that the workgroup barrier below waited for
  const int64_t cu_first = A.cu[0], cu_last = A.cu[batch];

  // ---- per-sequence lk and causal delta; batch of each query; cu checks
  for (int32_t x = tid; x < nslots; x += kFusedThreads) s_cnt[x] = 0;
  for (int32_t q = tid; q < tq; q += kFusedThreads) s_qb[q] = -1;
  if (tid == 0) {
    s_err = ~0ull;
    s_base_e = 0;
    s_base_ns = 0;
    s_base_uw = 0;
    s_base_um = 0;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kSeqPerThread; ++k) {
    const int32_t b = tid + kFusedThreads * k;
    if (b >= batch) break;
    const int64_t c0 = c0_k[k], c1 = c1_k[k];
    // kv_len_dev: used length clamped at 0, or the whole block-table row
    const int64_t lk = A.used == nullptr ? (int64_t)A.msb * A.block_size
                                         : (used_k[k] > 0 ? (int64_t)used_k[k] : 0);
    const int64_t qo_len = c1 - c0;
    s_lkb[b] = (int32_t)lk;
    s_dlb[b] = (int32_t)((lk >= qo_len ? lk - qo_len : 0) - c0);
    // cu_seqlens content (types.rs CuSeqlensQ::new): non-decreasing
    if (h == 0 && c1 < c0) atomicMin(&s_err, err_key(kRankCuContent, b + 1));
    if (c0 < c1 && c0 >= 0 && c0 < tq) s_qb[c0] = b;   // first query of a nonempty sequence
  }
  if (h == 0 && tid == 0) {
    if (cu_first != 0) atomicMin(&s_err, err_key(kRankCuContent, 0));
    if (cu_last != A.tq) atomicMin(&s_err, err_key(kRankCuTotal, 0));
  }
  __syncthreads();
  {
    // batch of q = last sequence starting at or before q (types.rs batch_of):
    // a max-scan over the queries, four a thread; up to 256 queries it is
    // wave 0's alone (no workgroup barriers)
    if (tq > 256 || tid < 64) {
      int v[4], m = -1;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int32_t q = 4 * tid + k;
        v[k] = q < tq ? s_qb[q] : -1;
        m = v[k] > m ? v[k] : m;
        v[k] = m;
      }
      const int pre = tq > 256 ? block_excl_max(m, s_w1)
                               : __builtin_amdgcn_update_dpp(-1, wave_incl_max(m), 0x138, 0xf, 0xf,
                                                             false);   // wave_shr:1
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int32_t q = 4 * tid + k;
        if (q < tq) s_qb[q] = v[k] > pre ? v[k] : pre;
      }
    }
  }
  __syncthreads();

  // ---- entries: drop padding and blocks past lk, flag bad ids and pages, count
  int32_t slot_k[kFusedItems], arr_k[kFusedItems];
  int64_t col0_k[kFusedItems];                      // first block-table column of the block
  int32_t len_k[kFusedItems];                       // keys of the block's valid range
#pragma unroll
  for (int k = 0; k < kFusedItems; ++k) {
    slot_k[k] = -1;
    arr_k[k] = 0;
    col0_k[k] = 0;
    len_k[k] = 0;
    if (k >= nk_wave) continue;
    const int32_t i = tid + kFusedThreads * k;
    if (i >= items) continue;
    const int32_t q = i / topk, r = i - q * topk;
    const int64_t idx = ((int64_t)q * hkv + h) * topk + r;
    const int32_t v = v_k[k];
    if (v == -1) continue;
    if (v < -1 || v >= A.msb) {
      atomicMin(&s_err, err_key(kRankSelected, (uint64_t)idx));
      continue;
    }
    const int32_t b = s_qb[q];
    if (b < 0) continue;                              // only with a cu error
    const int64_t lk = s_lkb[b];
    const int64_t block_start = (int64_t)v * A.block_size;
    if (block_start >= lk) continue;
    const int64_t block_end = block_start + A.block_size < lk ? block_start + A.block_size : lk;
    slot_k[k] = b * A.msb + v;
    col0_k[k] = (int64_t)b * A.max_pages + (int64_t)v * A.ppb;
    len_k[k] = (int32_t)(block_end - block_start);
  }
  if (A.num_pages >= 0) {
    // The pages each kept block's valid range touches must exist (the
    // forward's block-table check, moved into the build). The reads of all
    // entries go out together, kPageBatch pages of each per round: clamped
    // addresses, no load behind a branch.
    constexpr int kPageBatch = 4;
    int64_t bad_k[kFusedItems];
#pragma unroll
    for (int k = 0; k < kFusedItems; ++k) bad_k[k] = INT64_MAX;
    // (an empty block table has no element to clamp to, and then no entry is kept)
    const int32_t ppb_read = (int64_t)batch * A.max_pages > 0 ? A.ppb : 0;
    for (int32_t p0 = 0; p0 < ppb_read; p0 += kPageBatch) {
      int32_t page[kFusedItems][kPageBatch];
#pragma unroll
      for (int k = 0; k < kFusedItems; ++k) {
        if (k < nk_wave) {
#pragma unroll
          for (int x = 0; x < kPageBatch; ++x) {
            const int32_t pl = p0 + x;
            const bool touched = pl < A.ppb && pl * A.page_size < len_k[k];
            page[k][x] = A.block_tables[touched ? col0_k[k] + pl : 0];
          }
        } else {
#pragma unroll
          for (int x = 0; x < kPageBatch; ++x) page[k][x] = 0;
        }
      }
#pragma unroll
      for (int k = 0; k < kFusedItems; ++k)
#pragma unroll
        for (int x = 0; x < kPageBatch; ++x) {
          const int32_t pl = p0 + x;
          const bool touched = pl < A.ppb && pl * A.page_size < len_k[k];
          if (touched && page[k][x] >= A.num_pages && col0_k[k] + pl < bad_k[k])
            bad_k[k] = col0_k[k] + pl;
        }
    }
#pragma unroll
    for (int k = 0; k < kFusedItems; ++k)
      if (bad_k[k] != INT64_MAX) atomicMin(&s_err, err_key(kRankPage, (uint64_t)bad_k[k]));
  }
#pragma unroll
  for (int k = 0; k < kFusedItems; ++k)
    if (slot_k[k] >= 0) arr_k[k] = atomicAdd(&s_cnt[slot_k[k]], 1);   // arrival order, made stable below
  __syncthreads();

  // ---- one scan over the slots: counts -> exclusive offsets (in place), the
  // compact list of nonempty slots with their unit offsets, head totals
  const int32_t thr_e = (int32_t)(((int64_t)A.mfma_min_rows + A.qhead - 1) / A.qhead);
  const int32_t per = (nslots + kFusedThreads - 1) / kFusedThreads;   // slots [tid*per, +per)
  int32_t e_h, ns_h, uw_h, um_h;
  if (per == 4 && (nslots & 3) == 0) {
    // four slots a thread (decode: 4096 slots): one 16-byte LDS read and
    // write each, the slots' sums kept for the second pass
    const bool have = tid * 4 < nslots;
    const int4 c4 = have ? *reinterpret_cast<const int4*>(&s_cnt[tid * 4]) : make_int4(0, 0, 0, 0);
    const int c[4] = {c4.x, c4.y, c4.z, c4.w};
    uint2 t[4];
    uint2 mine = make_uint2(0u, 0u);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      t[x] = slot_sums(c[x], A, thr_e);
      mine.x += t[x].x;
      mine.y += t[x].y;
    }
    uint32_t ta, tb;
    uint2 run = block_excl_scan2(mine.x, mine.y, s_w2, &ta, &tb);
    e_h = (int32_t)(ta & 0xffffu);
    ns_h = (int32_t)(ta >> 16);
    uw_h = (int32_t)(tb & 0xffffu);
    um_h = (int32_t)(tb >> 16);
    int off[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      off[x] = (int32_t)(run.x & 0xffffu);
      if (c[x] > 0) {
        const int32_t j = (int32_t)(run.x >> 16);
        s_list[j] = tid * 4 + x;
        s_uoff[j] = run.y;
      }
      run.x += t[x].x;
      run.y += t[x].y;
    }
    if (have) *reinterpret_cast<int4*>(&s_cnt[tid * 4]) = make_int4(off[0], off[1], off[2], off[3]);
  } else {
    uint2 mine = make_uint2(0u, 0u);
    for (int32_t x = 0; x < per; ++x) {
      const int32_t sl = tid * per + x;
      const uint2 t = slot_sums(sl < nslots ? s_cnt[sl] : 0, A, thr_e);
      mine.x += t.x;
      mine.y += t.y;
    }
    uint32_t ta, tb;
    uint2 run = block_excl_scan2(mine.x, mine.y, s_w2, &ta, &tb);
    e_h = (int32_t)(ta & 0xffffu);
    ns_h = (int32_t)(ta >> 16);
    uw_h = (int32_t)(tb & 0xffffu);
    um_h = (int32_t)(tb >> 16);
    for (int32_t x = 0; x < per; ++x) {
      const int32_t sl = tid * per + x;
      if (sl >= nslots) break;
      const int32_t c = s_cnt[sl];
      s_cnt[sl] = (int32_t)(run.x & 0xffffu);
      if (c > 0) {
        const int32_t j = (int32_t)(run.x >> 16);
        s_list[j] = sl;
        s_uoff[j] = run.y;
      }
      const uint2 t = slot_sums(c, A, thr_e);
      run.x += t.x;
      run.y += t.y;
    }
  }
  // publish this head's totals (all of its error keys are in by now)
  if (tid == 0) {
    HeadAgg* ag = P.agg + h;
    ag->e = e_h;
    ag->ns = ns_h;
    ag->uw = uw_h;
    ag->um = um_h;
    ag->err = s_err;
    __hip_atomic_store(&ag->flag, A.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();

  // ---- member list of each slot (arrival order)
#pragma unroll
  for (int k = 0; k < kFusedItems; ++k)
    if (slot_k[k] >= 0) s_mem[s_cnt[slot_k[k]] + arr_k[k]] = tid + kFusedThreads * k;
  __syncthreads();

  // ---- head-local outputs, before waiting for the other heads: the rank of
  // each entry in its slot (members with a smaller entry index) gives inv;
  // compact slots and plateaued offsets
  int32_t inv_k[kFusedItems];
#pragma unroll
  for (int k = 0; k < kFusedItems; ++k) {
    const int32_t i = tid + kFusedThreads * k;
    inv_k[k] = -1;
    if (k >= nk_wave || i >= items) continue;
    const int32_t q = i / topk, r = i - q * topk;
    if (slot_k[k] >= 0) {
      const int32_t sl = slot_k[k];
      const int32_t off = s_cnt[sl];
      const int32_t end = sl + 1 < nslots ? s_cnt[sl + 1] : e_h;
      int32_t rank = 0;
      for (int32_t x = off; x < end; ++x) rank += s_mem[x] < i;
      inv_k[k] = off + rank;
    }
    P.inv[((int64_t)h * tq + q) * topk + r] = inv_k[k];
  }
  for (int32_t j = tid; j < ns_h; j += kFusedThreads) {
    const int32_t sl = s_list[j];
    P.sel_slots[(int64_t)h * nbs + j] = sl;
    P.sel_offsets[(int64_t)h * (nbs + 1) + j] = s_cnt[sl];
  }
  for (int64_t j = ns_h + tid; j < nbs; j += kFusedThreads) P.sel_slots[(int64_t)h * nbs + j] = -1;
  for (int64_t j = ns_h + tid; j <= nbs; j += kFusedThreads)
    P.sel_offsets[(int64_t)h * (nbs + 1) + j] = e_h;

  // ---- look-back: totals of the heads before h (all heads for the last one).
  // Thread hh polls head hh's flag, then reads its totals. With at most 64
  // heads before h the pollers are wave 0's lanes and fold the totals with
  // a wave reduction; beyond that, through LDS atomics.
  static_assert(offsetof(HeadAgg, ns) == 8 && offsetof(HeadAgg, um) == 16 &&
                offsetof(HeadAgg, err) == 24, "HeadAgg layout");
  auto read_head = [&](int32_t hh, unsigned long long* e, unsigned long long* ns, int32_t* uw,
                       int32_t* um, unsigned long long* err) -> bool {
    const HeadAgg* ag = P.agg + hh;
    int spins = 0;
    while (__hip_atomic_load(&ag->flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) != A.epoch &&
           spins < kLookbackSpins) {
      __builtin_amdgcn_s_sleep(1);
      ++spins;
    }
    if (spins >= kLookbackSpins) return false;
    // bytes 0..31 of the HeadAgg in two 16-byte loads: w0 = (e lo, e hi, ns, uw),
    // w1 = (um, pad, err lo, err hi)
    const int4 w0 = *reinterpret_cast<const int4*>(ag);
    const int4 w1 = *reinterpret_cast<const int4*>(reinterpret_cast<const char*>(ag) + 16);
    *e = (unsigned long long)(uint32_t)w0.x | ((unsigned long long)(uint32_t)w0.y << 32);
    *err = (unsigned long long)(uint32_t)w1.z | ((unsigned long long)(uint32_t)w1.w << 32);
    *ns = (unsigned long long)w0.z;
    *uw = w0.w;
    *um = w1.x;
    return true;
  };
  if (h <= 64) {
    if (tid < 64) {
      unsigned long long e = 0, ns = 0, err = ~0ull;
      int32_t uw = 0, um = 0;
      if (tid < h && !read_head(tid, &e, &ns, &uw, &um, &err)) {
        e = ns = 0;
        uw = um = 0;
        err = err_key(kRankLookback, 0);
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        e += __shfl_xor(e, off, 64);
        ns += __shfl_xor(ns, off, 64);
        uw += __shfl_xor(uw, off, 64);
        um += __shfl_xor(um, off, 64);
        const unsigned long long o = __shfl_xor(err, off, 64);
        err = o < err ? o : err;
      }
      if (tid == 0) {
        s_base_e = e;
        s_base_ns = ns;
        s_base_uw = uw;
        s_base_um = um;
        atomicMin(&s_err, err);
      }
    }
  } else {
    for (int32_t hh = tid; hh < h; hh += kFusedThreads) {
      unsigned long long e, ns, err;
      int32_t uw, um;
      if (!read_head(hh, &e, &ns, &uw, &um, &err)) {
        atomicMin(&s_err, err_key(kRankLookback, 0));
        continue;
      }
      atomicAdd(&s_base_e, e);
      atomicAdd(&s_base_ns, ns);
      atomicAdd(&s_base_uw, uw);
      atomicAdd(&s_base_um, um);
      atomicMin(&s_err, err);
    }
  }
  __syncthreads();
  const int64_t hb = (int64_t)s_base_e;
  const int32_t uw0 = s_base_uw, um0 = s_base_um;

  // ---- edges in (q, r) order inside each slot
#pragma unroll
  for (int k = 0; k < kFusedItems; ++k) {
    if (inv_k[k] < 0) continue;
    const int32_t i = tid + kFusedThreads * k;
    const int32_t q = i / topk, r = i - q * topk;
    *reinterpret_cast<int2*>(P.edges + 2 * (hb + inv_k[k])) = make_int2(q, r);
  }
  // ---- the slots' units: ceil(c / cap) near-equal parts
  for (int32_t j = tid; j < ns_h; j += kFusedThreads) {
    const int32_t sl = s_list[j];
    const int32_t off = s_cnt[sl];
    const int32_t c = (j + 1 < ns_h ? s_cnt[s_list[j + 1]] : e_h) - off;
    const uint32_t t = slot_sums(c, A, thr_e).y, uo = s_uoff[j];
    const bool is_m = c >= thr_e;
    const int32_t k_units = is_m ? (int32_t)(t >> 16) : (int32_t)(t & 0xffffu);
    Unit* dst = is_m ? P.units_mfma + um0 + (int32_t)(uo >> 16) : P.units_wave + uw0 + (int32_t)(uo & 0xffffu);
    const int32_t b = sl / A.msb, blk = sl - b * A.msb;
    const int32_t e_base = (int32_t)(hb + off);
    const int32_t lk = s_lkb[b], dl = s_dlb[b];
    // part u of k_units spans [u * c / k_units, (u + 1) * c / k_units): c <= 4096
    for (int32_t u = 0; u < k_units; ++u) {
      const int32_t s0 = (u * c) / k_units, s1 = ((u + 1) * c) / k_units;
      dst[u] = Unit{h, j, e_base + s0, e_base + s1, b, blk, lk, dl};
    }
  }
  if (tid == 0) {
    P.num_sel[h] = ns_h;
    P.edge_head_base[h] = hb;
    if (h == hkv - 1) {
      // the last head has looked back over all others: the header
      P.edge_head_base[hkv] = hb + e_h;
      DevHeader* hd = P.hdr;
      hd->what_code = kWhatNone;
      hd->err_expected = 0;
      hd->err_got = 0;
      hd->total_edges = hb + e_h;
      hd->num_units_wave = uw0 + uw_h;
      hd->num_units_mfma = um0 + um_h;
      hd->num_slots = (int64_t)s_base_ns + ns_h;
      P.sort_hist[kSortHistCounter] = 0;           // the unit sort's counter
      hd->geom[0] = (int32_t)A.tq;
      hd->geom[1] = A.hkv;
      hd->geom[2] = A.topk;
      hd->geom[3] = A.batch;
      hd->geom[4] = A.max_pages;
      hd->geom[5] = A.block_size;
      hd->geom[6] = A.page_size;
      hd->geom[7] = A.qhead;
      hd->err_key = s_err;
      set_status(hd, A, s_err);
    }
  }
}

size_t fused_lds_bytes(int64_t tq, int32_t topk, int64_t nbs, int32_t batch) {
  const size_t items = (size_t)tq * topk;
  const size_t nlist = (size_t)nbs < items ? (size_t)nbs : items;
  return 4 * ((size_t)nbs + items + 2 * nlist + (size_t)tq + 2 * (size_t)batch);
}
size_t fused_lds_bytes(const BuildArgs& a) { return fused_lds_bytes(a.tq, a.topk, a.nbs, a.batch); }

bool fused_fits(const BuildArgs& a) {
  return fused_build_fits(a.tq, a.topk, a.nbs, a.batch, a.hkv);
}

inline unsigned grid_for(int64_t n, int per) {
  int64_t g = (n + per - 1) / per;
  return (unsigned)(g < 1 ? 1 : g);
}

// ------------------------------------------------------------ MFMA unit order
// The MFMA units again, largest first (by 32-row tiles; within a bucket in
// any order), for the 32-row forward's static assignment: dealt in a snake
// over the workgroups, a size-sorted list gives every workgroup a near-equal
// share without a queue, and each workgroup knows its next units in advance.
// A counting sort in two launches of up to kSortGrid workgroups: each counts
// its range of units into per-workgroup bucket counts, and the last one to
// finish turns the counts into bucket-major offsets; then each workgroup
// moves its units to their places. (The order inside a bucket may differ
// from run to run; each unit's partials do not depend on where it runs.)
constexpr int kSortThreads = 512;
constexpr int kSortUnitsPerThread = 8;

// Bucket of a unit: group (b * hkv + h) % kSortGroups, then size (32-row
// tiles, bucket 0 of a group the largest).
__device__ inline int unit_bucket(const int4& lo, int32_t b, int32_t hkv, int32_t qhead) {
  const int32_t tiles = ((lo.w - lo.z) * qhead + 31) / 32;   // lo = (h, j, e0, e1)
  const int32_t t = tiles < 1 ? 1 : (tiles > kSortSizes ? kSortSizes : tiles);
  const int grp = (int)(((int64_t)b * hkv + lo.x) & (kSortGroups - 1));
  return grp * kSortSizes + (kSortSizes - t);
}

// units [u0, u1) of workgroup g of the sort's grid
__device__ inline void sort_range(int32_t n, int32_t& u0, int32_t& u1) {
  const int32_t per = (n + (int32_t)gridDim.x - 1) / (int32_t)gridDim.x;
  u0 = (int32_t)blockIdx.x * per;
  u1 = u0 + per < n ? u0 + per : n;
}

// Counts per (bucket, workgroup), bucket-major with the grid's size (a
// multiple of 4) as the stride. The last workgroup to finish chooses the
// list's order and turns the counts into offsets, thread x for bucket x:
// by group, then size within a group, when every group holds within 10% of
// an even share of the tiles (each XCD then takes one group, so its L2
// serves the q rows of an eighth of the (sequence, head) pairs); by size
// alone (the groups of a size together) otherwise.
__global__ __launch_bounds__(kSortThreads) void k_unit_count(IndexPtrs P, BuildArgs A) {
  static_assert(kSortBuckets == kSortThreads && kSortSizes == 64 && kSortGroups == kSortThreads / 64,
                "thread x of the sort holds bucket x: wave w holds group w, lane l its size index l");
  static_assert(kSortGrid % 4 == 0, "a bucket's counts as int4");
  __shared__ int32_t s_cnt[kSortBuckets];
  __shared__ bool s_last;
  if (P.hdr->status != SA_OK) return;            // a failed build: the forward does not run
  const int32_t n = P.hdr->num_units_mfma;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t G = (int32_t)gridDim.x;
  s_cnt[tid] = 0;
  __syncthreads();
  int32_t u0, u1;
  sort_range(n, u0, u1);
  const int4* src = reinterpret_cast<const int4*>(P.units_mfma);    // a unit is two int4: (h, j, e0, e1), (b, ...)
  for (int32_t base = u0; base < u1; base += kSortThreads * kSortUnitsPerThread) {
    int4 lo[kSortUnitsPerThread];
    int32_t bq[kSortUnitsPerThread];
#pragma unroll
    for (int k = 0; k < kSortUnitsPerThread; ++k) {
      const int32_t u = base + k * kSortThreads + tid;
      const int32_t uu = u < u1 ? u : u0;
      lo[k] = src[2 * (int64_t)uu];
      bq[k] = reinterpret_cast<const int32_t*>(src + 2 * (int64_t)uu + 1)[0];
    }
#pragma unroll
    for (int k = 0; k < kSortUnitsPerThread; ++k)
      if (base + k * kSortThreads + tid < u1) atomicAdd(&s_cnt[unit_bucket(lo[k], bq[k], A.hkv, A.qhead)], 1);
  }
  __syncthreads();
  int32_t* hist = P.sort_hist;
  hist[tid * G + blockIdx.x] = s_cnt[tid];
  // the last workgroup to finish orders the list
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const int32_t done = atomicAdd(&hist[kSortHistCounter], 1);
    s_last = done == G - 1;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  __shared__ int32_t s_tot[kSortBuckets], s_base[kSortBuckets], s_wsum[kSortThreads / 64];
  __shared__ int32_t s_gn[kSortGroups];
  __shared__ int64_t s_w[kSortGroups];
  __shared__ int32_t s_grouped;
  // this thread's bucket over the workgroups, in registers
  int4* col = reinterpret_cast<int4*>(hist + tid * G);
  int32_t c[kSortGrid];
#pragma unroll
  for (int q = 0; q < kSortGrid / 4; ++q) {
    const int4 v = 4 * q < G ? col[q] : make_int4(0, 0, 0, 0);
    c[4 * q] = v.x;
    c[4 * q + 1] = v.y;
    c[4 * q + 2] = v.z;
    c[4 * q + 3] = v.w;
  }
  int32_t tot = 0;
#pragma unroll
  for (int g = 0; g < kSortGrid; ++g) tot += c[g];
  s_tot[tid] = tot;
  {
    // this wave's group: its units and tiles
    int32_t un = tot;
    int64_t w = (int64_t)tot * (kSortSizes - lane);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      un += __shfl_xor(un, off, 64);
      w += __shfl_xor(w, off, 64);
    }
    if (lane == 0) {
      s_gn[wave] = un;
      s_w[wave] = w;
    }
  }
  __syncthreads();
  if (tid == 0) {
    int64_t wmax = 0, wsum = 0;
    for (int k = 0; k < kSortGroups; ++k) {
      wmax = s_w[k] > wmax ? s_w[k] : wmax;
      wsum += s_w[k];
    }
    s_grouped = wsum > 0 && 10 * kSortGroups * wmax <= 11 * wsum;
  }
  __syncthreads();
  const bool grouped = s_grouped != 0;
  // thread o: position o of the list's order, bucket o (group-major) or
  // (o % groups) * sizes + o / groups (size-major); exclusive scan of the
  // totals in that order
  const int32_t bo = grouped ? tid : (tid % kSortGroups) * kSortSizes + tid / kSortGroups;
  const int32_t to = s_tot[bo];
  int32_t incl = to;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int32_t before = 0;
  for (int v = 0; v < wave; ++v) before += s_wsum[v];
  s_base[bo] = before + incl - to;
  __syncthreads();
  // offsets of this thread's bucket: its first place, then the workgroups
  // in order (an empty bucket is never read)
  if (tot != 0) {
    int32_t run = s_base[tid];
#pragma unroll
    for (int q = 0; q < kSortGrid / 4; ++q) {
      if (4 * q < G) {
        int4 v;
        v.x = run;
        run += c[4 * q];
        v.y = run;
        run += c[4 * q + 1];
        v.z = run;
        run += c[4 * q + 2];
        v.w = run;
        run += c[4 * q + 3];
        col[q] = v;
      }
    }
  }
  // for the forward: the order, and each group's first unit
  if (tid == 0) {
    int32_t* info = hist + kSortHistInfo;
    info[0] = grouped ? 1 : 0;
    int32_t o = 0;
    for (int x = 0; x < kSortGroups; ++x) {
      info[1 + x] = o;
      o += s_gn[x];
    }
    info[1 + kSortGroups] = o;
    hist[kSortHistCounter] = 0;                    // the counter, for the next build
  }
}

__global__ __launch_bounds__(kSortThreads) void k_unit_place(IndexPtrs P, BuildArgs A) {
  __shared__ int32_t s_cur[kSortBuckets];
  if (P.hdr->status != SA_OK) return;
  const int32_t n = P.hdr->num_units_mfma;
  const int tid = threadIdx.x;
  const int32_t G = (int32_t)gridDim.x;
  s_cur[tid] = P.sort_hist[tid * G + blockIdx.x];
  __syncthreads();
  int32_t u0, u1;
  sort_range(n, u0, u1);
  // a unit is two 4-int vectors (native vectors: the arrays stay in registers)
  typedef int32_t v4i __attribute__((ext_vector_type(4)));
  const v4i* src = reinterpret_cast<const v4i*>(P.units_mfma);
  v4i* dst = reinterpret_cast<v4i*>(P.units_sorted);
  for (int32_t base = u0; base < u1; base += kSortThreads * kSortUnitsPerThread) {
    v4i lo[kSortUnitsPerThread], hi[kSortUnitsPerThread];
#pragma unroll
    for (int k = 0; k < kSortUnitsPerThread; ++k) {
      const int32_t u = base + k * kSortThreads + tid;
      const int32_t uu = u < u1 ? u : u0;
      lo[k] = src[2 * (int64_t)uu];
      hi[k] = src[2 * (int64_t)uu + 1];
    }
#pragma unroll
    for (int k = 0; k < kSortUnitsPerThread; ++k) {
      if (base + k * kSortThreads + tid < u1) {
        const int4 l = make_int4(lo[k].x, lo[k].y, lo[k].z, lo[k].w);
        const int32_t pos = atomicAdd(&s_cur[unit_bucket(l, hi[k].x, A.hkv, A.qhead)], 1);
        dst[2 * (int64_t)pos] = lo[k];
        dst[2 * (int64_t)pos + 1] = hi[k];
      }
    }
  }
}

}  // namespace

bool fused_build_fits(int64_t tq, int32_t topk, int64_t nbs, int32_t batch, int32_t hkv) {
  return tq * topk <= (int64_t)kFusedThreads * kFusedItems && nbs <= kFusedMaxSlots &&
         tq <= kFusedMaxQ && batch <= kFusedMaxBatch && hkv <= 65535 &&
         fused_lds_bytes(tq, topk, nbs, batch) <= kFusedMaxLds;
}

// The 32-row MFMA forward for head_dim 128 and blocks of 65..128 keys (fp32
// or 16-bit pages) walks the units in size order (the unit sort); other
// geometries do not read that list.
inline bool unit_sort_needed(const sa_index* idx, const BuildArgs& a) {
  return a.mfma_min_rows != INT32_MAX && idx->head_dim == kMfmaHeadDim && a.block_size > 64 &&
         a.block_size <= kMfmaMaxBlock;
}

// The sort's two launches: a workgroup for every kSortThreads *
// kSortUnitsPerThread units, 4 to kSortGrid of them in steps of 4.
inline void launch_unit_sort(const sa_index* idx, const IndexPtrs& P, const BuildArgs& a, hipStream_t s) {
  constexpr int64_t per = (int64_t)kSortThreads * kSortUnitsPerThread;
  int64_t g = (idx->max_units + per - 1) / per;
  g = (g + 3) / 4 * 4;
  g = g < 4 ? 4 : (g > kSortGrid ? kSortGrid : g);
  hipLaunchKernelGGL(k_unit_count, dim3((unsigned)g), dim3(kSortThreads), 0, s, P, a);
  hipLaunchKernelGGL(k_unit_place, dim3((unsigned)g), dim3(kSortThreads), 0, s, P, a);
}

hipError_t launch_build(const sa_index* idx, const BuildArgs& a, hipStream_t s) {
  const IndexPtrs P = index_ptrs(idx);
  // SA_BUILD_MULTIKERNEL=1 keeps small problems on the multi-kernel build
  // (both paths produce the same index; tests cover each).
  const char* force_multi = std::getenv("SA_BUILD_MULTIKERNEL");
  const bool multi = force_multi != nullptr && force_multi[0] == '1';
  if (!multi && fused_fits(a)) {
    // the LDS limit is a per-device attribute of the kernel: set once per device
    static thread_local int attr_dev = -1;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (attr_dev != dev) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_index_fused),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kFusedMaxLds);
      if (e != hipSuccess) return e;
      attr_dev = dev;
    }
    const size_t lds = fused_lds_bytes(a);
    hipLaunchKernelGGL(k_index_fused, dim3((unsigned)a.hkv), dim3(kFusedThreads), lds, s, P, a);
    if (unit_sort_needed(idx, a)) launch_unit_sort(idx, P, a, s);
    return hipGetLastError();
  }
  const int64_t slots = (int64_t)a.hkv * a.nbs;
  int64_t init_grid = ((slots > a.tq ? slots : a.tq) + 255) / 256;
  if (init_grid > 2048) init_grid = 2048;
  if (init_grid < 1) init_grid = 1;
  hipLaunchKernelGGL(k_index_init, dim3((unsigned)init_grid), dim3(256), 0, s, P, a);
  const int64_t entries = a.tq * a.hkv * a.topk;
  // Aggregate per workgroup where one sequence's (h, block) counters fit LDS,
  // slots repeat (4 entries a slot on average) and the chunks fill half the
  // CUs; elsewhere (few entries a slot, as in ragged batches) the LDS pass
  // costs more than the atomics it saves. SA_BUILD_AGG=1 / 0 forces the
  // choice where the counters fit (tests cover both kernels).
  const int64_t nloc = (int64_t)a.hkv * a.msb;
  const bool agg_fits = nloc > 0 && nloc <= kAggMaxSlots;
  bool agg = agg_fits && entries >= 4 * slots && entries >= (int64_t)cu_count() * kAggItems / 2;
  const char* force_agg = std::getenv("SA_BUILD_AGG");
  if (force_agg != nullptr && (force_agg[0] == '0' || force_agg[0] == '1'))
    agg = agg_fits && force_agg[0] == '1';
  if (agg)
    hipLaunchKernelGGL(k_index_hist_agg, dim3(grid_for(entries, kAggItems)), dim3(kAggThreads),
                       (size_t)nloc * 4, s, P, a);
  else
    hipLaunchKernelGGL(k_index_hist, dim3(grid_for(entries, 256)), dim3(256), 0, s, P, a);
  hipLaunchKernelGGL(k_index_scan, dim3((unsigned)(a.hkv * scan_chunks(a.nbs))), dim3(kScanThreads),
                     0, s, P, a);
  if (agg)
    hipLaunchKernelGGL(k_index_scatter_agg, dim3(grid_for(entries, kAggItems)), dim3(kAggThreads),
                       (size_t)nloc * 4, s, P, a);
  else
    hipLaunchKernelGGL(k_index_scatter, dim3(grid_for(entries, 256)), dim3(256), 0, s, P, a);
  // persistent: a few workgroups per CU loop over the nonempty slots; large
  // slots rank through an LDS bitmap over their sequence's key range when it
  // fits (the bitmap is sized for the whole tq*topk range, capped)
  BuildArgs ra = a;
  const int64_t words = (a.tq * a.topk + 31) / 32;   // no sequence has more keys
  ra.rank_bitmap_words = words <= kRankBitmapMaxWords ? (int32_t)words : kRankBitmapMaxWords;
  unsigned rank_grid = grid_for(slots, 4);
  if (rank_grid > 8 * cu_count()) rank_grid = 8 * cu_count();
  hipLaunchKernelGGL(k_index_rank, dim3(rank_grid), dim3(256), (size_t)ra.rank_bitmap_words * 4, s,
                     P, ra);
  if (unit_sort_needed(idx, a)) launch_unit_sort(idx, P, a, s);
  return hipGetLastError();
}

}  // namespace sa
