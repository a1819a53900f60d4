// Index build on the GPU: the KV-outer CSR index of types.rs (alice-llm
// 2.0.0, KvOuterIndex field docs) plus the work units that the forward walks.
//
//   k_index_init     zero the per-slot counters, reset the header, check
//                    cu_seqlens, and resolve (sequence, kv length) per query
//   k_index_hist     one thread per (q, h, r): drop padding / past-lk ranks,
//                    flag ids outside [-1, msb), check the block's touched
//                    page ids, count edges per (h, raw slot)
//   k_index_scan     one workgroup per head: exclusive scans of the counts,
//                    compaction of nonempty slots, plateaued offsets, unit
//                    counts per slot
//   k_index_scatter  one thread per kept (q, h, r): atomic cursor per slot,
//                    key q*topk + r into the slot's segment (unordered)
//   k_index_rank     per compact slot: rank of each key inside the segment
//                    (keys are unique) -> edges and inv in (q, r) order, then
//                    the slot's work units; workgroup 0 fills the header
#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kScanThreads = 1024;
constexpr int kScanItems = 4;

__device__ inline int4 add4(int4 a, int4 b) {
  return make_int4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}
__device__ inline int4 sub4(int4 a, int4 b) {
  return make_int4(a.x - b.x, a.y - b.y, a.z - b.z, a.w - b.w);
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

// Units of a slot with c edges. A slot with at least thr_e edges (rows >=
// the MFMA minimum) becomes ceil(c / cap) MFMA units; a smaller one becomes
// ceil(c / wave_cap) wavefront units. Part i of k spans
// [floor(i*c/k), floor((i+1)*c/k)), so the parts of a slot are near-equal.
__device__ inline void unit_split(int c, int cap, int wave_cap, int thr_e, int* n_wave,
                                  int* n_mfma) {
  *n_wave = 0;
  *n_mfma = 0;
  if (c <= 0) return;
  if (c >= thr_e) *n_mfma = (c + cap - 1) / cap;
  else *n_wave = (c + wave_cap - 1) / wave_cap;
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
    h->queue_mfma = 0;
    h->done_mfma = 0;
    h->queue_wave = 0;
    h->done_wave = 0;
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
__global__ __launch_bounds__(256) void k_index_hist(IndexPtrs P, BuildArgs A) {
  const int64_t total = A.tq * A.hkv * A.topk;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int32_t r = (int32_t)(idx % A.topk);
  const int64_t qh = idx / A.topk;
  const int32_t h = (int32_t)(qh % A.hkv);
  const int64_t q = qh / A.hkv;
  const int32_t v = A.selected[idx];
  const int2 qi = P.qinfo[q];
  P.inv[((int64_t)h * A.tq + q) * A.topk + r] = -1;
  if (v == -1) return;
  if (v < -1 || v >= A.msb) {
    atomicMin(&P.hdr->err_key, err_key(kRankSelected, (uint64_t)idx));
    return;
  }
  const int32_t b = qi.x;
  const int64_t lk = qi.y;
  const int64_t block_start = (int64_t)v * A.block_size;
  if (block_start >= lk) return;
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
  atomicAdd(&P.cnt[(int64_t)h * A.nbs + (int64_t)b * A.msb + v], 1);
}

__global__ __launch_bounds__(kScanThreads) void k_index_scan(IndexPtrs P, BuildArgs A) {
  const int32_t h = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  __shared__ int4 s_wave[kScanThreads / 64];
  __shared__ int4 s_carry;
  if (tid == 0) s_carry = make_int4(0, 0, 0, 0);
  __syncthreads();
  const int64_t nbs = A.nbs;
  int32_t* cnt = P.cnt + (int64_t)h * nbs;
  const int cap = A.cap_edges;
  const int thr_e = (int)(((int64_t)A.mfma_min_rows + A.qhead - 1) / A.qhead);
  for (int64_t base = 0; base < nbs; base += kScanThreads * kScanItems) {
    int c[kScanItems], nw[kScanItems], nm[kScanItems];
    int4 mine = make_int4(0, 0, 0, 0);    // edges, nonempty slots, wave units, mfma units
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
      const int64_t raw = base + (int64_t)tid * kScanItems + k;
      c[k] = raw < nbs ? cnt[raw] : 0;
    }
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
      unit_split(c[k], cap, A.wave_cap_edges, thr_e, &nw[k], &nm[k]);
      mine = add4(mine, make_int4(c[k], c[k] > 0, nw[k], nm[k]));
    }
    const int4 incl = wave_incl_scan4(mine);
    if (lane == 63) s_wave[wid] = incl;
    __syncthreads();
    if (wid == 0) {
      int4 w = lane < kScanThreads / 64 ? s_wave[lane] : make_int4(0, 0, 0, 0);
      w = wave_incl_scan4(w);
      if (lane < kScanThreads / 64) s_wave[lane] = w;
    }
    __syncthreads();
    const int4 carry = s_carry;
    int4 run = add4(carry, sub4(incl, mine));
    if (wid > 0) run = add4(run, s_wave[wid - 1]);
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
      const int64_t raw = base + (int64_t)tid * kScanItems + k;
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
    __syncthreads();
    if (tid == 0) s_carry = add4(carry, s_wave[kScanThreads / 64 - 1]);
    __syncthreads();
  }
  const int4 tot = s_carry;
  if (tid == 0) {
    P.num_sel[h] = tot.y;
    P.head_e[h] = tot.x;
    P.head_uw[h] = tot.z;
    P.head_um[h] = tot.w;
  }
  for (int64_t j = tot.y + tid; j < nbs; j += kScanThreads) P.sel_slots[(int64_t)h * nbs + j] = -1;
  for (int64_t j = tot.y + tid; j <= nbs; j += kScanThreads)
    P.sel_offsets[(int64_t)h * (nbs + 1) + j] = tot.x;
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
  const unsigned long long key = hd->err_key;
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
  } else {
    hd->status = SA_ERR_SHAPE;
    hd->what_code = kWhatPageId;
    hd->err_expected = A.num_pages;
    hd->err_got = A.block_tables[pos];
  }
}

constexpr int kRankChunk = 2048;   // keys staged in LDS per pass
constexpr int kRankKeys = 4;       // keys held per thread per pass

__device__ inline void write_edge(const IndexPtrs& P, const BuildArgs& A, int32_t h,
                                  int64_t head_base, int32_t off0, int32_t key, int32_t rank) {
  const int32_t q = key / A.topk, r = key % A.topk;
  const int64_t e = head_base + off0 + rank;
  *reinterpret_cast<int2*>(P.edges + 2 * e) = make_int2(q, r);
  P.inv[((int64_t)h * A.tq + q) * A.topk + r] = off0 + rank;
}

struct SlotInfo {
  int32_t n, h, j, off0, uw, um, b, blk, lk, delta;
  int64_t base;
};

// Each workgroup owns 4 consecutive compact-slot ids g = 4*blockIdx + wave
// over all heads (h = g / nbs, j = g % nbs). Slots with <= 64 keys are ranked
// by their wave with lane shuffles. If any of the 4 has more, the whole
// workgroup ranks them one after another through LDS.
__global__ __launch_bounds__(256) void k_index_rank(IndexPtrs P, BuildArgs A) {
  if (blockIdx.x == 0 && threadIdx.x == 0) finalize_header(P, A);
  if (A.nbs == 0) return;                          // no slots at all (msb == 0)
  __shared__ SlotInfo s_slot[4];
  __shared__ __align__(16) int32_t s_keys[kRankChunk];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t g = (int64_t)blockIdx.x * 4 + w;
  if (lane == 0) {
    SlotInfo si{};
    const int32_t h = (int32_t)(g / A.nbs);
    const int64_t j = g % A.nbs;
    if (h < A.hkv) {
      // all loads independent of each other
      const int32_t nsel = P.num_sel[h];
      const int32_t o0 = P.sel_offsets[(int64_t)h * (A.nbs + 1) + j];
      const int32_t o1 = P.sel_offsets[(int64_t)h * (A.nbs + 1) + j + 1];
      const int32_t raw = P.sel_slots[(int64_t)h * A.nbs + j];
      int32_t uw = P.slot_uw[(int64_t)h * A.nbs + j], um = P.slot_um[(int64_t)h * A.nbs + j];
      int64_t hb = 0;
      for (int32_t i = 0; i < h; ++i) {
        hb += P.head_e[i];
        uw += P.head_uw[i];
        um += P.head_um[i];
      }
      if (j < nsel) {
        si.n = o1 - o0;
        si.off0 = o0;
        si.base = hb;
        si.uw = uw;
        si.um = um;
        si.b = raw / A.msb;
        si.blk = raw % A.msb;
        const int64_t q0 = A.cu[si.b], qo_len = A.cu[si.b + 1] - q0;
        const int64_t lk = kv_len_dev(A.used, si.b, A.msb, A.block_size);
        si.lk = (int32_t)lk;
        si.delta = (int32_t)((lk >= qo_len ? lk - qo_len : 0) - q0);
      }
    }
    si.h = h;
    si.j = (int32_t)j;
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
  if (si.n == 0) return;
  const int32_t thr_e = (int32_t)(((int64_t)A.mfma_min_rows + A.qhead - 1) / A.qhead);
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

inline unsigned grid_for(int64_t n, int per) {
  int64_t g = (n + per - 1) / per;
  return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_build(const sa_index* idx, const BuildArgs& a, hipStream_t s) {
  const IndexPtrs P = index_ptrs(idx);
  const int64_t slots = (int64_t)a.hkv * a.nbs;
  int64_t init_grid = ((slots > a.tq ? slots : a.tq) + 255) / 256;
  if (init_grid > 2048) init_grid = 2048;
  if (init_grid < 1) init_grid = 1;
  hipLaunchKernelGGL(k_index_init, dim3((unsigned)init_grid), dim3(256), 0, s, P, a);
  const int64_t entries = a.tq * a.hkv * a.topk;
  hipLaunchKernelGGL(k_index_hist, dim3(grid_for(entries, 256)), dim3(256), 0, s, P, a);
  hipLaunchKernelGGL(k_index_scan, dim3((unsigned)a.hkv), dim3(kScanThreads), 0, s, P, a);
  hipLaunchKernelGGL(k_index_scatter, dim3(grid_for(entries, 256)), dim3(256), 0, s, P, a);
  hipLaunchKernelGGL(k_index_rank, dim3(grid_for(slots, 4)), dim3(256), 0, s, P, a);
  return hipGetLastError();
}

}  // namespace sa
