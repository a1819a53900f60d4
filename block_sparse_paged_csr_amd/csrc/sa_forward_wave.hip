// KV-outer forward, wavefront-reduction path (units with few rows).
//
// One workgroup (4 waves) processes one work unit at a time: a KV block
// (b, blk) of head h and the unit's edges e0..e1, each with qhead GQA lanes
// ("rows"). It computes, per row, the partial (o, m, l) of alice-llm 2.0.0
// forward.rs process_work_unit:
//   s_t = dot(q, k_t) * scale over the block's positions with a page >= 0 and
//   t < min((blk+1)*bs, lk_b), causally alive positions only; m = max s;
//   l = sum exp(s - m); o = sum exp(s - m) v_t; nothing alive -> (0, -inf, 0).
//
// Latency: the grid is persistent (a few workgroups per CU, units assigned
// round-robin). While a unit computes, the workgroup already holds the next
// unit's record and loads its query ids and first-chunk page ids, so the
// next unit starts with its K, V and q loads: one dependent round trip.
//
// Data movement, per key chunk of KC keys:
//  * K and V rows are gathered through the block table with 128-bit loads.
//  * Scores: TPK = D4P/NI threads share a key; thread (k, qq) holds the K
//    float4 columns qq + TPK*j (j < NI), so one load instruction reads
//    TPK*16 contiguous bytes per key. It forms 4 partial dots against q rows
//    read from LDS (broadcast), and a TPK-lane butterfly finishes them.
//  * V uses the PV layout: thread t owns float4 column c4 = t % D4P of keys
//    i*KS + t/D4P (KS = 256/D4P key slots).
//  * Softmax: wave w owns row w of the current 4-row group; it applies the
//    validity and causal masks, keeps the running (m, l) in base 2 (the
//    scale carries log2 e), writes p = exp2(s - m) back and the rescale
//    factor of the running output.
//  * PV: each thread accumulates p * v over its keys for 4 rows, a lane
//    butterfly and an LDS sum across waves finish the reduction, and the
//    running output rows (up to 16 per pass) live in LDS.
#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kRowsPerGroup = 4;     // one row per wave
constexpr int kRowsPerPass = 16;     // running output rows kept in LDS
constexpr float kLn2 = 0.69314718055994530942f;

__device__ inline float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ inline float dot4(float4 a, float4 b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}
__device__ inline float4 fma4(float s, float4 v, float4 a) {
  return make_float4(fmaf(s, v.x, a.x), fmaf(s, v.y, a.y), fmaf(s, v.z, a.z), fmaf(s, v.w, a.w));
}
__device__ inline float4 add4f(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}
__device__ inline float4 shfl_xor4(float4 v, int m) {
  return make_float4(__shfl_xor(v.x, m, 64), __shfl_xor(v.y, m, 64), __shfl_xor(v.z, m, 64),
                     __shfl_xor(v.w, m, 64));
}
__device__ inline float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}
__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x >> 1); }

template <int D4P>
struct WaveCfg {
  static constexpr int NI = D4P < 8 ? D4P : 8;      // float4 of K (and of V) per thread per chunk
  static constexpr int TPK = D4P / NI;              // threads per key in the score pass
  static constexpr int KC = 256 / TPK;              // keys per chunk (<= 256)
  static constexpr int KS = 256 / D4P;              // key slots of the PV pass
  static constexpr int MAXPG = KC + 1;              // pages one chunk can touch
};

// What a unit's first chunk needs before its K/V loads can be issued: the
// query ids of its first rows and the page ids of its first chunk.
struct Stage {
  int32_t qi;       // thread t < kRowsPerPass: query id of row t (or -1)
  int32_t page;     // thread t < npg: block-table entry of the chunk's page t
  bool ok;          // the page list fitted in one entry per thread
};

template <int D4P, int KVF>
__global__ __launch_bounds__(256) void k_fwd_wave(IndexPtrs P, FwdArgs A) {
  using C = WaveCfg<D4P>;
  constexpr int NI = C::NI, TPK = C::TPK, KC = C::KC, KS = C::KS;

  __shared__ float s_sc[kRowsPerGroup][KC];              // scores, then probabilities
  __shared__ int s_kvalid[KC];
  __shared__ float4 s_red[4][kRowsPerGroup][D4P];
  __shared__ float4 s_o[kRowsPerPass][D4P];
  __shared__ float4 s_q[kRowsPerPass][D4P];
  __shared__ float s_m[kRowsPerPass], s_l[kRowsPerPass], s_alpha[kRowsPerGroup];
  __shared__ int64_t s_qoff[kRowsPerPass];
  __shared__ int32_t s_lim[kRowsPerPass];
  __shared__ int64_t s_pg[C::MAXPG];

  const DevHeader* hdr = P.hdr;
  if (hdr->status != SA_OK) return;
  const int32_t num_units = hdr->num_units_wave;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  // score pass: key kq = tid / TPK, float4 columns qq + TPK*j
  const int kq = tid / TPK, qq = tid % TPK;
  // PV pass: float4 column c4 of keys i*KS + ks
  const int c4 = tid % D4P, ks = tid / D4P;
  const int D = A.head_dim, D4 = D >> 2;
  const bool col_ok = c4 < D4;
  const int32_t qhead = A.qhead;
  const int64_t page_stride = (int64_t)A.hkv * A.page_size * D;

  // Loads of a unit's first rows and first-chunk pages (into registers).
  auto stage_load = [&](const Unit& U) {
    Stage st{-1, -1, true};
    const int32_t rows = (U.e1 - U.e0) * qhead;
    if (tid < kRowsPerPass && tid < rows) st.qi = P.edges[2 * (int64_t)(U.e0 + tid / qhead)];
    const int64_t bstart = (int64_t)U.blk * A.block_size;
    int64_t bend = bstart + A.block_size;
    bend = bend < U.lk ? bend : U.lk;
    const int32_t nk = bend > bstart ? (int32_t)(bend - bstart) : 0;
    if (nk > 0) {
      const int32_t last = (KC < nk ? KC : nk) - 1;
      const int32_t npg = (int32_t)div_magic((uint32_t)last, A.ps_magic) + 1;
      st.ok = npg <= 256;
      if (tid < npg) st.page = A.block_tables[(int64_t)U.b * A.max_pages + (int64_t)U.blk * A.ppb + tid];
    }
    return st;
  };
  // Staged values into LDS for the unit about to run.
  auto stage_store = [&](const Unit& U, const Stage& st) {
    const int32_t rows = (U.e1 - U.e0) * qhead;
    if (tid < kRowsPerPass && tid < rows) {
      s_qoff[tid] = ((int64_t)st.qi * A.hq + (int64_t)U.h * qhead + tid % qhead) * D;
      s_lim[tid] = A.causal ? st.qi + U.delta : INT32_MAX;
    }
    const int64_t head_off = (int64_t)U.h * A.page_size * D;
    if (tid < C::MAXPG)
      s_pg[tid] = (st.page >= 0 && st.page < A.num_pages)
                      ? (int64_t)st.page * page_stride + head_off : -1;
  };

  int32_t u = blockIdx.x;
  Unit cur{};
  bool staged = false;                     // s_qoff / s_lim / s_pg hold cur's first chunk
  if (u < num_units) {
    cur = P.units_wave[u];
    const Stage st = stage_load(cur);
    stage_store(cur, st);
    staged = st.ok;
  }

  while (u < num_units) {
    const int32_t un = u + gridDim.x;
    Unit nxt{};
    if (un < num_units) nxt = P.units_wave[un];          // in flight with cur's loads
    Stage pre{-1, -1, false};
    bool have_pre = false;

    const int32_t h = cur.h, e0 = cur.e0, e1 = cur.e1;
    const int64_t lk = cur.lk;
    const int64_t block_start = (int64_t)cur.blk * A.block_size;
    int64_t block_end = block_start + A.block_size;
    block_end = block_end < lk ? block_end : lk;
    const int32_t rows = (e1 - e0) * qhead;
    const int64_t row0 = (int64_t)e0 * qhead;                 // first partial row
    const int32_t nkeys = block_end > block_start ? (int32_t)(block_end - block_start) : 0;
    const int64_t bt_row = (int64_t)cur.b * A.max_pages + (int64_t)cur.blk * A.ppb;
    const int64_t head_off = (int64_t)h * A.page_size * D;

    for (int32_t pass0 = 0; pass0 < rows; pass0 += kRowsPerPass) {
      const int32_t prow = rows - pass0 < kRowsPerPass ? rows - pass0 : kRowsPerPass;
      if (!staged) {
        // rows of a later pass: query ids fetched now
        __syncthreads();
        if (tid < prow) {
          const int32_t ur = pass0 + tid;
          const int32_t qi = P.edges[2 * (int64_t)(e0 + ur / qhead)];
          s_qoff[tid] = ((int64_t)qi * A.hq + (int64_t)h * qhead + ur % qhead) * D;
          s_lim[tid] = A.causal ? qi + cur.delta : INT32_MAX;
        }
      }
      if (tid < kRowsPerPass) {
        s_m[tid] = -INFINITY;
        s_l[tid] = 0.f;
      }
      for (int x = tid; x < kRowsPerPass * D4P; x += 256)
        s_o[x / D4P][x % D4P] = make_float4(0.f, 0.f, 0.f, 0.f);

      for (int32_t cp = 0; cp < nkeys; cp += KC) {
        const int32_t pg0 = (int32_t)div_magic((uint32_t)cp, A.ps_magic);
        const int32_t last = (cp + KC < nkeys ? cp + KC : nkeys) - 1;
        const int32_t npg = (int32_t)div_magic((uint32_t)last, A.ps_magic) - pg0 + 1;
        if (!(staged && cp == 0 && npg <= 256)) {
          __syncthreads();                                     // s_pg no longer read
          for (int x = tid; x < npg; x += 256) {
            const int32_t page = A.block_tables[bt_row + pg0 + x];
            s_pg[x] = (page >= 0 && page < A.num_pages) ? (int64_t)page * page_stride + head_off : -1;
          }
        }
        __syncthreads();
        // ---- K, V (this chunk) and, on the first chunk, q
        float4 kr[NI], vr[NI];
        {
          const int32_t tb = cp + kq;
          const int32_t pgl = (int32_t)div_magic((uint32_t)tb, A.ps_magic);
          const int64_t base = tb < nkeys ? s_pg[pgl - pg0] : -1;
          const bool valid = base >= 0;
          if (qq == 0) s_kvalid[kq] = valid;
          const int64_t krow = base + (int64_t)(tb - pgl * A.page_size) * D;
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            const int c = qq + TPK * j;
            kr[j] = (valid && c < D4) ? load_kv4<KVF>(A.k, krow + c * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
          }
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int32_t tb = cp + i * KS + ks;
          const int32_t pgl = (int32_t)div_magic((uint32_t)tb, A.ps_magic);
          const int64_t base = tb < nkeys ? s_pg[pgl - pg0] : -1;
          const int64_t off = base + (int64_t)(tb - pgl * A.page_size) * D + c4 * 4;
          vr[i] = (base >= 0 && col_ok) ? load_kv4<KVF>(A.v, off) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        if (cp == 0) {
          for (int x = tid; x < prow * D4P; x += 256) {
            const int r = x / D4P, c = x % D4P;
            s_q[r][c] = c < D4 ? ld4(A.q + s_qoff[r] + c * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
          }
          __syncthreads();
          if (pass0 == 0 && un < num_units) {
            // The next unit's record has arrived with this chunk's loads; its
            // first-chunk loads now overlap this unit's compute.
            pre = stage_load(nxt);
            have_pre = true;
          }
        }

        for (int32_t g0 = 0; g0 < prow; g0 += kRowsPerGroup) {
          // ---- scores of key kq for the group's 4 rows, reduced over TPK lanes
          float sc[kRowsPerGroup];
#pragma unroll
          for (int r = 0; r < kRowsPerGroup; ++r) {
            float acc = 0.f;
            if (g0 + r < prow) {
#pragma unroll
              for (int j = 0; j < NI; ++j) acc += dot4(s_q[g0 + r][qq + TPK * j], kr[j]);
            }
            sc[r] = acc;
            // one q row live at a time: keeps the K and V registers resident
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int m = 1; m < TPK; m <<= 1)
#pragma unroll
            for (int r = 0; r < kRowsPerGroup; ++r) sc[r] += __shfl_xor(sc[r], m, 64);
          if (g0 > 0) __syncthreads();                        // s_sc / s_red free again
          if (qq == 0) {
#pragma unroll
            for (int r = 0; r < kRowsPerGroup; ++r) s_sc[r][kq] = sc[r];
          }
          __syncthreads();
          // ---- softmax update: wave wid owns row g0 + wid
          {
            const int32_t lr = g0 + wid;                      // row within the pass
            if (lr < prow) {
              const int64_t limit = s_lim[lr];
              float mc = -INFINITY;
              for (int kk = lane; kk < KC; kk += 64) {
                const int64_t t = block_start + cp + kk;
                const bool alive = s_kvalid[kk] && t <= limit;
                const float s = alive ? s_sc[wid][kk] * A.scale_log2 : -INFINITY;
                s_sc[wid][kk] = s;
                mc = fmaxf(mc, s);
              }
              mc = wave_max(mc);
              const float m_old = s_m[lr];
              const float m_new = fmaxf(m_old, mc);
              float lc = 0.f;
              for (int kk = lane; kk < KC; kk += 64) {
                const float s = s_sc[wid][kk];
                const float p = (s == -INFINITY) ? 0.f : exp2f(s - m_new);
                s_sc[wid][kk] = p;
                lc += p;
              }
              lc = wave_sum(lc);
              const float alpha = (m_old == -INFINITY) ? 0.f : exp2f(m_old - m_new);
              if (lane == 0) {
                s_m[lr] = m_new;
                s_l[lr] = s_l[lr] * alpha + lc;
                s_alpha[wid] = alpha;
              }
            } else {
              if (lane == 0) s_alpha[wid] = 0.f;
              for (int kk = lane; kk < KC; kk += 64) s_sc[wid][kk] = 0.f;
            }
          }
          __syncthreads();
          // ---- PV over this thread's keys, 4 rows
          float4 acc[kRowsPerGroup];
#pragma unroll
          for (int r = 0; r < kRowsPerGroup; ++r) acc[r] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
          for (int i = 0; i < NI; ++i) {
            const int kk = i * KS + ks;
#pragma unroll
            for (int r = 0; r < kRowsPerGroup; ++r) acc[r] = fma4(s_sc[r][kk], vr[i], acc[r]);
          }
#pragma unroll
          for (int m = D4P; m < 64; m <<= 1)
#pragma unroll
            for (int r = 0; r < kRowsPerGroup; ++r) acc[r] = add4f(acc[r], shfl_xor4(acc[r], m));
          if (lane < D4P) {
#pragma unroll
            for (int r = 0; r < kRowsPerGroup; ++r) s_red[wid][r][lane] = acc[r];
          }
          __syncthreads();
          if (tid < kRowsPerGroup * D4P) {
            const int r = tid / D4P, c = tid % D4P;
            const int32_t lr = g0 + r;
            if (lr < prow) {
              float4 sum = s_red[0][r][c];
#pragma unroll
              for (int w = 1; w < 4; ++w) sum = add4f(sum, s_red[w][r][c]);
              const float a = s_alpha[r];
              const float4 prev = s_o[lr][c];
              s_o[lr][c] = make_float4(fmaf(prev.x, a, sum.x), fmaf(prev.y, a, sum.y),
                                       fmaf(prev.z, a, sum.z), fmaf(prev.w, a, sum.w));
            }
          }
        }
      }
      __syncthreads();
      // ---- store the pass's rows: (o, m, l) with m back in natural-log units
      for (int x = tid; x < prow * D4; x += 256) {
        const int r = x / D4, c = x % D4;
        *reinterpret_cast<float4*>(A.o + (row0 + pass0 + r) * D + c * 4) = s_o[r][c];
      }
      if (tid < prow) {
        const float m2 = s_m[tid];
        A.m[row0 + pass0 + tid] = (m2 == -INFINITY) ? -INFINITY : m2 * kLn2;
        A.l[row0 + pass0 + tid] = s_l[tid];
      }
      staged = false;
    }
    // ---- hand over to the next unit
    __syncthreads();                                          // all LDS reads of cur done
    if (un < num_units) {
      if (!have_pre) pre = stage_load(nxt);                   // cur had no keys or rows
      stage_store(nxt, pre);
      staged = pre.ok;
    }
    cur = nxt;
    u = un;
  }
}

template <int D4P, int KVF>
hipError_t launch_wave_kv(const IndexPtrs& P, const FwdArgs& a, hipStream_t s, unsigned max_grid) {
  // Persistent grid: as many workgroups as fit on the device at once.
  static thread_local int per_cu = 0;
  if (per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_fwd_wave<D4P, KVF>, 256, 0) != hipSuccess || n < 1)
      n = 1;
    per_cu = n;
  }
  unsigned grid = (unsigned)per_cu * cu_count();
  if (grid > max_grid) grid = max_grid;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((k_fwd_wave<D4P, KVF>), dim3(grid), dim3(256), 0, s, P, a);
  return hipGetLastError();
}

template <int D4P>
hipError_t launch_wave_t(const IndexPtrs& P, const FwdArgs& a, hipStream_t s, unsigned max_grid) {
  switch (a.kv_format) {
    case SA_KV_BF16: return launch_wave_kv<D4P, SA_KV_BF16>(P, a, s, max_grid);
    case SA_KV_F16: return launch_wave_kv<D4P, SA_KV_F16>(P, a, s, max_grid);
    default: return launch_wave_kv<D4P, SA_KV_F32>(P, a, s, max_grid);
  }
}

}  // namespace

hipError_t launch_forward_wave(const sa_index* idx, const FwdArgs& a, hipStream_t s,
                               unsigned grid) {
  const IndexPtrs P = index_ptrs(idx);
  const int d4 = a.head_dim / 4;
  if (d4 <= 1) return launch_wave_t<1>(P, a, s, grid);
  if (d4 <= 2) return launch_wave_t<2>(P, a, s, grid);
  if (d4 <= 4) return launch_wave_t<4>(P, a, s, grid);
  if (d4 <= 8) return launch_wave_t<8>(P, a, s, grid);
  if (d4 <= 16) return launch_wave_t<16>(P, a, s, grid);
  if (d4 <= 32) return launch_wave_t<32>(P, a, s, grid);
  return launch_wave_t<64>(P, a, s, grid);
}

}  // namespace sa
