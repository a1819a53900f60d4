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
// Data movement, per key chunk of KC keys:
//  * K and V rows are gathered through the block table with 128-bit loads.
//    Thread t owns float4 column c4 = t % D4P of keys i*KS + t/D4P (KS =
//    256/D4P key slots), so every load instruction reads whole rows.
//  * Scores: each thread forms NI*4 partial dot products (NI keys x 4 rows)
//    over its column, then a transpose-reduce across the D4P lanes of its
//    key slot leaves each lane with finished scores, written to LDS.
//  * Softmax: wave w owns row w of the current 4-row group; it applies the
//    validity and causal masks, keeps the running (m, l) in base 2 (the
//    scale carries log2 e), writes p = exp2(s - m) back and the rescale
//    factor of the running output.
//  * PV: each thread accumulates p * v over its keys for 4 rows, a lane
//    butterfly and an LDS sum across waves finish the reduction, and the
//    running output rows (up to 32 per pass) live in LDS.
#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kRowsPerGroup = 4;     // one row per wave
constexpr int kRowsPerPass = 32;     // running output rows kept in LDS
constexpr float kLn2 = 0.69314718055994530942f;

__device__ inline float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ inline float dot4(float4 a, float4 b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}
__device__ inline float4 fma4(float s, float4 v, float4 a) {
  return make_float4(fmaf(s, v.x, a.x), fmaf(s, v.y, a.y), fmaf(s, v.z, a.z), fmaf(s, v.w, a.w));
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
  static constexpr int KS = 256 / D4P;              // key slots per chunk step
  static constexpr int KC = NI * KS;                // keys per chunk (<= 256)
  static constexpr int NV = NI * kRowsPerGroup;     // partial dots per thread
  static constexpr int S = ilog2(D4P);              // butterfly stages inside a key slot
};

template <int D4P>
__global__ __launch_bounds__(256) void k_fwd_wave(IndexPtrs P, FwdArgs A) {
  using C = WaveCfg<D4P>;
  constexpr int NI = C::NI, KS = C::KS, KC = C::KC, NV = C::NV, S = C::S;

  __shared__ float s_sc[kRowsPerGroup][KC];              // scores, then probabilities
  __shared__ int s_kvalid[KC];
  __shared__ float4 s_red[4][kRowsPerGroup][D4P];
  __shared__ float4 s_o[kRowsPerPass][D4P];
  __shared__ float s_m[kRowsPerPass], s_l[kRowsPerPass], s_alpha[kRowsPerGroup];

  const DevHeader* hdr = P.hdr;
  if (hdr->status != SA_OK) return;
  const int32_t num_units = hdr->num_units_wave;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int c4 = tid % D4P;          // float4 column
  const int ks = tid / D4P;          // key slot
  const int D = A.head_dim, D4 = D >> 2;
  const bool col_ok = c4 < D4;
  const int32_t qhead = A.qhead;

  for (int32_t u = blockIdx.x; u < num_units; u += gridDim.x) {
    const int4 unit = P.units_wave[u];
    const int32_t h = unit.x, j = unit.y, e0 = unit.z, e1 = unit.w;
    const int32_t raw = P.sel_slots[(int64_t)h * A.nbs + j];
    const int32_t b = raw / A.msb, blk = raw % A.msb;
    const int64_t lk = kv_len_dev(A.used, b, A.msb, A.block_size);
    const int64_t block_start = (int64_t)blk * A.block_size;
    int64_t block_end = block_start + A.block_size;
    block_end = block_end < lk ? block_end : lk;
    const int32_t rows = (e1 - e0) * qhead;
    const int64_t row0 = (int64_t)e0 * qhead;                 // first partial row
    const int64_t q_start = A.cu[b];
    const int64_t qo_len = A.cu[b + 1] - q_start;
    const int32_t nkeys = block_end > block_start ? (int32_t)(block_end - block_start) : 0;
    const int64_t bt_row = (int64_t)b * A.max_pages + (int64_t)blk * A.ppb;

    for (int32_t pass0 = 0; pass0 < rows; pass0 += kRowsPerPass) {
      const int32_t prow = rows - pass0 < kRowsPerPass ? rows - pass0 : kRowsPerPass;
      __syncthreads();                                        // previous pass fully stored
      for (int x = tid; x < kRowsPerPass * D4P; x += 256)
        s_o[x / D4P][x % D4P] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (tid < kRowsPerPass) {
        s_m[tid] = -INFINITY;
        s_l[tid] = 0.f;
      }

      for (int32_t cp = 0; cp < nkeys; cp += KC) {
        // ---- gather the chunk's K and V rows (zero for invalid keys)
        float4 kr[NI], vr[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int32_t kk = i * KS + ks;
          const int32_t tb = cp + kk;                         // block-local position
          bool valid = tb < nkeys;
          int64_t off = 0;
          if (valid) {
            const int32_t page = A.block_tables[bt_row + tb / A.page_size];
            valid = page >= 0 && page < A.num_pages;
            off = (((int64_t)page * A.hkv + h) * A.page_size + tb % A.page_size) * D + c4 * 4;
          }
          if (c4 == 0) s_kvalid[kk] = valid;
          kr[i] = (valid && col_ok) ? ld4(A.k + off) : make_float4(0.f, 0.f, 0.f, 0.f);
          vr[i] = (valid && col_ok) ? ld4(A.v + off) : make_float4(0.f, 0.f, 0.f, 0.f);
        }

        for (int32_t g0 = 0; g0 < prow; g0 += kRowsPerGroup) {
          // ---- q of the group's 4 rows, this thread's column
          float4 qr[kRowsPerGroup];
#pragma unroll
          for (int r = 0; r < kRowsPerGroup; ++r) {
            const int32_t ur = pass0 + g0 + r;
            qr[r] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (ur < rows && col_ok) {
              const int32_t e = e0 + ur / qhead, qh = ur % qhead;
              const int64_t qi = P.edges[2 * (int64_t)e];
              qr[r] = ld4(A.q + ((qi * A.hq + (int64_t)h * qhead + qh) * D) + c4 * 4);
            }
          }
          float vals[NV];
#pragma unroll
          for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int r = 0; r < kRowsPerGroup; ++r) vals[i * kRowsPerGroup + r] = dot4(qr[r], kr[i]);
          // ---- transpose-reduce across the D4P lanes of the key slot
          int base = 0;
#pragma unroll
          for (int st = 0; st < S; ++st) {
            const int n = (NV >> st) > 1 ? (NV >> st) : 1;
            const bool hi = (lane >> st) & 1;
            if (n > 1) {
              const int half = n >> 1;
#pragma unroll
              for (int x = 0; x < half; ++x) {
                const float send = hi ? vals[x] : vals[x + half];
                const float keep = hi ? vals[x + half] : vals[x];
                vals[x] = keep + __shfl_xor(send, 1 << st, 64);
              }
              base += hi ? half : 0;
            } else {
              vals[0] += __shfl_xor(vals[0], 1 << st, 64);
            }
          }
          constexpr int NF = (NV >> S) > 1 ? (NV >> S) : 1;
          __syncthreads();                                    // s_sc / s_red free again
          // With D4P > NV the last stages are plain butterflies and lane pairs
          // hold the same sums; only the lower lane of each pair writes.
          const bool writer = (S <= ilog2(NV)) || ((lane >> ilog2(NV)) & ((D4P >> ilog2(NV)) - 1)) == 0;
          if (writer) {
#pragma unroll
            for (int x = 0; x < NF; ++x) {
              const int idx = base + x;
              s_sc[idx % kRowsPerGroup][(idx / kRowsPerGroup) * KS + ks] = vals[x];
            }
          }
          __syncthreads();
          // ---- softmax update: wave wid owns row g0 + wid
          {
            const int32_t lr = g0 + wid;                      // row within the pass
            const int32_t ur = pass0 + lr;
            if (ur < rows) {
              int64_t limit = INT64_MAX;
              if (A.causal) {
                const int32_t e = e0 + ur / qhead;
                const int64_t q_local = (int64_t)P.edges[2 * (int64_t)e] - q_start;
                limit = lk >= qo_len ? lk - qo_len + q_local : q_local;
              }
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
            } else if (lane == 0) {
              s_alpha[wid] = 0.f;
            }
            if (ur >= rows) {
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
            for (int r = 0; r < kRowsPerGroup; ++r) {
              const float4 o = shfl_xor4(acc[r], m);
              acc[r] = make_float4(acc[r].x + o.x, acc[r].y + o.y, acc[r].z + o.z, acc[r].w + o.w);
            }
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
              for (int w = 1; w < 4; ++w) {
                const float4 o = s_red[w][r][c];
                sum = make_float4(sum.x + o.x, sum.y + o.y, sum.z + o.z, sum.w + o.w);
              }
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
    }
  }
}

template <int D4P>
hipError_t launch_wave_t(const IndexPtrs& P, const FwdArgs& a, hipStream_t s, unsigned grid) {
  hipLaunchKernelGGL(k_fwd_wave<D4P>, dim3(grid), dim3(256), 0, s, P, a);
  return hipGetLastError();
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
