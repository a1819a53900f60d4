// KV-outer forward for small units: head_dim 128, blocks of at most 64 keys,
// at most 16 rows (edges * qhead) per unit. This covers decode-style batches,
// where each selected block serves one query or a few.
//
// Per unit it computes the partials (o, m, l) of alice-llm 2.0.0 forward.rs
// process_work_unit over the block's valid, causally alive positions, like the
// other forward kernels.
//
// One workgroup of 4 waves per unit. Wave w owns keys 16w..16w+15 of the block,
// and the unit's (up to) 16 rows form one 16x16 tile on fp32 matrix cores
// (v_mfma_f32_16x16x4f32):
//   S^T[key, row] = K[key, :] . Q[row, :]   lane group g = lane/16 takes d = 32g..32g+31
//   O^T[d, row] += V[key, d] * P[row, key]  output row i of an MFMA block stands for
//                                           d = 8*i + db, so a lane's V reads and O
//                                           writes are contiguous
// Each wave then holds a partial (o, m, l) over its 16 keys. The four are
// merged with the log-sum-exp rule through LDS, so no lane reduction crosses
// waves until the end.
//
// Latency: workgroups are persistent (units round-robin) and pipelined over
// three stages. While unit u computes, the block-table entries and query ids
// of unit u+G and the record of unit u+2G are in flight. Unit u+G therefore
// starts with its K, V and q loads, one round trip.
#include "sa_internal.h"

namespace sa {

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxKeys = 64;        // block_size <= 64
constexpr int kRows = 16;           // rows per unit
constexpr int kMaxPages = 64;       // block_size / page_size <= 64
constexpr float kLn2 = 0.69314718055994530942f;

// What a unit needs before its K/V/q loads: its record, page offsets
// (element offset of page slot pl for head h, or -1) and query ids per row.
struct Meta {
  int32_t rec[8];                   // a Unit
  int64_t pg[kMaxPages];
  int32_t qi[kRows];
};

__device__ inline Unit as_unit(const int32_t* r) {
  return Unit{r[0], r[1], r[2], r[3], r[4], r[5], r[6], r[7]};
}
__device__ inline floatx4 zero4() {
  floatx4 z;
  z[0] = z[1] = z[2] = z[3] = 0.f;
  return z;
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void k_fwd_small(IndexPtrs P, FwdArgs A) {
  __shared__ Meta s_meta[2];
  __shared__ __align__(16) float s_ow[kWaves][kRows][kD];   // per-wave partial o
  __shared__ float s_mw[kWaves][kRows], s_lw[kWaves][kRows];

  const DevHeader* hdr = P.hdr;
  if (hdr->status != SA_OK) return;
  const int32_t num_units = hdr->num_units_wave;
  const int32_t G = gridDim.x;
  int32_t u = blockIdx.x;
  if (u >= num_units) return;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, g = lane >> 4;
  const int32_t qhead = A.qhead;
  const int64_t page_stride = (int64_t)A.hkv * A.page_size * kD;
  const int32_t* units = reinterpret_cast<const int32_t*>(P.units_wave);

  // page offsets of a unit, one per thread t < ppb
  auto page_off = [&](const Unit& U, int t) -> int64_t {
    const int32_t page = A.block_tables[(int64_t)U.b * A.max_pages + (int64_t)U.blk * A.ppb + t];
    return (page >= 0 && page < A.num_pages)
               ? (int64_t)page * page_stride + (int64_t)U.h * A.page_size * kD : -1;
  };
  auto query_of = [&](const Unit& U, int r) -> int32_t {
    return P.edges[2 * (int64_t)(U.e0 + r / qhead)];
  };

  // ---- prologue: unit u staged in slot 0, record of u + G in slot 1
  int cur = 0;
  {
    if (tid < 8) s_meta[0].rec[tid] = units[8 * (int64_t)u + tid];
    if (tid < 8 && u + G < num_units) s_meta[1].rec[tid] = units[8 * (int64_t)(u + G) + tid];
    __syncthreads();
    const Unit U = as_unit(s_meta[0].rec);
    if (tid < A.ppb) s_meta[0].pg[tid] = page_off(U, tid);
    if (tid < kRows && tid < (U.e1 - U.e0) * qhead) s_meta[0].qi[tid] = query_of(U, tid);
    __syncthreads();
  }

  while (true) {
    const Meta& M = s_meta[cur];
    const Unit U = as_unit(M.rec);
    const int32_t rows = (U.e1 - U.e0) * qhead;
    const int64_t row0 = (int64_t)U.e0 * qhead;
    const int64_t block_start = (int64_t)U.blk * A.block_size;
    int64_t block_end = block_start + A.block_size;
    block_end = block_end < U.lk ? block_end : (int64_t)U.lk;
    const int32_t nkeys = block_end > block_start ? (int32_t)(block_end - block_start) : 0;

    // ---- K (this wave's 16 keys, d = 32g..32g+31) and V (keys 16w+4g+r, d = 8li..8li+7)
    float4 kr[8];
    {
      const int32_t key = 16 * w + li;
      int64_t base = -1;
      if (key < nkeys) {
        const int32_t pl = (int32_t)div_magic((uint32_t)key, A.ps_magic);
        base = M.pg[pl];
        if (base >= 0) base += (int64_t)(key - pl * A.page_size) * kD;
      }
      const float* kp = A.k + base + 32 * g;
#pragma unroll
      for (int t = 0; t < 8; ++t)
        kr[t] = base >= 0 ? *reinterpret_cast<const float4*>(kp + 4 * t) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float4 vr[4][2];
    uint32_t vvalid = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int32_t key = 16 * w + 4 * g + r;
      int64_t base = -1;
      if (key < nkeys) {
        const int32_t pl = (int32_t)div_magic((uint32_t)key, A.ps_magic);
        base = M.pg[pl];
        if (base >= 0) base += (int64_t)(key - pl * A.page_size) * kD;
      }
      const float* vp = A.v + base + 8 * li;
      vr[r][0] = base >= 0 ? *reinterpret_cast<const float4*>(vp) : make_float4(0.f, 0.f, 0.f, 0.f);
      vr[r][1] = base >= 0 ? *reinterpret_cast<const float4*>(vp + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
      vvalid |= (base >= 0 ? 1u : 0u) << r;
    }
    // ---- q rows of the tile (B operand): row li, d = 32g..32g+31
    float4 qr[8];
    const bool row_ok = li < rows;
    const int32_t qi = row_ok ? M.qi[li] : 0;
    {
      const float* qp = A.q + ((int64_t)qi * A.hq + (int64_t)U.h * qhead + (row_ok ? li % qhead : 0)) * kD + 32 * g;
#pragma unroll
      for (int t = 0; t < 8; ++t)
        qr[t] = row_ok ? *reinterpret_cast<const float4*>(qp + 4 * t) : make_float4(0.f, 0.f, 0.f, 0.f);
    }

    // ---- prefetch: metadata of unit u + G, record of unit u + 2G
    const int nxt = cur ^ 1;
    const bool has_n = u + G < num_units;
    int64_t pre_pg = -1;
    int32_t pre_qi = 0, pre_rec = 0;
    Unit Un{};
    if (has_n) {
      Un = as_unit(s_meta[nxt].rec);
      if (tid < A.ppb) pre_pg = page_off(Un, tid);
      if (tid < kRows && tid < (Un.e1 - Un.e0) * qhead) pre_qi = query_of(Un, tid);
    }
    const bool has_nn = u + 2 * G < num_units;
    if (has_nn && tid < 8) pre_rec = units[8 * (int64_t)(u + 2 * G) + tid];

    // ---- S^T = K . Q^T
    floatx4 sacc = zero4();
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(kr[t].x, qr[t].x, sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(kr[t].y, qr[t].y, sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(kr[t].z, qr[t].z, sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(kr[t].w, qr[t].w, sacc, 0, 0, 0);
    }
    // ---- mask and this wave's softmax stats for row li (base 2)
    int64_t klim = A.causal ? (int64_t)qi + U.delta - block_start : (int64_t)nkeys - 1;
    klim = klim < (int64_t)nkeys - 1 ? klim : (int64_t)nkeys - 1;
    const int32_t kmax = (int32_t)(klim < -1 ? -1 : klim) - (16 * w + 4 * g);
    float mw = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool alive = row_ok && ((vvalid >> r) & 1u) && r <= kmax;
      sacc[r] = alive ? sacc[r] * A.scale_log2 : -INFINITY;
      mw = fmaxf(mw, sacc[r]);
    }
    mw = fmaxf(mw, __shfl_xor(mw, 16, 64));
    mw = fmaxf(mw, __shfl_xor(mw, 32, 64));
    float lw = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = sacc[r] == -INFINITY ? 0.f : exp2f(sacc[r] - mw);
      sacc[r] = p;
      lw += p;
    }
    lw += __shfl_xor(lw, 16, 64);
    lw += __shfl_xor(lw, 32, 64);

    // ---- O^T = V^T . P^T (row i of block db stands for d = 8i + db)
    floatx4 oacc[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) oacc[db] = zero4();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x4f32((&vr[r][0].x)[db], sacc[r], oacc[db], 0, 0, 0);
#pragma unroll
      for (int db = 0; db < 4; ++db)
        oacc[4 + db] = __builtin_amdgcn_mfma_f32_16x16x4f32((&vr[r][1].x)[db], sacc[r], oacc[4 + db], 0, 0, 0);
    }
    // lane (li, g) holds row li, d = 32g + 8v + db in oacc[db][v]
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float* dst = &s_ow[w][li][32 * g + 8 * v];
      *reinterpret_cast<float4*>(dst) = make_float4(oacc[0][v], oacc[1][v], oacc[2][v], oacc[3][v]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(oacc[4][v], oacc[5][v], oacc[6][v], oacc[7][v]);
    }
    if (g == 0) {
      s_mw[w][li] = mw;
      s_lw[w][li] = lw;
    }
    __syncthreads();

    // ---- merge the four waves' partials, store the unit's rows
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int x = tid + k * kThreads;              // (row, float4 column)
      const int j = x >> 5, c = x & 31;
      if (j < rows) {
        float big = s_mw[0][j];
#pragma unroll
        for (int ww = 1; ww < kWaves; ++ww) big = fmaxf(big, s_mw[ww][j]);
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        float lsum = 0.f;
        if (big != -INFINITY) {
#pragma unroll
          for (int ww = 0; ww < kWaves; ++ww) {
            const float mwv = s_mw[ww][j];
            const float f = mwv == -INFINITY ? 0.f : exp2f(mwv - big);
            const float4 ov = *reinterpret_cast<const float4*>(&s_ow[ww][j][4 * c]);
            o = make_float4(fmaf(ov.x, f, o.x), fmaf(ov.y, f, o.y), fmaf(ov.z, f, o.z), fmaf(ov.w, f, o.w));
            lsum = fmaf(s_lw[ww][j], f, lsum);
          }
        }
        *reinterpret_cast<float4*>(A.o + (row0 + j) * kD + 4 * c) = o;
        if (c == 0) {
          A.m[row0 + j] = big == -INFINITY ? -INFINITY : big * kLn2;
          A.l[row0 + j] = lsum;
        }
      }
    }

    // ---- hand over: stage unit u + G, keep the record of u + 2G
    if (!has_n) break;
    if (has_n) {
      if (tid < A.ppb) s_meta[nxt].pg[tid] = pre_pg;
      if (tid < kRows && tid < (Un.e1 - Un.e0) * qhead) s_meta[nxt].qi[tid] = pre_qi;
    }
    __syncthreads();                                  // s_meta[cur] and s_ow reads done
    if (has_nn && tid < 8) s_meta[cur].rec[tid] = pre_rec;
    __syncthreads();
    cur = nxt;
    u += G;
  }
}

}  // namespace

bool small_kernel_fits(int head_dim, int block_size, int page_size, int qhead) {
  return head_dim == kD && block_size <= kMaxKeys && block_size / page_size <= kMaxPages &&
         qhead <= kRows;
}

int small_kernel_rows() { return kRows; }

hipError_t launch_forward_small(const sa_index* idx, const FwdArgs& a, hipStream_t s,
                                unsigned max_grid) {
  static thread_local int per_cu = 0;
  if (per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_fwd_small, kThreads, 0) != hipSuccess || n < 1)
      n = 1;
    per_cu = n;
  }
  unsigned grid = (unsigned)per_cu * cu_count();
  if (grid > max_grid) grid = max_grid;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(k_fwd_small, dim3(grid), dim3(kThreads), 0, s, index_ptrs(idx), a);
  return hipGetLastError();
}

}  // namespace sa
