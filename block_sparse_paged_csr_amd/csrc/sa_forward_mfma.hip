// KV-outer forward, MFMA path (units whose rows form dense 32-row tiles).
//
// Same partials as the wavefront path: for every edge (q, r) of the unit and
// GQA lane qh, (o, m, l) of alice-llm 2.0.0 forward.rs process_work_unit over
// the block's valid, causally alive positions.
//
// One workgroup (8 waves) per CU takes units from a device queue. For each
// unit it gathers the block's K and V rows once into LDS (row pitch padded
// so the MFMA operand reads do not conflict). Each wave then takes 32-row
// tiles of the unit and computes them on fp32 matrix cores
// (v_mfma_f32_32x32x2f32):
//
//   S^T[key, row] = K[key, :] . Q[row, :]       A = K from LDS, B = Q^T in registers
//   O^T[d, row]  += V[key, d] * P[row, key]      A = V^T from LDS, B = P^T in registers
//
// Computing S transposed leaves each lane holding one query row (lane % 32)
// and 64 of its 128 keys; lane ^ 32 holds the other 64. The row max and sum
// need one lane swap. The probabilities are already in the B-operand layout
// of the PV product, so P never goes through LDS. The contraction index of
// the QK product is permuted (lanes 0-31 take d = 0..63, lanes 32-63 take
// d = 64..127), which leaves the sum unchanged and makes each lane's K and Q
// reads contiguous.
#include "sa_internal.h"

namespace sa {

namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

__device__ inline floatx16 zero16() {
  floatx16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kD = 128;                 // head_dim of this kernel
constexpr int kMaxKeys = 128;           // block_size <= 128
constexpr int kKPitch = kD + 4;         // floats; 16-byte aligned rows, conflict-free b128 reads
constexpr int kVPitch = kD + 8;         // floats; the two key rows of a PV operand use disjoint banks
constexpr float kLn2 = 0.69314718055994530942f;

template <int NKB>   // 32-key blocks per KV block (block_size <= 32 * NKB)
__global__ __launch_bounds__(kThreads) void k_fwd_mfma(IndexPtrs P, FwdArgs A) {
  __shared__ __align__(16) float s_k[kMaxKeys * kKPitch];
  __shared__ __align__(16) float s_v[kMaxKeys * kVPitch];
  __shared__ int s_valid[kMaxKeys];
  __shared__ int s_unit;

  DevHeader* hdr = P.hdr;
  if (hdr->status != SA_OK) return;
  const int32_t num_units = hdr->num_units_mfma;
  // Workgroup g starts on unit g, then pulls units gridDim.x, gridDim.x+1, ...
  // from the queue. Workgroups without a first unit leave at once, so an
  // empty list costs no atomics.
  if ((int32_t)blockIdx.x >= num_units) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int lr = lane & 31, half = lane >> 5;
  const int32_t qhead = A.qhead;
  const int64_t page_stride = (int64_t)A.hkv * A.page_size * kD;

  for (int32_t u = blockIdx.x;;) {
    if (u >= num_units) break;
    const Unit U = P.units_mfma[u];
    const int64_t lk = U.lk;
    const int64_t block_start = (int64_t)U.blk * A.block_size;
    int64_t block_end = block_start + A.block_size;
    block_end = block_end < lk ? block_end : lk;
    const int32_t nkeys = block_end > block_start ? (int32_t)(block_end - block_start) : 0;
    const int64_t bt_row = (int64_t)U.b * A.max_pages + (int64_t)U.blk * A.ppb;
    const int64_t head_off = (int64_t)U.h * A.page_size * kD;

    // ---- gather K and V of the block into LDS (zero rows past the valid range)
    for (int x = tid; x < NKB * 32 * (kD / 4); x += kThreads) {
      const int key = x / (kD / 4), c4 = x % (kD / 4);
      bool valid = key < nkeys;
      int64_t off = 0;
      if (valid) {
        const int32_t pgl = (int32_t)div_magic((uint32_t)key, A.ps_magic);
        const int32_t page = A.block_tables[bt_row + pgl];
        valid = page >= 0 && page < A.num_pages;
        off = (int64_t)page * page_stride + head_off + (int64_t)(key - pgl * A.page_size) * kD + c4 * 4;
      }
      const float4 kv = valid ? *reinterpret_cast<const float4*>(A.k + off) : make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 vv = valid ? *reinterpret_cast<const float4*>(A.v + off) : make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<float4*>(&s_k[key * kKPitch + c4 * 4]) = kv;
      *reinterpret_cast<float4*>(&s_v[key * kVPitch + c4 * 4]) = vv;
      if (c4 == 0) s_valid[key] = valid;
    }
    __syncthreads();

    // Keys held by this lane in the S^T accumulators: kb*32 + 8*(r/4) + 4*half + r%4.
    // Bit r of vm[kb] says whether that key has a page (holes are rare).
    uint32_t vm[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      vm[kb] = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        vm[kb] |= (s_valid[kb * 32 + 8 * (r / 4) + 4 * half + (r % 4)] ? 1u : 0u) << r;
    }

    const int32_t rows = (U.e1 - U.e0) * qhead;
    const int64_t row0 = (int64_t)U.e0 * qhead;
    const int32_t ntiles = (rows + 31) / 32;
    for (int32_t tile = wv; tile < ntiles; tile += kWaves) {
      const int32_t row = tile * 32 + lr;
      const bool row_ok = row < rows;
      int32_t qi = 0;
      if (row_ok) qi = P.edges[2 * (int64_t)(U.e0 + row / qhead)];
      const float* qp = A.q + ((int64_t)qi * A.hq + (int64_t)U.h * qhead + (row_ok ? row % qhead : 0)) * kD + half * 64;
      float4 qr[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        qr[i] = row_ok ? *reinterpret_cast<const float4*>(qp + 4 * i) : make_float4(0.f, 0.f, 0.f, 0.f);
      // Key k is alive iff k < nkeys, its page exists and (causal) block_start + k
      // <= q + delta. kmax folds the two bounds; comparisons stay 32-bit.
      int64_t klim = A.causal ? (int64_t)qi + U.delta - block_start : (int64_t)nkeys - 1;
      klim = klim < (int64_t)nkeys - 1 ? klim : (int64_t)nkeys - 1;
      const int32_t kmaxh = (int32_t)(klim < -1 ? -1 : klim) - 4 * half;

      // ---- S^T = K . Q^T over d (lanes 0-31: d 0..63, lanes 32-63: d 64..127)
      floatx16 sacc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sacc[kb] = zero16();
#pragma unroll
      for (int m4 = 0; m4 < 16; ++m4) {
        float4 kv[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          kv[kb] = *reinterpret_cast<const float4*>(
              &s_k[(kb * 32 + lr) * kKPitch + half * 64 + m4 * 4]);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[kb].x, qr[m4].x, sacc[kb], 0, 0, 0);
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[kb].y, qr[m4].y, sacc[kb], 0, 0, 0);
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[kb].z, qr[m4].z, sacc[kb], 0, 0, 0);
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[kb].w, qr[m4].w, sacc[kb], 0, 0, 0);
        }
        // bound how far LDS reads run ahead of the MFMAs that use them
        __builtin_amdgcn_sched_barrier(0);
      }

      // ---- mask, row max and sum (base 2; the scale carries log2 e)
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool alive = ((vm[kb] >> r) & 1u) && (kb * 32 + 8 * (r / 4) + (r % 4)) <= kmaxh;
          const float s = alive ? sacc[kb][r] * A.scale_log2 : -INFINITY;
          sacc[kb][r] = s;
          mx = fmaxf(mx, s);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      float sum = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float s = sacc[kb][r];
          const float p = (s == -INFINITY) ? 0.f : exp2f(s - mx);
          sacc[kb][r] = p;
          sum += p;
        }
      sum += __shfl_xor(sum, 32, 64);

      // ---- O^T = V^T . P^T; the k pair of MFMA (kb, r) is keys kappa and kappa + 4
      floatx16 oacc[kD / 32];
#pragma unroll
      for (int db = 0; db < kD / 32; ++db) oacc[db] = zero16();
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + 8 * (r / 4) + 4 * half + (r % 4);
          const float* vrow = &s_v[key * kVPitch + lr];
          float va[kD / 32];
#pragma unroll
          for (int db = 0; db < kD / 32; ++db) va[db] = vrow[db * 32];
#pragma unroll
          for (int db = 0; db < kD / 32; ++db)
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(va[db], sacc[kb][r], oacc[db], 0, 0, 0);
          if ((r & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }

      // ---- store the tile's partial rows (o unnormalised, m in natural-log units)
      if (row_ok) {
        float* op = A.o + (row0 + row) * kD + 4 * half;
#pragma unroll
        for (int db = 0; db < kD / 32; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<float4*>(op + db * 32 + 8 * g) =
                make_float4(oacc[db][4 * g], oacc[db][4 * g + 1], oacc[db][4 * g + 2], oacc[db][4 * g + 3]);
        if (half == 0) {
          A.m[row0 + row] = mx == -INFINITY ? -INFINITY : mx * kLn2;
          A.l[row0 + row] = sum;
        }
      }
    }
    __syncthreads();                       // LDS of this unit no longer read
    if (tid == 0) s_unit = (int)gridDim.x + (int)atomicAdd(&hdr->queue_mfma, 1u);
    __syncthreads();
    u = s_unit;
  }
  // The last participating workgroup out resets the queue for the next launch.
  if (tid == 0) {
    __threadfence();
    const unsigned active = num_units < (int32_t)gridDim.x ? (unsigned)num_units : gridDim.x;
    const unsigned done = atomicAdd(&hdr->done_mfma, 1u);
    if (done == active - 1) {
      atomicExch(&hdr->queue_mfma, 0u);
      atomicExch(&hdr->done_mfma, 0u);
    }
  }
}

template <int NKB>
hipError_t launch_mfma_t(const IndexPtrs& P, const FwdArgs& a, hipStream_t s, unsigned grid) {
  hipLaunchKernelGGL(k_fwd_mfma<NKB>, dim3(grid), dim3(kThreads), 0, s, P, a);
  return hipGetLastError();
}

}  // namespace

bool mfma_enabled() { return true; }

hipError_t launch_forward_mfma(const sa_index* idx, const FwdArgs& a, hipStream_t s,
                               unsigned grid) {
  if (a.head_dim != kD || a.block_size > kMaxKeys) return hipErrorInvalidValue;
  const IndexPtrs P = index_ptrs(idx);
  const int nkb = (a.block_size + 31) / 32;
  if (nkb <= 1) return launch_mfma_t<1>(P, a, s, grid);
  if (nkb <= 2) return launch_mfma_t<2>(P, a, s, grid);
  if (nkb <= 3) return launch_mfma_t<3>(P, a, s, grid);
  return launch_mfma_t<4>(P, a, s, grid);
}

}  // namespace sa
