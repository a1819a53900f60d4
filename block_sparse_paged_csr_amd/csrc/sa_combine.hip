// Log-sum-exp combine of the KV-outer partials (the combine pass named in
// alice-llm 2.0.0 forward.rs's module doc: the FlashAttention LSE update).
//
// One workgroup per (query q, KV head h). Work item x covers GQA lane
// qh = x / D4 and float4 column c = x % D4. Over the ranks r with
// inv[h, q, r] >= 0 it reads partial row p = (edge_head_base[h] + inv)*qhead + qh
// and forms M = max m_p, L = sum l_p e^(m_p - M), O = sum o_p e^(m_p - M) / L.
//
// Ranks go in tiles of kRankTile. A tile's partial-row offsets and (m, l)
// are staged in LDS first, so the o reads of a tile do not depend on each
// other and are all in flight together. Across tiles the running (M, L, O)
// is rescaled. The qhead rows of one edge are contiguous, so each rank is one
// coalesced read of qhead*D floats.
#include "sa_internal.h"

namespace sa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kRankTile = 64;
constexpr int kMaxItems = 1;          // work items per thread (qhead * D4 <= blockDim <= 1024)

__global__ __launch_bounds__(1024) void k_combine(IndexPtrs P, CombineArgs A) {
  if (P.hdr->status != SA_OK) return;
  extern __shared__ __align__(16) unsigned char smem[];
  const int32_t qhead = A.qhead;
  int64_t* s_row = reinterpret_cast<int64_t*>(smem);                     // [kRankTile]
  float* s_m = reinterpret_cast<float*>(smem + 8 * kRankTile);           // [kRankTile][qhead]
  float* s_l = s_m + kRankTile * qhead;                                  // [kRankTile][qhead]

  const int64_t q = blockIdx.x / A.hkv;
  const int32_t h = blockIdx.x % A.hkv;
  const int32_t D4 = A.head_dim >> 2;
  const int32_t n_items = qhead * D4;
  const int64_t head_base = P.edge_head_base[h];
  const int32_t* inv = P.inv + ((int64_t)h * A.tq + q) * A.topk;
  const int tid = threadIdx.x, nthr = blockDim.x;

  float big[kMaxItems], total[kMaxItems];
  float4 acc[kMaxItems];
#pragma unroll
  for (int k = 0; k < kMaxItems; ++k) {
    big[k] = -INFINITY;
    total[k] = 0.f;
    acc[k] = make_float4(0.f, 0.f, 0.f, 0.f);
  }

  for (int32_t r0 = 0; r0 < A.topk; r0 += kRankTile) {
    const int32_t nr = A.topk - r0 < kRankTile ? A.topk - r0 : kRankTile;
    __syncthreads();
    for (int t = tid; t < nr; t += nthr) {
      const int32_t p = inv[r0 + t];
      s_row[t] = p >= 0 ? (head_base + p) * qhead : -1;
    }
    __syncthreads();
    for (int x = tid; x < nr * qhead; x += nthr) {
      const int t = x / qhead, qh = x % qhead;
      const int64_t row = s_row[t];
      s_m[x] = row >= 0 ? A.m[row + qh] : -INFINITY;
      s_l[x] = row >= 0 ? A.l[row + qh] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kMaxItems; ++k) {
      const int x = tid + k * nthr;
      if (x >= n_items) break;
      const int qh = x / D4, c = x % D4;
      float mt = -INFINITY;
      for (int t = 0; t < nr; ++t) mt = fmaxf(mt, s_m[t * qhead + qh]);
      const float m_new = fmaxf(big[k], mt);
      if (m_new == -INFINITY) continue;
      const float keep = big[k] == -INFINITY ? 0.f : exp2f((big[k] - m_new) * kLog2e);
      float4 a = make_float4(acc[k].x * keep, acc[k].y * keep, acc[k].z * keep, acc[k].w * keep);
      float lsum = total[k] * keep;
#pragma unroll 8
      for (int t = 0; t < nr; ++t) {
        const float mp = s_m[t * qhead + qh];
        const float w = mp == -INFINITY ? 0.f : exp2f((mp - m_new) * kLog2e);
        const int64_t row = s_row[t];
        const float4 o = w > 0.f ? *reinterpret_cast<const float4*>(
                                       A.o + (row + qh) * A.head_dim + c * 4)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
        a = make_float4(fmaf(o.x, w, a.x), fmaf(o.y, w, a.y), fmaf(o.z, w, a.z), fmaf(o.w, w, a.w));
        lsum = fmaf(s_l[t * qhead + qh], w, lsum);
      }
      acc[k] = a;
      total[k] = lsum;
      big[k] = m_new;
    }
  }
#pragma unroll
  for (int k = 0; k < kMaxItems; ++k) {
    const int x = tid + k * nthr;
    if (x >= n_items) break;
    const int qh = x / D4, c = x % D4;
    const int64_t out_off = (q * A.hq + (int64_t)h * qhead + qh) * A.head_dim + c * 4;
    if (big[k] == -INFINITY) {
      *reinterpret_cast<float4*>(A.out + out_off) = make_float4(0.f, 0.f, 0.f, 0.f);
      if (A.lse != nullptr && c == 0) A.lse[q * A.hq + (int64_t)h * qhead + qh] = -INFINITY;
    } else {
      const float inv_total = 1.f / total[k];
      *reinterpret_cast<float4*>(A.out + out_off) =
          make_float4(acc[k].x * inv_total, acc[k].y * inv_total, acc[k].z * inv_total,
                      acc[k].w * inv_total);
      if (A.lse != nullptr && c == 0)
        A.lse[q * A.hq + (int64_t)h * qhead + qh] = big[k] + logf(total[k]);
    }
  }
}

}  // namespace

hipError_t launch_combine(const sa_index* idx, const CombineArgs& a, hipStream_t s) {
  const IndexPtrs P = index_ptrs(idx);
  const int64_t grid = a.tq * a.hkv;
  const int n_items = a.qhead * (a.head_dim / 4);
  int block = (n_items + 63) / 64 * 64;
  if (block > 1024) block = 1024;
  if (n_items > block * kMaxItems) return hipErrorInvalidValue;   // plan rejects this
  const size_t smem = 8 * kRankTile + 2 * 4 * (size_t)kRankTile * a.qhead;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)grid), dim3(block), smem, s, P, a);
  return hipGetLastError();
}

}  // namespace sa
