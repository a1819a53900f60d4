// Log-sum-exp combine of the KV-outer partials (the combine pass named in
// alice-llm 2.0.0 forward.rs's module doc: the FlashAttention LSE update).
//
// One workgroup per (query q, KV head h). Thread x covers GQA lane
// qh = x / D4 and float4 column c = x % D4. Over the ranks r with
// inv[h, q, r] >= 0 it reads partial row p = (edge_head_base[h] + inv)*qhead + qh
// and forms M = max m_p, L = sum l_p e^(m_p - M), O = sum o_p e^(m_p - M) / L.
// The qhead rows of one edge are contiguous, so each rank is one coalesced
// read of qhead*D floats.
#include "sa_internal.h"

namespace sa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

__global__ __launch_bounds__(256) void k_combine(IndexPtrs P, CombineArgs A) {
  if (P.hdr->status != SA_OK) return;
  const int64_t q = blockIdx.x / A.hkv;
  const int32_t h = blockIdx.x % A.hkv;
  const int32_t D4 = A.head_dim >> 2;
  const int32_t qhead = A.qhead;
  const int64_t head_base = P.edge_head_base[h];
  const int32_t* inv = P.inv + ((int64_t)h * A.tq + q) * A.topk;
  for (int32_t x = threadIdx.x; x < qhead * D4; x += 256) {
    const int32_t qh = x / D4, c = x % D4;
    float big = -INFINITY;
    for (int32_t r = 0; r < A.topk; ++r) {
      const int32_t p = inv[r];
      if (p >= 0) big = fmaxf(big, A.m[(head_base + p) * qhead + qh]);
    }
    const int64_t out_off = (q * A.hq + (int64_t)h * qhead + qh) * A.head_dim + c * 4;
    if (big == -INFINITY) {
      *reinterpret_cast<float4*>(A.out + out_off) = make_float4(0.f, 0.f, 0.f, 0.f);
      if (A.lse != nullptr && c == 0) A.lse[q * A.hq + (int64_t)h * qhead + qh] = -INFINITY;
      continue;
    }
    float total = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int32_t r = 0; r < A.topk; ++r) {
      const int32_t p = inv[r];
      if (p < 0) continue;
      const int64_t row = (head_base + p) * qhead + qh;
      const float mp = A.m[row];
      if (mp == -INFINITY) continue;
      const float w = exp2f((mp - big) * kLog2e);
      total = fmaf(A.l[row], w, total);
      const float4 o = *reinterpret_cast<const float4*>(A.o + row * A.head_dim + c * 4);
      acc = make_float4(fmaf(o.x, w, acc.x), fmaf(o.y, w, acc.y), fmaf(o.z, w, acc.z),
                        fmaf(o.w, w, acc.w));
    }
    const float inv_total = 1.f / total;
    *reinterpret_cast<float4*>(A.out + out_off) =
        make_float4(acc.x * inv_total, acc.y * inv_total, acc.z * inv_total, acc.w * inv_total);
    if (A.lse != nullptr && c == 0)
      A.lse[q * A.hq + (int64_t)h * qhead + qh] = big + logf(total);
  }
}

}  // namespace

hipError_t launch_combine(const sa_index* idx, const CombineArgs& a, hipStream_t s) {
  const IndexPtrs P = index_ptrs(idx);
  const int64_t grid = a.tq * a.hkv;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)grid), dim3(256), 0, s, P, a);
  return hipGetLastError();
}

}  // namespace sa
