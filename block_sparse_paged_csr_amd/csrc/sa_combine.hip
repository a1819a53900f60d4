// Log-sum-exp combine of the KV-outer partials (the combine pass named in
// alice-llm 2.0.0 forward.rs's module doc: the FlashAttention LSE update).
//
// One workgroup per (query q, KV head h). Work item x covers GQA lane
// qh = x / D4 and float4 column c = x % D4. Over the ranks r with
// inv[h, q, r] >= 0 it reads partial row p = (edge_head_base[h] + inv)*qhead + qh
// and forms M = max m_p, L = sum l_p e^(m_p - M), O = sum o_p e^(m_p - M) / L.
//
// Latency: the index reads (status, head base, the ranks' inv) are issued
// together; then, per tile of kRankTile ranks, every item loads its rows' m,
// l and o float4 at once (none of them waits on another), so a tile costs one
// round trip. The running (M, L, O) is rescaled across tiles. The qhead rows
// of one edge are contiguous, so each rank is one coalesced read of
// qhead*D floats by the workgroup.
#include "sa_internal.h"

namespace sa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kRankTile = 16;
constexpr int kMaxBlock = 1024;      // qhead * D4 <= 1024: one item per thread

// Partial reads: plain, or non-temporal (NT) where the forward wrote the
// partials with non-temporal stores (the one-wave kernel). Every partial is
// read once; streamed that way, ragged's combine takes 47 instead of 52 us,
// while partials written with plain stores (the MFMA kernels) read faster
// plainly.
typedef float floatx4nt __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ inline float ld_f(const float* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT>
__device__ inline float4 ld_f4(const float* p) {
  if constexpr (NT) {
    const floatx4nt v = __builtin_nontemporal_load(reinterpret_cast<const floatx4nt*>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
  } else {
    return *reinterpret_cast<const float4*>(p);
  }
}

template <bool NT>
__global__ __launch_bounds__(kMaxBlock) void k_combine(IndexPtrs P, CombineArgs A) {
  const int32_t qhead = A.qhead;
  // Workgroup order: head-major over the one-wave kernel's partials (decode
  // combine 5.2 -> 5.1 us), query-major over the MFMA kernels' (prefill's
  // combine read them 2% slower head-major).
  int64_t q;
  int32_t h;
  if constexpr (NT) {
    const uint32_t tq32 = (uint32_t)A.tq;   // tq * hkv workgroups: fits 32 bits
    h = (int32_t)(blockIdx.x / tq32);
    q = (int64_t)(blockIdx.x - (uint32_t)h * tq32);
  } else {
    q = blockIdx.x / A.hkv;
    h = blockIdx.x % A.hkv;
  }
  const int32_t D4 = A.head_dim >> 2;
  const int x = threadIdx.x;
  const int qh = x / D4, c = x - qh * D4;
  const bool item = qh < qhead;
  const int32_t* inv = P.inv + ((int64_t)h * A.tq + q) * A.topk;

  // Independent reads first, in one round trip: status, head base and the
  // first tile's inv entries, one rank per lane (lane & 15) in a single vector
  // load, broadcast below with readlane. The rank index is clamped to
  // topk - 1, so every load is in bounds; inv is read before the status test
  // (a failed build leaves it allocated, and its values go unused then). The
  // empty asm makes the status branch wait for the inv and head-base loads
  // too, so that the compiler cannot sink them below the branch into round
  // trips of their own.
  const int32_t tl = (int32_t)(threadIdx.x & (kRankTile - 1));
  const int32_t status = P.hdr->status;
  const int64_t head_base = P.edge_head_base[h];
  int32_t mine = inv[tl < A.topk ? tl : A.topk - 1];
  asm volatile("" ::"v"(mine), "s"(head_base));
  if (status != SA_OK) {
    // The build failed (the pages return an error here): the forward wrote
    // nothing, so the output gets a defined value instead of stale memory.
    if (item) {
      const int64_t o_off = (q * A.hq + (int64_t)h * qhead + qh) * A.head_dim + c * 4;
      *reinterpret_cast<float4*>(A.out + o_off) = make_float4(NAN, NAN, NAN, NAN);
      if (A.lse != nullptr && c == 0) A.lse[q * A.hq + (int64_t)h * qhead + qh] = NAN;
    }
    return;
  }

  float big = -INFINITY, total = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int32_t r0 = 0; r0 < A.topk; r0 += kRankTile) {
    if (r0 > 0) mine = inv[r0 + tl < A.topk ? r0 + tl : A.topk - 1];
    int64_t row[kRankTile];
#pragma unroll
    for (int t = 0; t < kRankTile; ++t) {
      const int32_t p = r0 + t < A.topk ? __builtin_amdgcn_readlane(mine, t) : -1;
      row[t] = (p >= 0 && item) ? (head_base + p) * qhead + qh : -1;
    }
    float mv[kRankTile], lv[kRankTile];
    float4 ov[kRankTile];
#pragma unroll
    for (int t = 0; t < kRankTile; ++t) {
      const bool ok = row[t] >= 0;
      const int64_t rr = ok ? row[t] : 0;
      mv[t] = ok ? ld_f<NT>(A.m + rr) : -INFINITY;
      lv[t] = ok ? ld_f<NT>(A.l + rr) : 0.f;
      ov[t] = ok ? ld_f4<NT>(A.o + rr * A.head_dim + 4 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float mt = -INFINITY;
#pragma unroll
    for (int t = 0; t < kRankTile; ++t) mt = fmaxf(mt, mv[t]);
    const float m_new = fmaxf(big, mt);
    if (m_new == -INFINITY) continue;
    const float keep = big == -INFINITY ? 0.f : exp2f((big - m_new) * kLog2e);
    float4 a = make_float4(acc.x * keep, acc.y * keep, acc.z * keep, acc.w * keep);
    float lsum = total * keep;
#pragma unroll
    for (int t = 0; t < kRankTile; ++t) {
      const float w = mv[t] == -INFINITY ? 0.f : exp2f((mv[t] - m_new) * kLog2e);
      a = make_float4(fmaf(ov[t].x, w, a.x), fmaf(ov[t].y, w, a.y), fmaf(ov[t].z, w, a.z),
                      fmaf(ov[t].w, w, a.w));
      lsum = fmaf(lv[t], w, lsum);
    }
    acc = a;
    total = lsum;
    big = m_new;
  }
  if (!item) return;
  const int64_t out_off = (q * A.hq + (int64_t)h * qhead + qh) * A.head_dim + c * 4;
  if (big == -INFINITY) {
    *reinterpret_cast<float4*>(A.out + out_off) = make_float4(0.f, 0.f, 0.f, 0.f);
    if (A.lse != nullptr && c == 0) A.lse[q * A.hq + (int64_t)h * qhead + qh] = -INFINITY;
  } else {
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
  const int n_items = a.qhead * (a.head_dim / 4);
  int block = (n_items + 63) / 64 * 64;
  if (block > kMaxBlock) return hipErrorInvalidValue;             // plan rejects this
  // the one-wave forward (where it fits) writes its partials non-temporally
  if (small_kernel_fits(a.head_dim, idx->block_size, idx->page_size, a.qhead))
    hipLaunchKernelGGL(k_combine<true>, dim3((unsigned)grid), dim3(block), 0, s, P, a);
  else
    hipLaunchKernelGGL(k_combine<false>, dim3((unsigned)grid), dim3(block), 0, s, P, a);
  return hipGetLastError();
}

}  // namespace sa
