// KV-outer forward, MFMA path (units whose rows form dense 32-row tiles).
//
// Same partials as the wavefront path: for every edge (q, r) of the unit and
// GQA lane qh, (o, m, l) of alice-llm 2.0.0 forward.rs process_work_unit over
// the block's valid, causally alive positions.
//
// Persistent workgroups, one per CU for blocks of up to 128 keys (the
// direct-to-LDS kernel, units dealt statically in size order; the chunked
// kernel for other geometries), two per CU for blocks of up to 64 keys (the
// 16-row kernel). For each unit the workgroup resolves each key's K/V row
// offset through the block table and brings the block's K and V rows into
// LDS once, all loads in flight (rows padded or swizzled so that the MFMA
// operand reads do not conflict). The waves then compute the unit's 32-row
// tiles on fp32 matrix cores (v_mfma_f32_32x32x2f32):
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

constexpr int kD = 128;                 // head_dim of this kernel
constexpr int kMaxKeys = 128;           // block_size <= 128
constexpr int kKPitch = kD + 4;         // floats; 16-byte aligned rows, conflict-free b128 reads
constexpr int kVPitch = kD + 8;         // floats; the two key rows of a PV operand use disjoint banks
constexpr float kLn2 = 0.69314718055994530942f;
// Most edges in one MFMA unit (cap_edges <= kMaxUnitEdges, see the plan).
constexpr int kMaxUnitEdges = kCapUnitEdges;

// ---- pieces of one 32-row tile (fp32 rows in LDS), shared by the direct-to-LDS
// and chunked kernels below
// (K and V rows in LDS with pitches kKPitch and kVPitch floats).

// Bit r of the result for 32-key block kb: key kb*32 + 8*(r/4) + 4*half + r%4
// (the key of accumulator r of this lane) has a row, from the block's
// validity words; `all_rows` is set when every key of the block has one.
template <int NKB>
__device__ __forceinline__ void lane_key_bits(const uint32_t* valid, int half, uint32_t (&vm)[NKB],
                                              bool& all_rows) {
  all_rows = true;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    const uint32_t wbits = valid[kb];
    all_rows = all_rows && wbits == 0xffffffffu;
    uint32_t m = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) m |= ((wbits >> (8 * (r / 4) + 4 * half + (r % 4))) & 1u) << r;
    vm[kb] = m;
  }
}

// S^T = K . Q^T over d for the lane's row (lane % 32); the K operands of
// each step are read one step ahead.
template <int NKB, int D = kD>
__device__ __forceinline__ void tile_scores(const float* sk, const float4 (&qr)[D / 8], int lr, int half,
                                            floatx16 (&sacc)[NKB]) {
  constexpr int KP = D + 4, M4 = D / 8;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) sacc[kb] = zero16();
  float4 kc[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
    kc[kb] = *reinterpret_cast<const float4*>(&sk[(kb * 32 + lr) * KP + half * (D / 2)]);
  __builtin_amdgcn_sched_group_barrier(0x0100, NKB, 0);
#pragma unroll
  for (int m4 = 0; m4 < M4; ++m4) {
    float4 kn[NKB];
    if (m4 < M4 - 1) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        kn[kb] = *reinterpret_cast<const float4*>(&sk[(kb * 32 + lr) * KP + half * (D / 2) + (m4 + 1) * 4]);
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kc[kb].x, qr[m4].x, sacc[kb], 0, 0, 0);
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kc[kb].y, qr[m4].y, sacc[kb], 0, 0, 0);
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kc[kb].z, qr[m4].z, sacc[kb], 0, 0, 0);
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kc[kb].w, qr[m4].w, sacc[kb], 0, 0, 0);
    }
    // the next step's LDS reads go out before this step's products
    if (m4 < M4 - 1) __builtin_amdgcn_sched_group_barrier(0x0100, NKB, 0);
    __builtin_amdgcn_sched_group_barrier(0x0008, 4 * NKB, 0);
    if (m4 < M4 - 1) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) kc[kb] = kn[kb];
    }
  }
}

// Mask, block max and sum. The scores are raw dot products; the largest
// scaled score c2*s is c2 times the largest raw score (c2 >= 0) or the
// smallest (c2 < 0), and p = exp2(c2*s - that), base 2 with log2 e in c2.
// Replaces the scores by p (0 for dead keys) and returns the max scaled
// score in base-2 units (-inf: no alive key) and the row sum. `full`: every
// key alive for every row of the tile, so the masks are skipped; otherwise
// key k of the lane is alive iff its bit in vm is set and its index in the
// block, less 4*half, is at most kmaxh.
//
// Bits r (0..15) of a 32-key block whose key 8*(r/4) + r%4 is at most x.
__device__ __forceinline__ uint32_t keys_upto(int32_t x) {
  if (x < 0) return 0u;
  x = x < 31 ? x : 31;
  const uint32_t grp = (uint32_t)x >> 3, w = ((uint32_t)x & 7u) + 1u;
  const uint32_t lo = (1u << (4 * grp)) - 1u;
  return lo | (((1u << (w < 4u ? w : 4u)) - 1u) << (4 * grp));
}
//
// kRaw: vm holds the block's validity words themselves (bit k: key 32kb + k
// has a row), read where they are needed instead of kept as per-lane masks.
// Accumulator r of the lane then stands for bit 8*(r/4) + r%4 of the word
// shifted right by 4*half.
__device__ __forceinline__ uint32_t bits_upto(int32_t x) {
  return x < 0 ? 0u : (x >= 31 ? 0xffffffffu : (2u << x) - 1u);
}
template <int NKB, bool kRaw = false>
__device__ __forceinline__ void tile_softmax(floatx16 (&sacc)[NKB], bool full, const uint32_t* vm, int half,
                                             int32_t kmaxh, float c2, float& mb2, float& sum) {
  const bool up = c2 >= 0.f;
  if (!full) {
    // dead keys' scores become the identity of the max (min); the alive
    // bits are formed here for each tile, as plain per-lane words
    const float dead = up ? -INFINITY : INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      uint32_t w = vm[kb];
      if (kRaw) {
        const uint32_t aw = (w >> (4 * half)) & 0x0f0f0f0fu & bits_upto(kmaxh - kb * 32);
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = ((aw >> (8 * (r / 4) + r % 4)) & 1u) ? sacc[kb][r] : dead;
      } else {
        asm volatile("" : "+v"(w));
        const uint32_t aw = w & keys_upto(kmaxh - kb * 32);
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = ((aw >> r) & 1u) ? sacc[kb][r] : dead;
      }
    }
  }
  float ext = up ? -INFINITY : INFINITY;
  if (up) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) ext = fmaxf(ext, sacc[kb][r]);
  } else {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) ext = fminf(ext, sacc[kb][r]);
  }
  {
    const float other = __shfl_xor(ext, 32, 64);
    ext = up ? fmaxf(ext, other) : fminf(ext, other);
  }
  const bool none = up ? ext == -INFINITY : ext == INFINITY;
  mb2 = none ? -INFINITY : ext * c2;
  const float nref = none ? 0.f : -mb2;
  // p = exp2(c2*s - mb2); a dead key's infinite score gives exp2(-inf) = 0,
  // or NaN when c2 == 0, which the max with 0 turns into 0 (masked tiles only)
  float sum4[4] = {0.f, 0.f, 0.f, 0.f};
  if (full) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], c2, nref));
        sacc[kb][r] = p;
        sum4[r & 3] += p;
      }
  } else {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fmaxf(__builtin_amdgcn_exp2f(fmaf(sacc[kb][r], c2, nref)), 0.f);
        sacc[kb][r] = p;
        sum4[r & 3] += p;
      }
  }
  sum = (sum4[0] + sum4[1]) + (sum4[2] + sum4[3]);
  sum += __shfl_xor(sum, 32, 64);
}

// O^T = V^T . P^T; the k pair of MFMA (kb, r) is keys kappa and kappa + 4.
// The V operands of each pair of r are read one pair ahead.
template <int NKB, int D = kD>
__device__ __forceinline__ void tile_pv(const float* sv, const floatx16 (&sacc)[NKB], int lr, int half,
                                        floatx16 (&oacc)[D / 32], bool accumulate = false) {
  constexpr int VP = D + 8;
  if (!accumulate) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = zero16();
  }
  float vc[2][D / 32];
  auto read_v = [&](int r0, float (&dst)[2][D / 32]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = r0 + j, kb = r / 16, rr = r % 16;
      const float* vrow = &sv[(kb * 32 + 8 * (rr / 4) + 4 * half + (rr % 4)) * VP + lr];
#pragma unroll
      for (int db = 0; db < D / 32; ++db) dst[j][db] = vrow[db * 32];
    }
  };
  read_v(0, vc);
  __builtin_amdgcn_sched_group_barrier(0x0100, 2 * (D / 32), 0);
#pragma unroll
  for (int r0 = 0; r0 < 16 * NKB; r0 += 2) {
    float vn[2][D / 32];
    if (r0 + 2 < 16 * NKB) read_v(r0 + 2, vn);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vc[j][db], sacc[(r0 + j) / 16][(r0 + j) % 16],
                                                        oacc[db], 0, 0, 0);
    if (r0 + 2 < 16 * NKB) __builtin_amdgcn_sched_group_barrier(0x0100, 2 * (D / 32), 0);
    __builtin_amdgcn_sched_group_barrier(0x0008, 2 * (D / 32), 0);
    if (r0 + 2 < 16 * NKB) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) vc[j][db] = vn[j][db];
    }
  }
}

// The tile's partial row `row` of the unit (o unnormalised, m in natural-log units).
template <int D = kD>
__device__ __forceinline__ void tile_store(const FwdArgs& A, int64_t row0, int32_t row, int half,
                                           const floatx16 (&oacc)[D / 32], float mb2, float sum) {
  float* op = A.o + (row0 + row) * D + 4 * half;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<float4*>(op + db * 32 + 8 * g) =
          make_float4(oacc[db][4 * g], oacc[db][4 * g + 1], oacc[db][4 * g + 2], oacc[db][4 * g + 3]);
  if (half == 0) {
    A.m[row0 + row] = mb2 * kLn2;
    A.l[row0 + row] = sum;
  }
}

// ---- pieces of one 16-row tile on v_mfma_f32_16x16x4f32 (same LDS layout),
// for the direct-to-LDS kernel below. Operand layout (lane li = lane % 16 of
// lane group g = lane / 16):
//   S^T[key, row]: MFMA t, component c takes d = 16t + 4g + c; lane (li, g)
//                  gets row li, keys 16ch + 4g + r (r = 0..3) of 16-key chunk ch
//   O^T[d, row]:   output row i of MFMA block db stands for d = 4i + (db & 3) + 64 (db >> 2)
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ inline floatx4 zero4v() {
  floatx4 z;
  z[0] = z[1] = z[2] = z[3] = 0.f;
  return z;
}

// Raw scores of row li over the NCH 16-key chunks; q in qr[0..7] (d = 16t + 4g ..).
template <int NCH>
__device__ __forceinline__ void tile16_scores(const float* sk, const float4 (&qr)[16], int li, int g,
                                              float (&s)[NCH][4]) {
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    floatx4 sa0 = zero4v(), sa1 = zero4v();
    const float* kr = &sk[(16 * ch + li) * kKPitch + 4 * g];
#pragma unroll
    for (int t = 0; t < 8; t += 2) {
      const float4 ka = *reinterpret_cast<const float4*>(kr + 16 * t);
      const float4 kb = *reinterpret_cast<const float4*>(kr + 16 * (t + 1));
      sa0 = __builtin_amdgcn_mfma_f32_16x16x4f32(ka.x, qr[t].x, sa0, 0, 0, 0);
      sa1 = __builtin_amdgcn_mfma_f32_16x16x4f32(kb.x, qr[t + 1].x, sa1, 0, 0, 0);
      sa0 = __builtin_amdgcn_mfma_f32_16x16x4f32(ka.y, qr[t].y, sa0, 0, 0, 0);
      sa1 = __builtin_amdgcn_mfma_f32_16x16x4f32(kb.y, qr[t + 1].y, sa1, 0, 0, 0);
      sa0 = __builtin_amdgcn_mfma_f32_16x16x4f32(ka.z, qr[t].z, sa0, 0, 0, 0);
      sa1 = __builtin_amdgcn_mfma_f32_16x16x4f32(kb.z, qr[t + 1].z, sa1, 0, 0, 0);
      sa0 = __builtin_amdgcn_mfma_f32_16x16x4f32(ka.w, qr[t].w, sa0, 0, 0, 0);
      sa1 = __builtin_amdgcn_mfma_f32_16x16x4f32(kb.w, qr[t + 1].w, sa1, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);   // bound how far LDS reads run ahead
#pragma unroll
    for (int r = 0; r < 4; ++r) s[ch][r] = sa0[r] + sa1[r];
  }
}

// Mask, max and sum of row li as tile_softmax does for 32-row tiles: key
// 16ch + 4g + r of the lane is alive iff its bit in the block's validity words
// is set and it is at most kmax.
template <int NCH>
__device__ __forceinline__ void tile16_softmax(float (&s)[NCH][4], bool full, const uint32_t* valid, int g,
                                               int32_t kmax, float c2, float& mb2, float& sum) {
  const bool up = c2 >= 0.f;
  if (!full) {
    const float dead = up ? -INFINITY : INFINITY;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      const int32_t x = kmax - 16 * ch - 4 * g;   // keys r <= x of this group are in range
      uint32_t w = (valid[ch >> 1] >> (16 * (ch & 1) + 4 * g)) & 15u;
      w &= x < 0 ? 0u : (x >= 3 ? 15u : (2u << x) - 1u);
#pragma unroll
      for (int r = 0; r < 4; ++r) s[ch][r] = ((w >> r) & 1u) ? s[ch][r] : dead;
    }
  }
  float ext = up ? -INFINITY : INFINITY;
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
    for (int r = 0; r < 4; ++r) ext = up ? fmaxf(ext, s[ch][r]) : fminf(ext, s[ch][r]);
#pragma unroll
  for (int x = 16; x <= 32; x *= 2) {
    const float other = __shfl_xor(ext, x, 64);
    ext = up ? fmaxf(ext, other) : fminf(ext, other);
  }
  const bool none = up ? ext == -INFINITY : ext == INFINITY;
  mb2 = none ? -INFINITY : ext * c2;
  const float nref = none ? 0.f : -mb2;
  float sum4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float p = __builtin_amdgcn_exp2f(fmaf(s[ch][r], c2, nref));
      if (!full) p = fmaxf(p, 0.f);
      s[ch][r] = p;
      sum4[r] += p;
    }
  sum = (sum4[0] + sum4[1]) + (sum4[2] + sum4[3]);
  sum += __shfl_xor(sum, 16, 64);
  sum += __shfl_xor(sum, 32, 64);
}

// O^T = V^T . P^T over the NCH chunks; the k index of MFMA (ch, r) is key 16ch + 4g + r.
template <int NCH>
__device__ __forceinline__ void tile16_pv(const float* sv, const float (&s)[NCH][4], int li, int g,
                                          floatx4 (&oacc)[8]) {
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float* vr = &sv[(16 * ch + 4 * g + r) * kVPitch + 4 * li];
      const floatx4 v0 = *reinterpret_cast<const floatx4*>(vr);
      const floatx4 v1 = *reinterpret_cast<const floatx4*>(vr + 64);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const floatx4 acc = (ch == 0 && r == 0) ? zero4v() : oacc[db];
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(db < 4 ? v0[db & 3] : v1[db & 3], s[ch][r], acc, 0, 0, 0);
      }
      if (r & 1) __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Row `row` of the unit from a 16-row tile: lane (li, g) holds d = 16g + 4v +
// (db & 3) + 64 (db >> 2) in oacc[db][v].
__device__ __forceinline__ void tile16_store(const FwdArgs& A, int64_t row0, int32_t row, int g,
                                             const floatx4 (&oacc)[8], float mb2, float sum) {
  float* dst = A.o + (row0 + row) * kD + 16 * g;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    *reinterpret_cast<floatx4*>(dst + 4 * v) = floatx4{oacc[0][v], oacc[1][v], oacc[2][v], oacc[3][v]};
    *reinterpret_cast<floatx4*>(dst + 64 + 4 * v) = floatx4{oacc[4][v], oacc[5][v], oacc[6][v], oacc[7][v]};
  }
  if (g == 0) {
    A.m[row0 + row] = mb2 * kLn2;
    A.l[row0 + row] = sum;
  }
}

// ---- the same tiles from 16-bit pages. The block's K and V rows stay raw
// 16-bit words in LDS, 16 chunks of 8 words a row with no padding. In K,
// chunk c of row r sits at chunk c ^ (r & 15) of the row, which spreads the
// 32 rows of one operand read over all the banks; V is stored as is (an
// operand read of the 32-row tiles covers one whole row, and its addresses
// then fold into immediate offsets; the 16-row tiles' reads of rows four
// apart meet in the same banks, a 2-way conflict, which measured cheaper
// than forming swizzled V addresses). The words go to the 16-bit matrix
// cores as they are (below).
__device__ __forceinline__ int swz16(int row, int chunk) { return row * 128 + ((chunk ^ (row & 15)) << 3); }




// 16-bit pages on the 16-bit matrix cores (v_mfma_f32_32x32x16_bf16 / _f16
// and the 16x16x32 forms): the K and V words enter the products as stored,
// and each fp32 operand is written as a sum of terms of the pages' format by
// repeated rounding toward zero (q three terms, which carry its 24
// significand bits; p two, within 2^-16 of it). A product of two such terms
// is exact in fp32, and the products accumulate in fp32. fp16 terms have a
// narrow range: a tile's q row is first scaled by a power of two 2^sx that
// brings its largest element into [2^14, 2^15), and the row's score factor
// takes 2^-sx back (exactly: a power of two). p lies in [0, 1].
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef unsigned int uintx4v __attribute__((ext_vector_type(4)));
// The word of the high terms of (x0, x1), low half first; x0 and x1 keep the
// remainders (exact in fp32).
template <int KVF>
__device__ __forceinline__ uint32_t split_pair(float& x0, float& x1) {
  if constexpr (KVF == SA_KV_BF16) {
    const float h0 = __uint_as_float(__float_as_uint(x0) & 0xffff0000u);
    const float h1 = __uint_as_float(__float_as_uint(x1) & 0xffff0000u);
    x0 -= h0;
    x1 -= h1;
    return (__float_as_uint(h0) >> 16) | (__float_as_uint(h1) & 0xffff0000u);
  } else {
    const auto h = __builtin_amdgcn_cvt_pkrtz(x0, x1);
    x0 -= (float)h[0];
    x1 -= (float)h[1];
    return __builtin_bit_cast(uint32_t, h);
  }
}
template <int KVF>
__device__ __forceinline__ floatx16 mfma32x32x16(uintx4v a, uintx4v b, const floatx16& c) {
  if constexpr (KVF == SA_KV_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a), __builtin_bit_cast(halfx8, b), c,
                                                  0, 0, 0);
}
template <int KVF>
__device__ __forceinline__ floatx4 mfma16x16x32(uintx4v a, uintx4v b, const floatx4& c) {
  if constexpr (KVF == SA_KV_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(halfx8, a), __builtin_bit_cast(halfx8, b), c,
                                                  0, 0, 0);
}
// The power of two 2^sx that fp16 terms take the q row in (0 for bf16): a
// 32-row tile holds the row in lanes lr and lr + 32 (qr[0..15]), a 16-row
// tile in lanes li + 16g (qr[0..7]).
template <int KVF, bool k16>
__device__ __forceinline__ int q_row_exp(const float4 (&qr)[16]) {
  if constexpr (KVF != SA_KV_F16) {
    return 0;
  } else {
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < (k16 ? 8 : 16); ++i)
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(qr[i].x), fabsf(qr[i].y)), fmaxf(fabsf(qr[i].z), fabsf(qr[i].w))));
    if (k16) mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    int sx = 0;
    if (mx > 0.f && mx <= 3.0e38f) {
      int e;
      (void)frexpf(mx, &e);                     // mx = f * 2^e, f in [0.5, 1)
      sx = 15 - e;
      sx = sx < -120 ? -120 : (sx > 120 ? 120 : sx);
    }
    return sx;
  }
}
// q values (x0..x7) as three terms of the format, words m of term t
template <int KVF>
__device__ __forceinline__ void split_q8(float (&x)[8], int sx, uint32_t (&w)[3][4]) {
  if constexpr (KVF == SA_KV_F16) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = ldexpf(x[e], sx);
  }
#pragma unroll
  for (int t = 0; t < 3; ++t)
#pragma unroll
    for (int m = 0; m < 4; ++m) w[t][m] = split_pair<KVF>(x[2 * m], x[2 * m + 1]);
}

// S^T = K . Q^T with 16-bit K words: step p takes chunk half*8 + p of the
// lane's key row (d = half*64 + 8p .. +7, the k slots of the lane's half) and
// the same d of q, split into three terms at the step. Returns the row's
// score factor (c2, times 2^-sx for fp16).
template <int NKB, int KVF>
__device__ __forceinline__ float tile_scores_m16(const uint16_t* sk, const float4 (&qr)[16], int lr, int half,
                                                 floatx16 (&sacc)[NKB], float c2) {
  const int sx = q_row_exp<KVF, false>(qr);
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) sacc[kb] = zero16();
  uint4 kc[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) kc[kb] = *reinterpret_cast<const uint4*>(&sk[swz16(kb * 32 + lr, half * 8)]);
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    uint4 kn[NKB];
    if (p < 7) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        kn[kb] = *reinterpret_cast<const uint4*>(&sk[swz16(kb * 32 + lr, half * 8 + p + 1)]);
    }
    float x[8] = {qr[2 * p].x, qr[2 * p].y, qr[2 * p].z, qr[2 * p].w,
                  qr[2 * p + 1].x, qr[2 * p + 1].y, qr[2 * p + 1].z, qr[2 * p + 1].w};
    uint32_t w[3][4];
    split_q8<KVF>(x, sx, w);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const uintx4v k{kc[kb].x, kc[kb].y, kc[kb].z, kc[kb].w};
#pragma unroll
      for (int t = 0; t < 3; ++t)
        sacc[kb] = mfma32x32x16<KVF>(k, uintx4v{w[t][0], w[t][1], w[t][2], w[t][3]}, sacc[kb]);
    }
    if (p < 7) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) kc[kb] = kn[kb];
    }
  }
  return KVF == SA_KV_F16 ? ldexpf(c2, -sx) : c2;
}

// tile_pv: lane lr reads words 4 phi(lr) .. + 3 of a key row, with
// phi(8g + 4h + c) = 8g + 2c + h (g, c < 4, h < 2), so output row m of MFMA
// block db stands for d = 4 phi(m) + db: the rows that lanes lr and lr + 32
// hold side by side are adjacent d, and each store of tile_store16 writes 32
// contiguous bytes of a row, as the fp32 tiles' stores do.
__device__ __forceinline__ int pv16_word(int lr) { return 4 * (8 * (lr >> 3) + 2 * (lr & 3) + ((lr >> 2) & 1)); }

// O^T = V^T . P^T with 16-bit V words. Step (kb, u) takes the lane's
// accumulators 8u .. 8u + 7 of block kb: element e stands for key kb*32 +
// 16u + 8(e/4) + 4half + e%4 on both operands (p, split into two terms, and
// the V words of those keys at the lane's words 4 phi(lr) .. +3).
template <int NKB, int KVF>
__device__ __forceinline__ void tile_pv_m16(const uint16_t* sv, const floatx16 (&sacc)[NKB], int lr, int half,
                                            floatx16 (&oacc)[4]) {
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = zero16();
  const int word = pv16_word(lr);
  auto read_v = [&](int kb, int u, uint2 (&dst)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      dst[e] = *reinterpret_cast<const uint2*>(&sv[(kb * 32 + 16 * u + 8 * (e >> 2) + 4 * half + (e & 3)) * 128 + word]);
  };
  uint2 vc[8];
  read_v(0, 0, vc);
#pragma unroll
  for (int st = 0; st < 2 * NKB; ++st) {
    const int kb = st >> 1, u = st & 1;
    uint2 vn[8];
    if (st + 1 < 2 * NKB) read_v((st + 1) >> 1, (st + 1) & 1, vn);
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float a = sacc[kb][8 * u + 2 * m], b = sacc[kb][8 * u + 2 * m + 1];
      ph[m] = split_pair<KVF>(a, b);
      pl[m] = split_pair<KVF>(a, b);
    }
    const uintx4v phi{ph[0], ph[1], ph[2], ph[3]}, plo{pl[0], pl[1], pl[2], pl[3]};
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      // word db of key e's four: half db & 1 of .x (db < 2) or .y
      uint32_t a[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t w0 = db < 2 ? vc[2 * m].x : vc[2 * m].y, w1 = db < 2 ? vc[2 * m + 1].x : vc[2 * m + 1].y;
        a[m] = (db & 1) ? (w0 >> 16) | (w1 & 0xffff0000u) : (w0 & 0xffffu) | (w1 << 16);
      }
      const uintx4v v{a[0], a[1], a[2], a[3]};
      oacc[db] = mfma32x32x16<KVF>(v, phi, oacc[db]);
      oacc[db] = mfma32x32x16<KVF>(v, plo, oacc[db]);
    }
    if (st + 1 < 2 * NKB) {
#pragma unroll
      for (int e = 0; e < 8; ++e) vc[e] = vn[e];
    }
  }
}

// Accumulator i = 4g + c of block db holds d = 4 phi(8g + 4half + c) + db =
// 32g + 8c + 4half + db of row `row`.
__device__ __forceinline__ void tile_store16(const FwdArgs& A, int64_t row0, int32_t row, int half,
                                             const floatx16 (&oacc)[4], float mb2, float sum) {
  float* op = A.o + (row0 + row) * kD + 4 * half;
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *reinterpret_cast<float4*>(op + 32 * g + 8 * c) =
          make_float4(oacc[0][4 * g + c], oacc[1][4 * g + c], oacc[2][4 * g + c], oacc[3][4 * g + c]);
  if (half == 0) {
    A.m[row0 + row] = mb2 * kLn2;
    A.l[row0 + row] = sum;
  }
}



// 16-row tiles with 16-bit words on the 16x16x32 form. Scores: step t (of
// four) takes K words d = 32t + 4g .. +3 and 32t + 16 + 4g .. +3 of the
// lane's key row and q at the same d (q[2t], q[2t + 1]), split into three
// terms once a step for all chunks. Returns the row's score factor.
template <int NCH, int KVF>
__device__ __forceinline__ float tile16_scores_m16(const uint16_t* sk, const float4 (&qr)[16], int li, int g,
                                                   float (&s)[NCH][4], float c2) {
  const int sx = q_row_exp<KVF, true>(qr);
  floatx4 acc[NCH];
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) acc[ch] = zero4v();
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    float x[8] = {qr[2 * t].x, qr[2 * t].y, qr[2 * t].z, qr[2 * t].w,
                  qr[2 * t + 1].x, qr[2 * t + 1].y, qr[2 * t + 1].z, qr[2 * t + 1].w};
    uint32_t w[3][4];
    split_q8<KVF>(x, sx, w);
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      const int row = 16 * ch + li;
      const uint2 wa = *reinterpret_cast<const uint2*>(&sk[swz16(row, 4 * t + (g >> 1)) + 4 * (g & 1)]);
      const uint2 wb = *reinterpret_cast<const uint2*>(&sk[swz16(row, 4 * t + 2 + (g >> 1)) + 4 * (g & 1)]);
      const uintx4v kw{wa.x, wa.y, wb.x, wb.y};
#pragma unroll
      for (int k = 0; k < 3; ++k) acc[ch] = mfma16x16x32<KVF>(kw, uintx4v{w[k][0], w[k][1], w[k][2], w[k][3]}, acc[ch]);
    }
  }
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
    for (int r = 0; r < 4; ++r) s[ch][r] = acc[ch][r];
  return KVF == SA_KV_F16 ? ldexpf(c2, -sx) : c2;
}

// O^T += V^T . P^T, 16-row tiles with 16-bit words: element e of lane group
// g stands for key 16ch + 4g + (e & 3), p's high term for e < 4 and its low
// term for e >= 4 (V's word twice); output row i of block db stands for d =
// 4i + (db & 3) + 64 (db >> 2).
template <int NCH, int KVF>
__device__ __forceinline__ void tile16_pv_m16(const uint16_t* sv, const float (&s)[NCH][4], int li, int g,
                                              floatx4 (&oacc)[8]) {
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    uint2 w0[4], w1[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * ch + 4 * g + r;
      w0[r] = *reinterpret_cast<const uint2*>(&sv[row * 128 + 4 * li]);
      w1[r] = *reinterpret_cast<const uint2*>(&sv[row * 128 + 64 + 4 * li]);
    }
    float x0 = s[ch][0], x1 = s[ch][1], x2 = s[ch][2], x3 = s[ch][3];
    const uint32_t h01 = split_pair<KVF>(x0, x1), h23 = split_pair<KVF>(x2, x3);
    const uint32_t l01 = split_pair<KVF>(x0, x1), l23 = split_pair<KVF>(x2, x3);
    const uintx4v pw{h01, h23, l01, l23};
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      uint32_t wr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint2 x = db < 4 ? w0[r] : w1[r];
        wr[r] = (db & 2) ? x.y : x.x;
      }
      const uint32_t v01 = (db & 1) ? (wr[0] >> 16) | (wr[1] & 0xffff0000u) : (wr[0] & 0xffffu) | (wr[1] << 16);
      const uint32_t v23 = (db & 1) ? (wr[2] >> 16) | (wr[3] & 0xffff0000u) : (wr[2] & 0xffffu) | (wr[3] << 16);
      oacc[db] = mfma16x16x32<KVF>(uintx4v{v01, v23, v01, v23}, pw, ch == 0 ? zero4v() : oacc[db]);
    }
  }
}

// A unit's rows in 16-row quanta, dealt to the four SIMDs of the workgroup in
// near-equal contiguous shares (the unit ends when its largest share does).
// A share of q quanta is q / 2 32-row tiles and, for odd q, one 16-row tile
// last. Waves w and w + 4 of a workgroup run on the same SIMD; share w % 4 is
// theirs and they take its tiles alternately (a wave alone on the SIMD still
// keeps the matrix pipe nearly busy, and 16-row tiles cost more per row).
struct SimdShare {
  int32_t start;     // first row of the share
  int32_t npieces;   // tiles in the share
  int32_t n32;       // 32-row tiles; tile n32, if any, is the 16-row one
};
__device__ __forceinline__ SimdShare simd_share(int32_t rows, int simd) {
  const int32_t quanta = (rows + 15) >> 4, base = quanta >> 2, extra = quanta & 3;
  const int32_t q = base + (simd < extra ? 1 : 0);
  return SimdShare{16 * (simd * base + (simd < extra ? simd : extra)), (q >> 1) + (q & 1), q >> 1};
}

// Blocks of 65..128 keys, fp32 or 16-bit pages (KVF; 16-bit words stay raw in
// LDS, see tile_scores16): the same tiles, with everything a unit reads from
// memory besides q brought into LDS by direct-to-LDS loads
// (global_load_lds: each lane moves 4 or 16 bytes from its own global address
// into LDS; no registers hold the data):
//   - the block-table entries and query ids of the unit two ahead go out
//     when a unit starts, its record at the end of the unit before; the key
//     offsets of the next unit are formed from them when a unit starts;
//   - the next unit's K and V rows go out as soon as every wave has left
//     this unit's tiles, all in flight at once (about 17 wave instructions
//     of 1 KB each for fp32 pages, 8 for 16-bit ones), and one wait and one
//     barrier publish them;
//   - each wave's first q rows of the next unit load after its last QK
//     products of this unit.
// Within a unit the waves run their tiles without further barriers, so the
// two waves of a SIMD drift apart and one's softmax overlaps the other's
// matrix products. The units, sorted largest first by the index build, are
// dealt statically (workgroup g takes unit k*G + g for even k and k*G + G-1-g
// for odd k, G workgroups): near-equal shares without a queue, and every
// lookahead is known.
//
// The padded K and V regions are filled as a whole: 16-byte chunk i of a
// region (row i / pitch, column chunk i % pitch) comes from the key's row, or
// from a zero line for padding, missing keys and the tail of the last
// instruction. A wave waits for its own direct-to-LDS loads with vmcnt (they
// complete in order with its other vector memory operations) and a
// workgroup barrier then publishes them.
constexpr int kSlots = 3;
__device__ const float g_zero_row[kD] = {};

typedef const __attribute__((address_space(1))) void gvoid;
typedef __attribute__((address_space(3))) void lvoid;

// s_waitcnt with vmcnt(N), no wait on the other counters (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Workgroup barrier once this wave's LDS operations have completed (its
// vector memory operations may still be in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// A lane index the compiler cannot see through, so that address arithmetic
// built on it is formed where it is used rather than kept live.
__device__ __forceinline__ int opaque_lane(int lane) {
  asm volatile("" : "+v"(lane));
  return lane;
}

template <int NKB, int KVF>
__global__ __launch_bounds__(512) void k_fwd_mfma_dma(IndexPtrs P, FwdArgs A) {
  constexpr int kWaves = 8;
  constexpr int kThreads = kWaves * 64;
  constexpr int kKeys = NKB * 32;
  constexpr bool kF32 = KVF == SA_KV_F32;
  // wave instructions (64 chunks of 16 bytes) filling the K and V regions:
  // padded fp32 rows, or unpadded rows of 16-bit words
  constexpr int kKInstr = kF32 ? (kKeys * (kKPitch / 4) + 63) / 64 : kKeys / 4;
  constexpr int kVInstr = kF32 ? (kKeys * (kVPitch / 4) + 63) / 64 : kKeys / 4;
  static_assert(kKeys <= kThreads && kMaxUnitEdges <= kThreads, "one key and one edge per thread");
  static_assert(kMaxUnitEdges % 64 == 0, "query ids move in whole waves");
  __shared__ __align__(16) float s_k[kKInstr * 256];
  __shared__ __align__(16) float s_v[kVInstr * 256];
  __shared__ int64_t s_off[kKeys];                   // key row offsets of the next unit (-1: none)
  __shared__ uint32_t s_valid[2][NKB];               // validity bits, by unit parity
  __shared__ int32_t s_rec[kSlots][8];               // records, slot j % 3 for unit j
  __shared__ int32_t s_page[kSlots][kKeys];          // block-table entry of each key
  __shared__ int32_t s_qid[kSlots][kMaxUnitEdges];   // query id of each edge

  const DevHeader* hdr = P.hdr;
  if (hdr->status != SA_OK) return;
  // The units, sorted by size (within groups of (sequence, head) pairs where
  // the sort found the groups balanced: workgroup g, on XCD g % 8, then
  // takes the units of group g % 8, and its XCD's L2 serves their q rows),
  // dealt in a snake: units [lo, hi) to the Gs workgroups of the share.
  const int32_t* sinfo = P.sort_hist + kSortHistInfo;
  const int32_t G = gridDim.x, g = blockIdx.x;
  int32_t lo = 0, hi = hdr->num_units_mfma, Gs = G, gs = g;
  if (sinfo[0] != 0 && G % kSortGroups == 0) {
    lo = sinfo[1 + g % kSortGroups];
    hi = sinfo[2 + g % kSortGroups];
    Gs = G / kSortGroups;
    gs = g / kSortGroups;
  }
  auto unit_at = [&](int32_t k) -> int32_t { return lo + k * Gs + ((k & 1) ? Gs - 1 - gs : gs); };
  if (unit_at(0) >= hi) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, in a scalar register
  const int32_t qhead = A.qhead;
  const int64_t page_stride = (int64_t)A.hkv * A.page_size * kD;
  const float c2 = A.scale_log2;
  const int32_t* units = reinterpret_cast<const int32_t*>(P.units_sorted);   // largest first
  // Per-lane constants (row lane, half of the lanes) are formed again from
  // an opaque lane index where they are used, instead of being kept live
  // across the unit loop: the tile code needs nearly every register.

  // a record from LDS, in scalar registers (the fields are uniform)
  auto unit_of = [&](int sl) {
    const int32_t* r = s_rec[sl];
    return Unit{__builtin_amdgcn_readfirstlane(r[0]), __builtin_amdgcn_readfirstlane(r[1]),
                __builtin_amdgcn_readfirstlane(r[2]), __builtin_amdgcn_readfirstlane(r[3]),
                __builtin_amdgcn_readfirstlane(r[4]), __builtin_amdgcn_readfirstlane(r[5]),
                __builtin_amdgcn_readfirstlane(r[6]), __builtin_amdgcn_readfirstlane(r[7])};
  };
  auto keys_of = [&](int32_t blk, int32_t lk) -> int32_t {
    const int64_t start = (int64_t)blk * A.block_size;
    int64_t end = start + A.block_size;
    end = end < lk ? end : (int64_t)lk;
    return end > start ? (int32_t)(end - start) : 0;
  };
  // ---- metadata, all by direct-to-LDS loads: the record of unit u into
  // slot sl (lanes 0-7 of wave 0), then from it the block-table entry of
  // every key and the query id of every edge
  auto fetch_record = [&](int sl, int32_t u) {
    if (wv == 0 && lane < 8)
      __builtin_amdgcn_global_load_lds((gvoid*)(units + 8 * (int64_t)u + opaque_lane(lane)),
                                       (lvoid*)&s_rec[sl][0], 4, 0, 0);
  };
  auto fetch_lists = [&](int sl, const Unit& U) {
    if (tid < kKeys) {
      const int key = opaque_lane(lane) + 64 * wv;
      const int kk = key < A.block_size ? key : 0;
      const int32_t pgl = (int32_t)div_magic((uint32_t)kk, A.ps_magic);
      __builtin_amdgcn_global_load_lds(
          (gvoid*)(A.block_tables + (int64_t)U.b * A.max_pages + (int64_t)U.blk * A.ppb + pgl),
          (lvoid*)&s_page[sl][64 * wv], 4, 0, 0);
    }
    if (tid < U.e1 - U.e0)
      __builtin_amdgcn_global_load_lds((gvoid*)(P.edges + 2 * ((int64_t)U.e0 + opaque_lane(lane) + 64 * wv)),
                                       (lvoid*)&s_qid[sl][64 * wv], 4, 0, 0);
  };
  // key row offsets and validity bits of the unit in slot sl (parity par)
  auto form_offsets = [&](int sl, int par) {
    if (tid < kKeys) {
      const Unit U = unit_of(sl);
      const int32_t page = s_page[sl][tid];
      int64_t off = -1;
      if (tid < keys_of(U.blk, U.lk) && page >= 0 && page < A.num_pages) {
        const int32_t pgl = (int32_t)div_magic((uint32_t)tid, A.ps_magic);
        off = (int64_t)page * page_stride + (int64_t)U.h * A.page_size * kD + (int64_t)(tid - pgl * A.page_size) * kD;
      }
      s_off[tid] = off;
      const uint64_t bits = __ballot(off >= 0);
      if ((lane & 31) == 0) s_valid[par][tid >> 5] = (uint32_t)(bits >> (lane & 32));
    }
  };
  // ---- direct-to-LDS gather of a block's K and V rows into their padded
  // regions. Every source address is formed (from the key offsets in LDS)
  // before the first load goes out: an LDS read behind a direct-to-LDS load
  // would wait for it.
  auto gather_kv = [&]() __attribute__((always_inline)) {
    constexpr int kPerWave = (kVInstr + kWaves - 1) / kWaves;
    const float* srck[kPerWave];
    const float* srcv[kPerWave];
    // Branch-free: a key without a row reads the zero line (its probability
    // is 0, and its V row must be finite); a padding chunk, never read, and
    // the tail past the last key take any chunk of a row in the block.
    // (pitch4: float4 chunks a padded fp32 row; swizzled: the 16-bit K layout)
    auto src_of = [&](const float* base, int pitch4, int n, bool swizzled) -> const float* {
      const int c = 64 * n + opaque_lane(lane);
      if constexpr (kF32) {
        const int row = c / pitch4, col = c - row * pitch4;
        const int64_t off = s_off[row < kKeys ? row : 0];
        const float* rowp = off >= 0 ? base + off : g_zero_row;
        return rowp + 4 * (col < kD / 4 ? col : kD / 4 - 1);
      } else {
        // chunk c of the region: row c / 16, which holds chunk (c % 16) ^ (row % 16)
        // of the key's row in K and chunk c % 16 in V
        const int row = c >> 4, chunk = (c & 15) ^ (swizzled ? row & 15 : 0);
        const int64_t off = s_off[row];
        const uint16_t* rowp = off >= 0 ? reinterpret_cast<const uint16_t*>(base) + off
                                        : reinterpret_cast<const uint16_t*>(g_zero_row);
        return reinterpret_cast<const float*>(rowp + 8 * chunk);
      }
    };
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int n = i * kWaves + wv;
      srck[i] = src_of(A.k, kKPitch / 4, n < kKInstr ? n : 0, true);
      srcv[i] = src_of(A.v, kVPitch / 4, n < kVInstr ? n : 0, false);
    }
    // the rounds in which every wave has an instruction need no test
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int n = i * kWaves + wv;
      if (i < kKInstr / kWaves || n < kKInstr)
        __builtin_amdgcn_global_load_lds((gvoid*)srck[i], (lvoid*)(s_k + 256 * n), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int n = i * kWaves + wv;
      if (i < kVInstr / kWaves || n < kVInstr)
        __builtin_amdgcn_global_load_lds((gvoid*)srcv[i], (lvoid*)(s_v + 256 * n), 16, 0, 0);
    }
  };
  // q of the lane's row in the piece that starts at row prow of the unit in
  // slot sl: a 32-row tile takes half of row prow + lane % 32 (float4 i at
  // 4i), a 16-row tile row prow + lane % 16 at d = 16t + 4g (float4 t at
  // 16t). Rows past the unit read its last row: they stay in their own lanes
  // and are never stored.
  auto piece_q = [&](int sl, int32_t h, int32_t rows, int32_t prow, bool is16, int32_t* qi_out) -> const float* {
    const int ln = opaque_lane(lane);
    int32_t row = prow + (is16 ? (ln & 15) : (ln & 31));
    row = row < rows ? row : rows - 1;
    const int32_t qi = s_qid[sl][row / qhead];
    *qi_out = qi;
    return A.q + ((int64_t)qi * A.hq + (int64_t)h * qhead + row % qhead) * kD +
           (is16 ? 4 * ((ln >> 4) & 3) : 64 * (ln >> 5));
  };
  // the first q loads of a piece (all of a 16-row tile's), then the rest of a 32-row tile's
  auto load_q_first = [&](const float* qp, bool is16, float4 (&qr)[16]) __attribute__((always_inline)) {
    if (is16) {
#pragma unroll
      for (int i = 0; i < 8; ++i) qr[i] = *reinterpret_cast<const float4*>(qp + 16 * i);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) qr[i] = *reinterpret_cast<const float4*>(qp + 4 * i);
    }
  };
  auto load_q_rest = [&](const float* qp, float4 (&qr)[16]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 8; i < 16; ++i) qr[i] = *reinterpret_cast<const float4*>(qp + 4 * i);
  };

  // ---- prologue: records of units 0..2, lists of units 0 and 1, offsets of
  // unit 0; then unit 0's first q rows, K and V
  fetch_record(0, unit_at(0));
  if (unit_at(1) < hi) fetch_record(1, unit_at(1));
  if (unit_at(2) < hi) fetch_record(2, unit_at(2));
  wait_vm<0>();
  lds_barrier();
  fetch_lists(0, unit_of(0));
  if (unit_at(1) < hi) fetch_lists(1, unit_of(1));
  wait_vm<0>();
  lds_barrier();
  form_offsets(0, 0);
  lds_barrier();
  float4 qr[16];
  int32_t qi = 0;
  const float* qp = nullptr;
  const int simd = wv & 3, second = wv >> 2;   // wave wv runs on SIMD wv % 4 with wave wv ^ 4
  {
    const Unit U0 = unit_of(0);
    const int32_t rows0 = (U0.e1 - U0.e0) * qhead;
    const SimdShare sh = simd_share(rows0, simd);
    if (second < sh.npieces) {
      const bool is16 = second == sh.n32;
      qp = piece_q(0, U0.h, rows0, sh.start + 32 * second, is16, &qi);
      load_q_first(qp, is16, qr);
      if (!is16) load_q_rest(qp, qr);
    }
  }
  gather_kv();

  for (int32_t j = 0;; ++j) {
    if (unit_at(j) >= hi) break;
    const int ms = j % kSlots, ms1 = (j + 1) % kSlots, ms2 = (j + 2) % kSlots;
    const bool has1 = unit_at(j + 1) < hi, has2 = unit_at(j + 2) < hi;
    const bool has3 = unit_at(j + 3) < hi;
    const Unit U = unit_of(ms);
    const int64_t block_start = (int64_t)U.blk * A.block_size;
    const int32_t nkeys = keys_of(U.blk, U.lk);
    const int32_t rows = (U.e1 - U.e0) * qhead;
    const int64_t row0 = (int64_t)U.e0 * qhead;
    const SimdShare sh = simd_share(rows, simd);
    // every key of the block has a row (uniform)
    bool all_rows = true;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) all_rows = all_rows && s_valid[j & 1][kb] == 0xffffffffu;

    // ---- this unit's K and V rows (and this wave's first q rows, the lists
    // of unit j + 1 and the record of unit j + 2): this wave's, then every
    // wave's. Nothing goes to LDS directly from here to the end of the
    // tiles, so no LDS read below waits on memory.
    wait_vm<0>();
    lds_barrier();
    // the next unit's key offsets
    if (has1) form_offsets(ms1, (j + 1) & 1);

    bool q_next = false;   // this wave has requested its first q rows of unit j + 1
    // The q rows of this wave's next piece: its next one in this unit, or
    // its first one in unit j + 1. Returns whether there is one; its kind in nq16.
    auto next_q = [&](int32_t p, bool& nq16) -> bool {
      if (p + 2 < sh.npieces) {
        nq16 = p + 2 == sh.n32;
        qp = piece_q(ms, U.h, rows, sh.start + 32 * (p + 2), nq16, &qi);
        return true;
      }
      if (!has1) return false;
      const Unit U1 = unit_of(ms1);
      const int32_t rows1 = (U1.e1 - U1.e0) * qhead;
      const SimdShare sh1 = simd_share(rows1, simd);
      q_next = true;
      if (second >= sh1.npieces) return false;
      nq16 = second == sh1.n32;
      qp = piece_q(ms1, U1.h, rows1, sh1.start + 32 * second, nq16, &qi);
      return true;
    };
    // this wave's 32-row tiles (every other one of the share), then the
    // share's 16-row tile if it is this wave's turn
    for (int32_t p = second; p < sh.n32; p += 2) {
      const int ln = opaque_lane(lane), lr = ln & 31, half = ln >> 5;
      const int32_t row = sh.start + 32 * p + lr;
      const bool row_ok = row < rows;
      // key k is alive iff it has a row and (causal) block_start + k <= q + delta
      int64_t klim = A.causal ? (int64_t)qi + U.delta - block_start : (int64_t)nkeys - 1;
      klim = klim < (int64_t)nkeys - 1 ? klim : (int64_t)nkeys - 1;
      const int32_t kmaxh = (int32_t)(klim < -1 ? -1 : klim) - 4 * half;
      const bool full = __all(!row_ok || klim >= kKeys - 1) && all_rows;
      floatx16 sacc[NKB];
      float c2t = c2;                  // the row's score factor
      if constexpr (kF32) tile_scores<NKB>(s_k, qr, lr, half, sacc);
      else c2t = tile_scores_m16<NKB, KVF>(reinterpret_cast<const uint16_t*>(s_k), qr, lr, half, sacc, c2);
      // ---- the first half of the next q rows (all of them for a 16-row tile)
      bool nq16 = false;
      const bool nq = next_q(p, nq16);
      if (nq) load_q_first(qp, nq16, qr);
      float mb2, sum;
      tile_softmax<NKB, true>(sacc, full, s_valid[j & 1], half, kmaxh, c2t, mb2, sum);
      floatx16 oacc[kD / 32];
      if constexpr (kF32) tile_pv<NKB>(s_v, sacc, lr, half, oacc);
      else tile_pv_m16<NKB, KVF>(reinterpret_cast<const uint16_t*>(s_v), sacc, lr, half, oacc);
      // the second half, before the stores (a wait for a load also waits
      // for every store issued before it)
      if (nq && !nq16) load_q_rest(qp, qr);
      if (row_ok) {
        if constexpr (kF32) tile_store(A, row0, row, half, oacc, mb2, sum);
        else tile_store16(A, row0, row, half, oacc, mb2, sum);
      }
    }
    if (sh.n32 < sh.npieces && sh.n32 >= second && ((sh.n32 - second) & 1) == 0) {
      const int ln = opaque_lane(lane), li = ln & 15, gq = ln >> 4;
      const int32_t row = sh.start + 32 * sh.n32 + li;
      const bool row_ok = row < rows;
      int64_t klim = A.causal ? (int64_t)qi + U.delta - block_start : (int64_t)nkeys - 1;
      klim = klim < (int64_t)nkeys - 1 ? klim : (int64_t)nkeys - 1;
      const int32_t kmax = (int32_t)(klim < -1 ? -1 : klim);
      const bool full = __all(!row_ok || klim >= kKeys - 1) && all_rows;
      float s16[2 * NKB][4];
      float c2t = c2;                  // the row's score factor
      if constexpr (kF32) tile16_scores<2 * NKB>(s_k, qr, li, gq, s16);
      else c2t = tile16_scores_m16<2 * NKB, KVF>(reinterpret_cast<const uint16_t*>(s_k), qr, li, gq, s16, c2);
      bool nq16 = false;
      const bool nq = next_q(sh.n32, nq16);
      if (nq) load_q_first(qp, nq16, qr);
      float mb2, sum;
      tile16_softmax<2 * NKB>(s16, full, s_valid[j & 1], gq, kmax, c2t, mb2, sum);
      floatx4 o16[8];
      if constexpr (kF32) tile16_pv<2 * NKB>(s_v, s16, li, gq, o16);
      else tile16_pv_m16<2 * NKB, KVF>(reinterpret_cast<const uint16_t*>(s_v), s16, li, gq, o16);
      if (nq && !nq16) load_q_rest(qp, qr);
      if (row_ok) tile16_store(A, row0, row, gq, o16, mb2, sum);
    }
    // ---- every wave has left this unit's tiles: the next unit's K and V
    // rows, the first q rows of waves that had no tile here, the lists of
    // unit j + 2 and the record of unit j + 3 (into this unit's slots). The
    // LDS reads all come before the first direct-to-LDS load.
    lds_barrier();
    if (has1) {
      const Unit U1 = unit_of(ms1);
      const int32_t rows1 = (U1.e1 - U1.e0) * qhead;
      const SimdShare sh1 = simd_share(rows1, simd);
      const bool load_first_q = !q_next && second < sh1.npieces;
      const bool first16 = second == sh1.n32;
      if (load_first_q) qp = piece_q(ms1, U1.h, rows1, sh1.start + 32 * second, first16, &qi);
      Unit U2{};
      if (has2) U2 = unit_of(ms2);
      gather_kv();
      if (has2) fetch_lists(ms2, U2);
      if (load_first_q) {
        load_q_first(qp, first16, qr);
        if (!first16) load_q_rest(qp, qr);
      }
    }
    if (has3) fetch_record(ms, unit_at(j + 3));
  }
  // no direct-to-LDS load may outlive the workgroup's LDS
  wait_vm<0>();
}

// Other geometries on the matrix cores: head_dim 64, 128 or 256 and blocks of
// any size (for head_dim 128, those of more than 128 keys). The block goes
// through LDS in chunks of 32 * NKB keys, one after the other; a 32-row tile
// keeps its row max, row sum and unnormalised output in registers across the
// chunks and rescales them when a later chunk raises the max (the online
// softmax of the combine, here inside one block), so the partials are those
// of the whole block: max over its alive scores, the sum of exp(s - max) and
// the weighted sum of V rows. Same tile layout as above (S^T = K . Q^T,
// O^T = V^T . P^T on v_mfma_f32_32x32x2f32), with the q row and the output
// accumulators held across the chunks; head_dim 128 and 256 run four waves a
// workgroup (one a SIMD) for their registers, head_dim 64 eight. The build caps the units of
// multi-chunk blocks at one tile a wave, so each chunk is gathered once a
// unit; a one-chunk block is gathered once for all of a unit's tiles. The
// gathers go through registers (16-bit pages are converted there).
template <int D, int NKB, int WAVES, int KVF>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(WAVES == 4 ? 1 : 2)))
void k_fwd_mfma_gen(IndexPtrs P, FwdArgs A) {
  constexpr int kThreads = WAVES * 64;
  constexpr int C = NKB * 32;                       // keys a chunk
  constexpr int KP = D + 4, VP = D + 8;             // LDS row pitches (floats), as above
  constexpr int kIters = C * (D / 4) / kThreads;    // gather float4 per thread (K and V each)
  static_assert(C * (D / 4) % kThreads == 0 && kThreads % (D / 4) == 0, "gather tiling");
  __shared__ __align__(16) float s_k[C * KP];
  __shared__ __align__(16) float s_v[C * VP];
  __shared__ int64_t s_off[C];
  __shared__ int32_t s_qid[kMaxUnitEdges];
  __shared__ uint32_t s_valid[NKB];

  const DevHeader* hdr = P.hdr;
  if (hdr->status != SA_OK) return;
  const int32_t num_units = hdr->num_units_mfma;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int lr = lane & 31, half = lane >> 5;
  const int32_t qhead = A.qhead;
  const int64_t page_stride = (int64_t)A.hkv * A.page_size * D;
  const float c2 = A.scale_log2;
  const int32_t nchunks = (A.block_size + C - 1) / C;

  // row offsets and validity bits of chunk c's keys (key c*C + i of the block)
  auto chunk_meta = [&](const Unit& U, int32_t nkeys, int32_t c) {
    for (int i = tid; i < C; i += kThreads) {
      const int32_t key = c * C + i;
      int64_t off = -1;
      if (key < nkeys) {
        const int32_t pgl = (int32_t)div_magic((uint32_t)key, A.ps_magic);
        const int32_t page = A.block_tables[(int64_t)U.b * A.max_pages + (int64_t)U.blk * A.ppb + pgl];
        if (page >= 0 && page < A.num_pages)
          off = (int64_t)page * page_stride + (int64_t)U.h * A.page_size * D + (int64_t)(key - pgl * A.page_size) * D;
      }
      s_off[i] = off;
      const uint64_t bits = __ballot(off >= 0);
      if ((lane & 31) == 0) s_valid[i >> 5] = (uint32_t)(bits >> (lane & 32));
    }
  };
  // the chunk's K and V rows into LDS (zero rows where a key has none), in
  // batches of kBatch float4 of each, so that the registers they take stay
  // few next to the q row and the output held across the chunks
  constexpr int kBatch = kIters < 4 ? kIters : 4;
  static_assert(kIters % kBatch == 0, "gather batches");
  auto gather = [&]() {
    const int c4 = tid % (D / 4);
#pragma unroll
    for (int i0 = 0; i0 < kIters; i0 += kBatch) {
      float4 kv[kBatch], vv[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int64_t off = s_off[(tid + (i0 + i) * kThreads) / (D / 4)];
        kv[i] = off >= 0 ? load_kv4<KVF>(A.k, off + c4 * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
        vv[i] = off >= 0 ? load_kv4<KVF>(A.v, off + c4 * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int key = (tid + (i0 + i) * kThreads) / (D / 4);
        *reinterpret_cast<float4*>(&s_k[key * KP + c4 * 4]) = kv[i];
        *reinterpret_cast<float4*>(&s_v[key * VP + c4 * 4]) = vv[i];
      }
      __builtin_amdgcn_sched_barrier(0);    // one batch in registers at a time
    }
  };

  for (int32_t u = blockIdx.x; u < num_units; u += gridDim.x) {
    const Unit U = P.units_mfma[u];
    const int64_t block_start = (int64_t)U.blk * A.block_size;
    int64_t block_end = block_start + A.block_size;
    block_end = block_end < U.lk ? block_end : (int64_t)U.lk;
    const int32_t nkeys = block_end > block_start ? (int32_t)(block_end - block_start) : 0;
    const int32_t n_e = U.e1 - U.e0;
    const int32_t rows = n_e * qhead;
    const int64_t row0 = (int64_t)U.e0 * qhead;
    const int32_t ntiles = (rows + 31) / 32;
    const int32_t rounds = (ntiles + WAVES - 1) / WAVES;

    __syncthreads();                                  // the previous unit's LDS reads are done
    for (int e = tid; e < n_e; e += kThreads) s_qid[e] = P.edges[2 * (int64_t)(U.e0 + e)];
    if (nchunks == 1) {
      chunk_meta(U, nkeys, 0);
      __syncthreads();
      gather();
    }
    __syncthreads();

    for (int32_t rd = 0; rd < rounds; ++rd) {
      const int32_t tile = rd * WAVES + wv;
      const bool has = tile < ntiles;
      const int32_t row = tile * 32 + lr;
      const bool row_ok = row < rows;
      // q of the lane's row (rows past the unit read its last row; never stored)
      float4 qr[D / 8];
      int32_t qi = 0;
      if (has) {
        const int32_t rr = row < rows ? row : rows - 1;
        qi = s_qid[rr / qhead];
        const float* qp = A.q + ((int64_t)qi * A.hq + (int64_t)U.h * qhead + rr % qhead) * D + half * (D / 2);
#pragma unroll
        for (int i = 0; i < D / 8; ++i) qr[i] = *reinterpret_cast<const float4*>(qp + 4 * i);
      }
      // last alive key of the lane's row within the block (causal bound, valid range)
      int64_t klim = A.causal ? (int64_t)qi + U.delta - block_start : (int64_t)nkeys - 1;
      klim = klim < (int64_t)nkeys - 1 ? klim : (int64_t)nkeys - 1;
      floatx16 oacc[D / 32];
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] = zero16();
      float m_run = -INFINITY, l_run = 0.f;           // base-2, scaled units

      for (int32_t c = 0; c < nchunks; ++c) {
        if (nchunks > 1) {
          __syncthreads();                            // the previous chunk's LDS reads are done
          chunk_meta(U, nkeys, c);
          __syncthreads();
          gather();
          __syncthreads();
        }
        if (!has) continue;
        uint32_t vm[NKB];
        bool all_rows;
        lane_key_bits<NKB>(s_valid, half, vm, all_rows);
        const int64_t kl = klim - (int64_t)c * C;      // last alive key index within this chunk
        const int32_t kmaxh = (int32_t)(kl < -1 ? -1 : (kl > C - 1 ? C - 1 : kl)) - 4 * half;
        const bool full = __all(!row_ok || kl >= C - 1) && all_rows;
        floatx16 sacc[NKB];
        tile_scores<NKB, D>(s_k, qr, lr, half, sacc);
        // scaled scores (dead keys -inf), the chunk's max, and the running
        // max, sum and output brought to the new max
        float ext = -INFINITY;
        if (full) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              sacc[kb][r] *= c2;
              ext = fmaxf(ext, sacc[kb][r]);
            }
        } else {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            uint32_t w = vm[kb];
            asm volatile("" : "+v"(w));
            const uint32_t aw = w & keys_upto(kmaxh - kb * 32);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              sacc[kb][r] = ((aw >> r) & 1u) ? sacc[kb][r] * c2 : -INFINITY;
              ext = fmaxf(ext, sacc[kb][r]);
            }
          }
        }
        ext = fmaxf(ext, __shfl_xor(ext, 32, 64));
        const float m_new = fmaxf(m_run, ext);
        const bool none = m_new == -INFINITY;
        const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);   // 0 when m_run = -inf
        const float nref = none ? 0.f : -m_new;
        float sum4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(sacc[kb][r] + nref);           // exp2(-inf) = 0
            sacc[kb][r] = p;
            sum4[r & 3] += p;
          }
        float sum = (sum4[0] + sum4[1]) + (sum4[2] + sum4[3]);
        sum += __shfl_xor(sum, 32, 64);
        l_run = l_run * alpha + sum;
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        tile_pv<NKB, D>(s_v, sacc, lr, half, oacc, true);
      }
      if (has && row_ok) tile_store<D>(A, row0, row, half, oacc, m_run, l_run);
    }
  }
}

// Blocks of up to 64 keys: 16-row tiles on v_mfma_f32_16x16x4f32, so that
// units of 17..64 rows (most units of mixed batches) keep 2..4 waves busy.
// The block's K and V are staged in LDS once per unit as above; each wave then
// computes whole 16-row tiles against every key, with this operand layout
// (its operands come from LDS, so their order does not affect the loads):
//   S^T[key, row]: MFMA t, component c, lane group g takes d = 16t + 4g + c
//   O^T[d, row]:   output row i of MFMA block db stands for d = 4i + (db & 3) + 64 (db >> 2)
// and an exact softmax over the block from register-resident scores.
template <int NKB, int KVF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_fwd_mfma16(IndexPtrs P, FwdArgs A) {
  constexpr int kWaves = 4;
  constexpr int kThreads = 256;
  constexpr int kKeys = NKB * 32;
  constexpr int kChunks = kKeys / 16;     // 16-key chunks
  constexpr int kIters = kKeys * (kD / 4) / kThreads;   // gather float4 per thread (K and V each)
  static_assert(kKeys * (kD / 4) % kThreads == 0, "gather tiling");
  __shared__ __align__(16) float s_k[kKeys * kKPitch];
  __shared__ __align__(16) float s_v[kKeys * kVPitch];
  __shared__ int64_t s_off[2][kKeys];     // key row offsets (-1: none) of units j and j+1
  __shared__ int32_t s_rec[3][8];         // records of units j, j+1, j+2
  __shared__ int32_t s_qid[2][kMaxUnitEdges];   // query id of each edge of units j and j+1

  DevHeader* hdr = P.hdr;
  if (hdr->status != SA_OK) return;
  const int32_t num_units = hdr->num_units_mfma;
  const int32_t G = gridDim.x;
  const int32_t u0 = blockIdx.x;
  if (u0 >= num_units) return;
  const int32_t n_units = (num_units - u0 + G - 1) / G;   // units u0, u0 + G, ...
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int li = lane & 15, g = lane >> 4;
  const int32_t qhead = A.qhead;
  const int64_t page_stride = (int64_t)A.hkv * A.page_size * kD;
  const int32_t* units = reinterpret_cast<const int32_t*>(P.units_mfma);

  auto unit_of = [&](int slot) { const int32_t* r = s_rec[slot]; return Unit{r[0], r[1], r[2], r[3], r[4], r[5], r[6], r[7]}; };
  auto keys_of = [&](const Unit& U) -> int32_t {
    const int64_t start = (int64_t)U.blk * A.block_size;
    int64_t end = start + A.block_size;
    end = end < U.lk ? end : (int64_t)U.lk;
    return end > start ? (int32_t)(end - start) : 0;
  };
  // block-table entry of key `key` (clamped into the block) and the key's row offset
  auto page_of = [&](const Unit& U, int key) -> int32_t {
    const int kk = key < A.block_size ? key : 0;
    const int32_t pgl = (int32_t)div_magic((uint32_t)kk, A.ps_magic);
    return A.block_tables[(int64_t)U.b * A.max_pages + (int64_t)U.blk * A.ppb + pgl];
  };
  auto key_off = [&](const Unit& U, int key, int32_t page) -> int64_t {
    if (key >= keys_of(U) || page < 0 || page >= A.num_pages) return -1;
    const int32_t pgl = (int32_t)div_magic((uint32_t)key, A.ps_magic);
    return (int64_t)page * page_stride + (int64_t)U.h * A.page_size * kD + (int64_t)(key - pgl * A.page_size) * kD;
  };
  auto load_kv = [&](int sl, float4 (&kv)[kIters], float4 (&vv)[kIters]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      const int x = tid + i * kThreads, key = x / (kD / 4), c4 = x % (kD / 4);
      const int64_t off = s_off[sl][key];
      kv[i] = off >= 0 ? load_kv4<KVF>(A.k, off + c4 * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
      vv[i] = off >= 0 ? load_kv4<KVF>(A.v, off + c4 * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };

  // ---- prologue: records of units 0..2, key offsets of units 0 and 1, K/V of unit 0
  if (tid < 8) {
    s_rec[0][tid] = units[8 * (int64_t)u0 + tid];
    if (n_units > 1) s_rec[1][tid] = units[8 * (int64_t)(u0 + G) + tid];
    if (n_units > 2) s_rec[2][tid] = units[8 * (int64_t)(u0 + 2 * G) + tid];
  }
  __syncthreads();
  for (int key = tid; key < kKeys; key += kThreads) {
    const Unit U0 = unit_of(0);
    s_off[0][key] = key_off(U0, key, page_of(U0, key));
    if (n_units > 1) {
      const Unit U1 = unit_of(1);
      s_off[1][key] = key_off(U1, key, page_of(U1, key));
    }
  }
  for (int e = tid; e < kMaxUnitEdges; e += kThreads) {
    const Unit U0 = unit_of(0);
    if (e < U0.e1 - U0.e0) s_qid[0][e] = P.edges[2 * (int64_t)(U0.e0 + e)];
    if (n_units > 1) {
      const Unit U1 = unit_of(1);
      if (e < U1.e1 - U1.e0) s_qid[1][e] = P.edges[2 * (int64_t)(U1.e0 + e)];
    }
  }
  __syncthreads();
  float4 kv[kIters], vv[kIters];
  load_kv(0, kv, vv);

  for (int32_t j = 0; j < n_units; ++j) {
    const int cur = j & 1, nxt = cur ^ 1;
    const int rs = j % 3, rs2 = (j + 2) % 3;
    // ---- K/V of unit j into LDS
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      const int x = tid + i * kThreads, key = x / (kD / 4), c4 = x % (kD / 4);
      *reinterpret_cast<float4*>(&s_k[key * kKPitch + c4 * 4]) = kv[i];
      *reinterpret_cast<float4*>(&s_v[key * kVPitch + c4 * 4]) = vv[i];
    }
    __syncthreads();
    // ---- ahead: K/V of unit j+1, block-table entries of unit j+2, record of unit j+3
    if (j + 1 < n_units) load_kv(nxt, kv, vv);
    int32_t pre_page = 0, pre_rec = 0;
    int32_t pre_qid[kMaxUnitEdges / kThreads];
    const bool has2 = j + 2 < n_units, has3 = j + 3 < n_units;
    if (has2) {
      const Unit U2 = unit_of(rs2);
      if (tid < kKeys) pre_page = page_of(U2, tid);
#pragma unroll
      for (int k = 0; k < kMaxUnitEdges / kThreads; ++k) {
        const int e = tid + k * kThreads;
        pre_qid[k] = e < U2.e1 - U2.e0 ? P.edges[2 * (int64_t)(U2.e0 + e)] : 0;
      }
    }
    if (has3 && tid < 8) pre_rec = units[8 * (int64_t)(u0 + (j + 3) * G) + tid];

    // ---- the tiles of unit j
    const Unit U = unit_of(rs);
    const int32_t nkeys = keys_of(U);
    const int64_t block_start = (int64_t)U.blk * A.block_size;
    const int32_t rows = (U.e1 - U.e0) * qhead;
    const int64_t row0 = (int64_t)U.e0 * qhead;
    const int32_t ntiles = (rows + 15) / 16;
    for (int32_t tile = wv; tile < ntiles; tile += kWaves) {
      const int32_t row = tile * 16 + li;
      const bool row_ok = row < rows;
      const int32_t qi = row_ok ? s_qid[cur][row / qhead] : 0;   // staged with the unit
      const float* qp = A.q + ((int64_t)qi * A.hq + (int64_t)U.h * qhead + (row_ok ? row % qhead : 0)) * kD + 4 * g;
      floatx4 qr[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) qr[t] = row_ok ? *reinterpret_cast<const floatx4*>(qp + 16 * t) : zero4v();
      int64_t klim = A.causal ? (int64_t)qi + U.delta - block_start : (int64_t)nkeys - 1;
      klim = klim < (int64_t)nkeys - 1 ? klim : (int64_t)nkeys - 1;
      const int32_t kmax = (int32_t)(klim < -1 ? -1 : klim);

      // ---- scores of every key: S^T = K . Q^T per 16-key chunk
      float sreg[kChunks][4];
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        floatx4 sa0 = zero4v(), sa1 = zero4v();
        const float* kr = &s_k[(16 * c + li) * kKPitch + 4 * g];
#pragma unroll
        for (int t = 0; t < 8; t += 2) {
          const floatx4 ka = *reinterpret_cast<const floatx4*>(kr + 16 * t);
          const floatx4 kb = *reinterpret_cast<const floatx4*>(kr + 16 * (t + 1));
          sa0 = __builtin_amdgcn_mfma_f32_16x16x4f32(ka.x, qr[t].x, sa0, 0, 0, 0);
          sa1 = __builtin_amdgcn_mfma_f32_16x16x4f32(kb.x, qr[t + 1].x, sa1, 0, 0, 0);
          sa0 = __builtin_amdgcn_mfma_f32_16x16x4f32(ka.y, qr[t].y, sa0, 0, 0, 0);
          sa1 = __builtin_amdgcn_mfma_f32_16x16x4f32(kb.y, qr[t + 1].y, sa1, 0, 0, 0);
          sa0 = __builtin_amdgcn_mfma_f32_16x16x4f32(ka.z, qr[t].z, sa0, 0, 0, 0);
          sa1 = __builtin_amdgcn_mfma_f32_16x16x4f32(kb.z, qr[t + 1].z, sa1, 0, 0, 0);
          sa0 = __builtin_amdgcn_mfma_f32_16x16x4f32(ka.w, qr[t].w, sa0, 0, 0, 0);
          sa1 = __builtin_amdgcn_mfma_f32_16x16x4f32(kb.w, qr[t + 1].w, sa1, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);   // bound how far LDS reads run ahead
        const floatx4 sv = sa0 + sa1;   // lane (li, g), reg r: key 16c + 4g + r, row li
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = 16 * c + 4 * g + r;
          const bool alive = row_ok && key <= kmax && s_off[cur][key] >= 0;
          sreg[c][r] = alive ? sv[r] * A.scale_log2 : -INFINITY;
        }
      }
      // ---- softmax of row li over the block (base 2)
      float mx = -INFINITY;
#pragma unroll
      for (int c = 0; c < kChunks; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sreg[c][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      float ls = 0.f;
#pragma unroll
      for (int c = 0; c < kChunks; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = sreg[c][r] == -INFINITY ? 0.f : exp2f(sreg[c][r] - mx);
          sreg[c][r] = p;
          ls += p;
        }
      ls += __shfl_xor(ls, 16, 64);
      ls += __shfl_xor(ls, 32, 64);

      // ---- O^T = V^T . P^T
      floatx4 oacc[8];
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float* vr = &s_v[(16 * c + 4 * g + r) * kVPitch + 4 * li];
          const floatx4 v0 = *reinterpret_cast<const floatx4*>(vr);
          const floatx4 v1 = *reinterpret_cast<const floatx4*>(vr + 64);
#pragma unroll
          for (int db = 0; db < 8; ++db) {
            const floatx4 acc = (c == 0 && r == 0) ? zero4v() : oacc[db];
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(db < 4 ? v0[db & 3] : v1[db & 3], sreg[c][r],
                                                            acc, 0, 0, 0);
          }
          if (r & 1) __builtin_amdgcn_sched_barrier(0);
        }
      }
      // ---- the tile's partial rows: lane (li, g) holds row li,
      // d = 16g + 4v + (db & 3) + 64 (db >> 2) in oacc[db][v]
      if (row_ok) {
        float* dst = A.o + (row0 + row) * kD + 16 * g;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          *reinterpret_cast<floatx4*>(dst + 4 * v) = floatx4{oacc[0][v], oacc[1][v], oacc[2][v], oacc[3][v]};
          *reinterpret_cast<floatx4*>(dst + 64 + 4 * v) = floatx4{oacc[4][v], oacc[5][v], oacc[6][v], oacc[7][v]};
        }
        if (g == 0) {
          A.m[row0 + row] = mx == -INFINITY ? -INFINITY : mx * kLn2;
          A.l[row0 + row] = ls;
        }
      }
    }
    __syncthreads();   // every read of s_k, s_v, s_off[cur], s_qid[cur] and s_rec[rs] is done
    // ---- stage unit j+2's key offsets and query ids, and unit j+3's record
    if (has2) {
      if (tid < kKeys) s_off[cur][tid] = key_off(unit_of(rs2), tid, pre_page);
#pragma unroll
      for (int k = 0; k < kMaxUnitEdges / kThreads; ++k) s_qid[cur][tid + k * kThreads] = pre_qid[k];
    }
    if (has3 && tid < 8) s_rec[rs][tid] = pre_rec;
  }
}

template <int NKB, int KVF>
hipError_t launch_mfma16_kv(const IndexPtrs& P, const FwdArgs& a, hipStream_t s, unsigned cus) {
  static thread_local int per_cu = 0;
  if (per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_fwd_mfma16<NKB, KVF>, 256, 0) != hipSuccess || n < 1)
      n = 1;
    per_cu = n;
  }
  hipLaunchKernelGGL((k_fwd_mfma16<NKB, KVF>), dim3((unsigned)per_cu * cus), dim3(256), 0, s, P, a);
  return hipGetLastError();
}

template <int NKB>
hipError_t launch_mfma16_t(const IndexPtrs& P, const FwdArgs& a, hipStream_t s, unsigned cus) {
  switch (a.kv_format) {
    case SA_KV_BF16: return launch_mfma16_kv<NKB, SA_KV_BF16>(P, a, s, cus);
    case SA_KV_F16: return launch_mfma16_kv<NKB, SA_KV_F16>(P, a, s, cus);
    default: return launch_mfma16_kv<NKB, SA_KV_F32>(P, a, s, cus);
  }
}

template <int NKB, int KVF>
hipError_t launch_mfma_dma_kv(const IndexPtrs& P, const FwdArgs& a, hipStream_t s, unsigned cus) {
  static thread_local int per_cu = 0;
  if (per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_fwd_mfma_dma<NKB, KVF>, 512, 0) != hipSuccess || n < 1)
      n = 1;
    per_cu = n;
  }
  hipLaunchKernelGGL((k_fwd_mfma_dma<NKB, KVF>), dim3((unsigned)per_cu * cus), dim3(512), 0, s, P, a);
  return hipGetLastError();
}

template <int NKB>
hipError_t launch_mfma_dma(const IndexPtrs& P, const FwdArgs& a, hipStream_t s, unsigned cus) {
  switch (a.kv_format) {
    case SA_KV_BF16: return launch_mfma_dma_kv<NKB, SA_KV_BF16>(P, a, s, cus);
    case SA_KV_F16: return launch_mfma_dma_kv<NKB, SA_KV_F16>(P, a, s, cus);
    default: return launch_mfma_dma_kv<NKB, SA_KV_F32>(P, a, s, cus);
  }
}

template <int D, int NKB, int WAVES>
hipError_t launch_mfma_gen(const IndexPtrs& P, const FwdArgs& a, hipStream_t s, unsigned cus) {
  auto launch = [&](auto kernel) -> hipError_t {
    static thread_local int per_cu = 0;
    if (per_cu == 0) {
      int n = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, WAVES * 64, 0) != hipSuccess || n < 1) n = 1;
      per_cu = n;
    }
    hipLaunchKernelGGL(kernel, dim3((unsigned)per_cu * cus), dim3(WAVES * 64), 0, s, P, a);
    return hipGetLastError();
  };
  switch (a.kv_format) {
    case SA_KV_BF16: return launch(k_fwd_mfma_gen<D, NKB, WAVES, SA_KV_BF16>);
    case SA_KV_F16: return launch(k_fwd_mfma_gen<D, NKB, WAVES, SA_KV_F16>);
    default: return launch(k_fwd_mfma_gen<D, NKB, WAVES, SA_KV_F32>);
  }
}

}  // namespace

bool mfma_enabled() { return true; }

bool mfma_general_fits(int head_dim, int block_size) {
  return (head_dim == 64 || head_dim == 128 || head_dim == 256) &&
         !(head_dim == kD && block_size <= kMaxKeys);
}

int mfma_general_tile_rows(int head_dim) { return head_dim == 64 ? 8 * 32 : 4 * 32; }

int mfma_general_chunk_keys(int head_dim, int block_size) {
  if (head_dim == 256) return block_size <= 32 ? 32 : 64;
  if (head_dim == 64) return block_size <= 64 ? 64 : 128;
  return 128;
}

hipError_t launch_forward_mfma(const sa_index* idx, const FwdArgs& a, hipStream_t s,
                               unsigned grid) {
  const IndexPtrs P = index_ptrs(idx);
  if (mfma_general_fits(a.head_dim, a.block_size)) {
    const int chunk = mfma_general_chunk_keys(a.head_dim, a.block_size);
    if (a.head_dim == 64) return chunk == 64 ? launch_mfma_gen<64, 2, 8>(P, a, s, grid)
                                             : launch_mfma_gen<64, 4, 8>(P, a, s, grid);
    if (a.head_dim == 128) return launch_mfma_gen<128, 4, 4>(P, a, s, grid);
    return chunk == 32 ? launch_mfma_gen<256, 1, 4>(P, a, s, grid) : launch_mfma_gen<256, 2, 4>(P, a, s, grid);
  }
  if (a.head_dim != kD || a.block_size > kMaxKeys) return hipErrorInvalidValue;
  const int nkb = (a.block_size + 31) / 32;
  if (nkb <= 1) return launch_mfma16_t<1>(P, a, s, grid);
  if (nkb <= 2) return launch_mfma16_t<2>(P, a, s, grid);
  if (nkb <= 3) return launch_mfma_dma<3>(P, a, s, grid);
  return launch_mfma_dma<4>(P, a, s, grid);
}

}  // namespace sa
