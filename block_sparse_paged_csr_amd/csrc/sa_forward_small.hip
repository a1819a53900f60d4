// KV-outer forward for small units: head_dim 128, blocks of at most 64 keys,
// at most 16 rows (edges * qhead) per unit. This covers decode-style batches,
// where each selected block serves one query or a few.
//
// Per unit it computes the partials (o, m, l) of alice-llm 2.0.0 forward.rs
// process_work_unit over the block's valid, causally alive positions, like the
// other forward kernels.
//
// One wavefront per unit: the four waves of a workgroup run their own unit
// streams (units w0, w0 + NW, w0 + 2 NW, ... for NW waves in the grid), kept
// in step by one workgroup barrier per unit and sharing nothing else. The unit's (up to) 16 rows form one 16x16 tile on
// fp32 matrix cores (v_mfma_f32_16x16x4f32) and its block is streamed in
// pieces of 16 keys: first the K pieces (scores of all keys stay in registers),
// then the exact softmax over the block, then the V pieces. The contraction
// index d is permuted so that each lane reads 8 consecutive elements of a
// row per pair of register groups (one 16-byte load for 16-bit pages, two
// for fp32):
//   S^T[key, row] = K[key, :] . Q[row, :]   register group i, component c, lane group
//                                           g = lane/16 takes d = 32 (i >> 1) + 8g +
//                                           4 (i & 1) + c (q loaded the same way)
//   O^T[d, row] += V[key, d] * P[row, key]  output row i of MFMA block db stands for
//                                           d = 8i + db
// Every d is taken once on both sides, so the sums are those of the method.
// With 16-bit pages the pieces keep their words, and the products run on the
// 16-bit matrix cores (v_mfma_f32_16x16x32_bf16 / _f16, helpers below).
// Latency: the next piece (the next unit's first K piece at the end of a unit)
// is in flight while a piece computes, and the next unit's query rows load
// during the V pieces. Unit metadata runs further ahead through small per-wave
// LDS rings: at a unit's first piece the record of unit j+3 and the
// block-table entries and query ids of unit j+2 are fetched. A unit's pieces
// are unrolled, so every load count is static and the compiler waits for
// exactly the piece it needs.
#include <type_traits>

#include "sa_internal.h"

namespace sa {

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
// Pointers into device global memory, so loads through them (also through a
// pointer chosen between two of them) stay global_load rather than flat_load.
typedef const __attribute__((address_space(1))) float gfloat;
typedef const __attribute__((address_space(1))) floatx4 gfloatx4;
typedef const __attribute__((address_space(1))) int32_t gint;

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kPiece = 16;          // keys per piece
constexpr int kMaxKeys = 64;        // block_size <= 64
constexpr int kRows = 16;           // rows per unit
constexpr int kRecRing = 4;         // records of units j .. j+3
constexpr int kMetaRing = 3;        // key offsets / validity / query ids of units j .. j+2
constexpr float kLn2 = 0.69314718055994530942f;

// A lane with nothing to load reads this zero line instead and gets zeros,
// so every load is issued and the loads stay countable.
__device__ const float g_zero[kD] = {};
__device__ inline gfloat* zero_line() { return (gfloat*)g_zero; }

constexpr int kStageStride = kD + 4;  // padded row of the output staging tile

struct WaveLds {
  int32_t rec[kRecRing][8];         // Unit records
  int64_t ko[kMetaRing][kMaxKeys];  // element offset of each key's K/V row, or -1
  uint64_t vm[kMetaRing];           // bit t: key t of the block is inside it and on a page
  int32_t qi[kMetaRing][kRows];     // query id of each row
  float ostage[kRows][kStageStride];  // the unit's o tile on its way out
};

// K/V storage formats: fp32 as the pages define them, or 16-bit storage
// (bf16 / IEEE fp16), multiplied as stored on the 16-bit matrix cores.
enum KvFormat : int { kKvF32 = SA_KV_F32, kKvBf16 = SA_KV_BF16, kKvF16 = SA_KV_F16 };

typedef const __attribute__((address_space(1))) uint16_t gu16;
typedef unsigned int uintx2 __attribute__((ext_vector_type(2)));
typedef unsigned int uintx4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) uintx4 guint4;

// One piece of a unit in registers: 8 groups of 4 elements a lane.
//   K piece c: x[i] = K[key 16c + li][32 (i >> 1) + 8g + 4 (i & 1) .. +3]
//   V piece c: x[2r + h] = V[key 16c + 4g + r][8li + 4h .. +3]
// fp32 keeps a float4 per group, 16-bit formats the raw 8 bytes (elements
// 0, 1 in .x, 2, 3 in .y, low half first).
template <int KVF>
struct PieceT {
  floatx4 x[8];
};
template <>
struct PieceT<kKvBf16> {
  uintx2 x[8];
};
template <>
struct PieceT<kKvF16> {
  uintx2 x[8];
};

// Element c of group i of an fp32 piece.
__device__ inline float kv_elem(const PieceT<kKvF32>& pc, int i, int c) { return pc.x[i][c]; }

template <int N>
using IC = std::integral_constant<int, N>;

__device__ inline Unit as_unit(const int32_t* r) {
  return Unit{r[0], r[1], r[2], r[3], r[4], r[5], r[6], r[7]};
}
__device__ inline floatx4 zero4() {
  floatx4 z;
  z[0] = z[1] = z[2] = z[3] = 0.f;
  return z;
}

// 16-bit pages on the 16-bit matrix cores (v_mfma_f32_16x16x32_bf16 / _f16):
// the K and V words enter the products as stored, and each fp32 operand is
// written as a sum of terms of the pages' format by repeated rounding toward
// zero (q three terms, which carry its 24 significand bits; p two, within
// 2^-16 of it). A product of two such terms is exact in fp32, and the
// products accumulate in fp32. fp16 terms have a narrow range: a q row is
// first scaled by a power of two 2^sx that brings its largest element into
// [2^14, 2^15), and the scores take 2^-sx back in the factor that scales
// them (exactly: a power of two). p lies in [0, 1].
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
__device__ inline float bf16_trunc(float x) { return __uint_as_float(__float_as_uint(x) & 0xffff0000u); }
// The word of the high terms of (x0, x1), low half first; x0 and x1 keep the
// remainders (exact in fp32).
template <int KVF>
__device__ inline uint32_t split_pair(float& x0, float& x1) {
  if constexpr (KVF == kKvBf16) {
    const float h0 = bf16_trunc(x0), h1 = bf16_trunc(x1);
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
// D += A . B on 16x16x32 with 8 elements of the format a lane in each operand
template <int KVF>
__device__ inline floatx4 mfma16x16x32(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, uint32_t b0,
                                      uint32_t b1, uint32_t b2, uint32_t b3, floatx4 c) {
  if constexpr (KVF == kKvBf16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, uintx4{a0, a1, a2, a3}),
                                                   __builtin_bit_cast(bf16x8, uintx4{b0, b1, b2, b3}), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(halfx8, uintx4{a0, a1, a2, a3}),
                                                  __builtin_bit_cast(halfx8, uintx4{b0, b1, b2, b3}), c, 0, 0, 0);
}
// The q row in the B-operand layout (q[i]: d = 32 (i >> 1) + 8g + 4 (i & 1)
// .. +3; lanes li, li + 16, li + 32, li + 48 hold row li) as three terms;
// word 4t + m of term k holds d = 32t + 8g + 2m and 2m + 1, the elements of
// the K words they meet. Returns the factor of the row's raw scores:
// `scale` (bf16), or `scale` * 2^-sx (fp16, q scaled by 2^sx).
template <int KVF>
__device__ inline float split_q16(const floatx4 (&q)[8], uint32_t (&qw)[3][16], float scale) {
  int sx = 0;
  if constexpr (KVF == kKvF16) {
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) mx = fmaxf(mx, fabsf(q[i][c]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (mx > 0.f && mx <= 3.0e38f) {
      int e;
      (void)frexpf(mx, &e);                   // mx = f * 2^e, f in [0.5, 1)
      sx = 15 - e;
      sx = sx < -120 ? -120 : (sx > 120 ? 120 : sx);
    }
  }
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float x0 = q[2 * t + (m >> 1)][2 * (m & 1)], x1 = q[2 * t + (m >> 1)][2 * (m & 1) + 1];
      if constexpr (KVF == kKvF16) {
        x0 = ldexpf(x0, sx);
        x1 = ldexpf(x1, sx);
      }
#pragma unroll
      for (int k = 0; k < 3; ++k) qw[k][4 * t + m] = split_pair<KVF>(x0, x1);
    }
  return KVF == kKvF16 ? ldexpf(scale, -sx) : scale;
}
// Raw scores of a K piece of 16-bit words, S^T = K . Q^T: lane (li, g), reg r
// holds key 4g + r of the piece against row li. Element e of lane group g
// stands for d = 32t + 8g + e on both operands.
template <int KVF>
__device__ inline floatx4 scores16(const PieceT<KVF>& kp, const uint32_t (&qw)[3][16]) {
  floatx4 s0 = zero4(), s1 = zero4(), s2 = zero4();
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t k0 = kp.x[2 * t].x, k1 = kp.x[2 * t].y, k2 = kp.x[2 * t + 1].x, k3 = kp.x[2 * t + 1].y;
    s0 = mfma16x16x32<KVF>(k0, k1, k2, k3, qw[0][4 * t], qw[0][4 * t + 1], qw[0][4 * t + 2], qw[0][4 * t + 3], s0);
    s1 = mfma16x16x32<KVF>(k0, k1, k2, k3, qw[1][4 * t], qw[1][4 * t + 1], qw[1][4 * t + 2], qw[1][4 * t + 3], s1);
    s2 = mfma16x16x32<KVF>(k0, k1, k2, k3, qw[2][4 * t], qw[2][4 * t + 1], qw[2][4 * t + 2], qw[2][4 * t + 3], s2);
  }
  return s0 + (s1 + s2);
}
// O^T += V^T . P^T for a V piece of 16-bit words (row i of block db: d = 8i +
// db), p[r] the probability of key 4g + r for row li. Element e of lane
// group g stands for key 4g + (e & 3): p's high term for e < 4, its low
// term for e >= 4, V's word twice. `fresh`: the products start the sums.
template <int KVF>
__device__ inline void pv16(const PieceT<KVF>& vp, const float (&p)[4], floatx4 (&oacc)[8], bool fresh) {
  float x0 = p[0], x1 = p[1], x2 = p[2], x3 = p[3];
  const uint32_t h01 = split_pair<KVF>(x0, x1), h23 = split_pair<KVF>(x2, x3);
  const uint32_t l01 = split_pair<KVF>(x0, x1), l23 = split_pair<KVF>(x2, x3);
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    // V[key 4g + r][8li + db]: half (db & 1) of word (db >> 1) & 1 of group 2r + (db >> 2)
    uint32_t w[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) w[r] = (db & 2) ? vp.x[2 * r + (db >> 2)].y : vp.x[2 * r + (db >> 2)].x;
    const uint32_t v01 = (db & 1) ? (w[0] >> 16) | (w[1] & 0xffff0000u) : (w[0] & 0xffffu) | (w[1] << 16);
    const uint32_t v23 = (db & 1) ? (w[2] >> 16) | (w[3] & 0xffff0000u) : (w[2] & 0xffffu) | (w[3] << 16);
    oacc[db] = mfma16x16x32<KVF>(v01, v23, v01, v23, h01, h23, l01, l23, fresh ? zero4() : oacc[db]);
  }
}
__device__ inline int32_t unit_keys(const Unit& U, int32_t block_size) {
  const int64_t start = (int64_t)U.blk * block_size;
  int64_t end = start + block_size;
  end = end < U.lk ? end : (int64_t)U.lk;
  return end > start ? (int32_t)(end - start) : 0;
}

// Element offset of key t of unit U (head U.h) on page `page`, or -1 when t is
// past the block's keys or the page id is outside [0, num_pages).
__device__ inline int64_t key_offset(const FwdArgs& A, int64_t page_stride, const Unit& U, int t,
                                     int32_t page) {
  const int32_t pl = (int32_t)div_magic((uint32_t)t, A.ps_magic);
  return (t < unit_keys(U, A.block_size) && page >= 0 && page < A.num_pages)
             ? (int64_t)page * page_stride + ((int64_t)U.h * A.page_size + (t - pl * A.page_size)) * kD
             : -1;
}
// Block-table entry holding key t of unit U (t clamped into the block).
__device__ inline gint* page_id_ptr(const FwdArgs& A, const Unit& U, int t) {
  const int32_t tt = t < A.block_size ? t : 0;
  const int32_t pl = (int32_t)div_magic((uint32_t)tt, A.ps_magic);
  return (gint*)(A.block_tables + (int64_t)U.b * A.max_pages + (int64_t)U.blk * A.ppb + pl);
}

// NCH = pieces per block side (ceil(block_size / 16)); a unit takes 2 NCH steps.
template <int NCH, int KVF>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void k_fwd_small(IndexPtrs P, FwdArgs A) {
  using Piece = PieceT<KVF>;
  __shared__ WaveLds s_wave[kWaves];

  const DevHeader* hdr = P.hdr;
  if (hdr->status != SA_OK) return;
  const int32_t num_units = hdr->num_units_wave;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int li = lane & 15, g = lane >> 4;
  const int32_t NW = (int32_t)gridDim.x * kWaves;
  const int32_t u0 = (int32_t)blockIdx.x * kWaves + w;
  // The four waves of a workgroup take four neighbouring units at each step
  // of their loops (the split units of one slot read the same block), and a
  // workgroup barrier per unit keeps them in step, so that the second read
  // of a block finds it in cache. Every wave passes the same number of
  // barriers: that of the workgroup's first wave, which has the most units.
  const int32_t ub = u0 - w;
  const int32_t n_bar = ub < num_units ? (num_units - ub + NW - 1) / NW : 0;
  if (u0 >= num_units) {
    for (int32_t i = 0; i < n_bar; ++i) __builtin_amdgcn_s_barrier();
    return;
  }
  WaveLds& S = s_wave[w];

  const int32_t qhead = A.qhead;
  const int64_t page_stride = (int64_t)A.hkv * A.page_size * kD;
  const int32_t* units = reinterpret_cast<const int32_t*>(P.units_wave);
  const int32_t n_units = (num_units - u0 + NW - 1) / NW;
  gint* zi = (gint*)zero_line();

  auto rec_ptr = [&](int32_t j, bool ok) -> gint* {
    return ok ? (gint*)(units + 8 * (int64_t)(u0 + j * NW) + (lane & 7)) : zi;
  };
  auto qid_ptr = [&](const Unit& U, bool ok) -> gint* {
    const int r = lane < kRows ? lane : 0;
    return (ok && r < (U.e1 - U.e0) * qhead) ? (gint*)(P.edges + 2 * (int64_t)(U.e0 + r / qhead)) : zi;
  };
  auto stage_meta = [&](int ms, const Unit& U, int32_t page, int32_t qid) {
    const int64_t ko = key_offset(A, page_stride, U, lane, page);
    S.ko[ms][lane] = ko;
    const uint64_t vm = __ballot(ko >= 0);
    if (lane == 0) S.vm[ms] = vm;
    if (lane < kRows) S.qi[ms][lane] = qid;
  };
  // Issue piece pk (K pieces 0..NCH-1, then V pieces) of the unit in meta slot ms.
  auto load_piece = [&](auto pkc, int ms, bool live, Piece& pc) __attribute__((always_inline)) {
    constexpr int pk = decltype(pkc)::value;
    if constexpr (KVF == kKvF32) {
      if constexpr (pk < NCH) {
        const int64_t kb = S.ko[ms][kPiece * pk + li];
        gfloat* kp = (live && kb >= 0 ? (gfloat*)(A.k + kb) : zero_line()) + 8 * g;
#pragma unroll
        for (int i = 0; i < 8; ++i) pc.x[i] = *(gfloatx4*)(kp + 32 * (i >> 1) + 4 * (i & 1));
      } else {
        constexpr int c = pk - NCH;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t kb = S.ko[ms][kPiece * c + 4 * g + r];
          gfloat* vp = (live && kb >= 0 ? (gfloat*)(A.v + kb) : zero_line()) + 8 * li;
          pc.x[2 * r] = *(gfloatx4*)vp;
          pc.x[2 * r + 1] = *(gfloatx4*)(vp + 4);
        }
      }
    } else {
      // 16-bit storage: the same element offsets, half the bytes: one
      // 16-byte load per pair of register groups
      gu16* kbase = (gu16*)A.k;
      gu16* vbase = (gu16*)A.v;
      gu16* zero = (gu16*)zero_line();
      if constexpr (pk < NCH) {
        const int64_t kb = S.ko[ms][kPiece * pk + li];
        gu16* kp = (live && kb >= 0 ? kbase + kb : zero) + 8 * g;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uintx4 w = *(guint4*)(kp + 32 * t);
          pc.x[2 * t] = uintx2{w.x, w.y};
          pc.x[2 * t + 1] = uintx2{w.z, w.w};
        }
      } else {
        constexpr int c = pk - NCH;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t kb = S.ko[ms][kPiece * c + 4 * g + r];
          gu16* vp = (live && kb >= 0 ? vbase + kb : zero) + 8 * li;
          const uintx4 w = *(guint4*)vp;
          pc.x[2 * r] = uintx2{w.x, w.y};
          pc.x[2 * r + 1] = uintx2{w.z, w.w};
        }
      }
    }
  };
  // The B operand of the unit in record slot rs / meta slot ms: row li,
  // d = 32 (i >> 1) + 8g + 4 (i & 1) .. +3 in q[i]; zero past its rows.
  auto load_q = [&](int rs, int ms, bool live, floatx4 (&q)[8]) __attribute__((always_inline)) {
    const Unit U = as_unit(S.rec[rs]);
    const int32_t rows = live ? (U.e1 - U.e0) * qhead : 0;
    const int64_t qrow = (int64_t)S.qi[ms][li] * A.hq + (int64_t)U.h * qhead + li % qhead;
    gfloat* src = (li < rows ? (gfloat*)(A.q + qrow * kD) : zero_line()) + 8 * g;
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = *(gfloatx4*)(src + 32 * (i >> 1) + 4 * (i & 1));
  };

  // ---- prologue: records of units 0..2, metadata of units 0 and 1, q and the first piece of unit 0
  {
    int32_t rv[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) rv[j] = *rec_ptr(j, j < n_units);
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (lane < 8) S.rec[j][lane] = rv[j];
    int32_t pg[2], qv[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const Unit U = as_unit(S.rec[j]);
      pg[j] = *(j < n_units ? page_id_ptr(A, U, lane) : zi);
      qv[j] = *qid_ptr(U, j < n_units);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) stage_meta(j, as_unit(S.rec[j]), pg[j], qv[j]);
  }
  floatx4 qreg[8];
  load_q(0, 0, true, qreg);
  Piece bufA, bufB;
  load_piece(IC<0>{}, 0, true, bufA);

  for (int32_t j = 0; j < n_units; ++j) {
    __builtin_amdgcn_s_barrier();
    const int rs = j & (kRecRing - 1), ms = j % kMetaRing;
    const int rs1 = (j + 1) & (kRecRing - 1), ms1 = (j + 1) % kMetaRing;
    const int rs2 = (j + 2) & (kRecRing - 1), ms2 = (j + 2) % kMetaRing;
    const bool ok1 = j + 1 < n_units;

    const Unit U = as_unit(S.rec[rs]);
    const int32_t rows = (U.e1 - U.e0) * qhead;
    const bool row_ok = li < rows;
    const int64_t block_start = (int64_t)U.blk * A.block_size;
    const int32_t nkeys = unit_keys(U, A.block_size);
    const uint64_t vm = S.vm[ms];
    int64_t klim = A.causal ? (int64_t)S.qi[ms][li] + U.delta - block_start : (int64_t)nkeys - 1;
    klim = klim < (int64_t)nkeys - 1 ? klim : (int64_t)nkeys - 1;
    const int32_t kmax = (int32_t)(klim < -1 ? -1 : klim);   // last alive key of row li

    float sreg[NCH][4];
    floatx4 oacc[8];
    float m_row = -INFINITY, l_row = 0.f;
    int32_t pre_rec = 0, pre_page = 0, pre_qi = 0;
    uint32_t qw[KVF != kKvF32 ? 3 : 1][16];      // 16-bit pages: this unit's q as terms of the format
    float c2q = A.scale_log2;                    // the factor of the raw scores

    auto step = [&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      if constexpr (k < 2 * NCH) {
        Piece& cur = (k & 1) ? bufB : bufA;
        Piece& nxt = (k & 1) ? bufA : bufB;
        // ---- loads ahead: metadata (first step), the next piece, the next unit's q
        if constexpr (k == 0) {
          const Unit U2 = as_unit(S.rec[rs2]);
          pre_rec = *rec_ptr(j + 3, j + 3 < n_units);
          pre_page = *(j + 2 < n_units ? page_id_ptr(A, U2, lane) : zi);
          pre_qi = *qid_ptr(U2, j + 2 < n_units);
        }
        if constexpr (k + 1 < 2 * NCH) load_piece(IC<k + 1>{}, ms, true, nxt);
        else load_piece(IC<0>{}, ms1, ok1, nxt);
        if constexpr (k == NCH) load_q(rs1, ms1, ok1, qreg);
        // keep the loads above the math: the scheduler would otherwise sink
        // them below it to share registers with `cur`
        __builtin_amdgcn_sched_barrier(0);

        if constexpr (k < NCH) {
          // ---- scores of piece k: S^T = K . Q^T
          floatx4 s;                      // lane (li, g), reg r: key 16k + 4g + r, row li
          if constexpr (KVF != kKvF32) {
            if constexpr (k == 0) c2q = split_q16<KVF>(qreg, qw, A.scale_log2);
            s = scores16<KVF>(cur, qw);
          } else {
            floatx4 sa0 = zero4(), sa1 = zero4();
#pragma unroll
            for (int t = 0; t < 8; t += 2) {
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                sa0 = __builtin_amdgcn_mfma_f32_16x16x4f32(kv_elem(cur, t, c), qreg[t][c], sa0, 0, 0, 0);
                sa1 = __builtin_amdgcn_mfma_f32_16x16x4f32(kv_elem(cur, t + 1, c), qreg[t + 1][c], sa1,
                                                           0, 0, 0);
              }
            }
            s = sa0 + sa1;
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = kPiece * k + 4 * g + r;
            const bool alive = row_ok && ((vm >> key) & 1ull) && key <= kmax;
            sreg[k][r] = alive ? s[r] * c2q : -INFINITY;
          }
          if constexpr (k == NCH - 1) {
            // ---- softmax of row li over the whole block (base 2)
            float mx = -INFINITY;
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
              for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sreg[c][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            float ls = 0.f;
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float p = sreg[c][r] == -INFINITY ? 0.f : exp2f(sreg[c][r] - mx);
                sreg[c][r] = p;
                ls += p;
              }
            ls += __shfl_xor(ls, 16, 64);
            ls += __shfl_xor(ls, 32, 64);
            m_row = mx;
            l_row = ls;
          }
        } else {
          // ---- O^T += V^T . P^T for piece c (row i of block db: d = 8i + db)
          constexpr int c = k - NCH;
          if constexpr (KVF != kKvF32) {
            pv16<KVF>(cur, sreg[c], oacc, c == 0);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
#pragma unroll
              for (int db = 0; db < 8; ++db) {
                const floatx4 acc = (c == 0 && r == 0) ? zero4() : oacc[db];
                oacc[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(kv_elem(cur, 2 * r + (db >> 2), db & 3),
                                                                sreg[c][r], acc, 0, 0, 0);
              }
            }
          }
        }

        if constexpr (k == 1) {
          // ---- stage the metadata fetched at the first step
          if (lane < 8) S.rec[(j + 3) & (kRecRing - 1)][lane] = pre_rec;
          stage_meta(ms2, as_unit(S.rec[rs2]), pre_page, pre_qi);
        }
        if constexpr (k == 2 * NCH - 1) {
          // ---- the unit's partials: lane (li, g) holds row li,
          // d = 32g + 8v + db in oacc[db][v]. The tile goes through this
          // wave's LDS so that every store instruction writes 64 lanes x 16 B
          // of contiguous rows (the unit's rows are consecutive in the
          // partial arrays); stored straight from the accumulators, each
          // instruction would write 16-B pieces 32 B apart.
          if (row_ok) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              *reinterpret_cast<floatx4*>(&S.ostage[li][32 * g + 8 * v]) =
                  floatx4{oacc[0][v], oacc[1][v], oacc[2][v], oacc[3][v]};
              *reinterpret_cast<floatx4*>(&S.ostage[li][32 * g + 8 * v + 4]) =
                  floatx4{oacc[4][v], oacc[5][v], oacc[6][v], oacc[7][v]};
            }
            if (g == 0) {
              const int64_t row = (int64_t)U.e0 * qhead + li;
              A.m[row] = m_row == -INFINITY ? -INFINITY : m_row * kLn2;
              A.l[row] = l_row;
            }
          }
          // non-temporal: the partials are read back only by the combine,
          // so they need not take L2 lines from the blocks that the
          // neighbouring units read again (ragged 364 -> 355 us)
          float* dst0 = A.o + (int64_t)U.e0 * qhead * kD;
          for (int i = lane; i < rows * (kD / 4); i += 64) {
            const int r = i >> 5, c = i & 31;
            __builtin_nontemporal_store(*reinterpret_cast<const floatx4*>(&S.ostage[r][4 * c]),
                                        reinterpret_cast<floatx4*>(dst0 + r * kD + 4 * c));
          }
        }
      }
    };
    step(IC<0>{}); step(IC<1>{}); step(IC<2>{}); step(IC<3>{});
    step(IC<4>{}); step(IC<5>{}); step(IC<6>{}); step(IC<7>{});
  }
  for (int32_t i = n_units; i < n_bar; ++i) __builtin_amdgcn_s_barrier();
}

template <int NCH, int KVF>
hipError_t launch_nch(const sa_index* idx, const FwdArgs& a, hipStream_t s, unsigned max_units) {
  static thread_local int per_cu = 0;
  if (per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_fwd_small<NCH, KVF>, kThreads, 0) != hipSuccess || n < 1)
      n = 1;
    per_cu = n;
  }
  // one wave per unit stream
  unsigned grid = (unsigned)per_cu * cu_count();
  const unsigned need = (max_units + kWaves - 1) / kWaves;
  if (grid > need) grid = need;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((k_fwd_small<NCH, KVF>), dim3(grid), dim3(kThreads), 0, s, index_ptrs(idx), a);
  return hipGetLastError();
}


// ------------------------------------------------------------ fused forward + combine
// One workgroup per (query q, KV head h) computes the final rows O[q, h*qhead
// .. h*qhead + qhead) and their lse in one launch, with no partials in
// memory: the forward's block partials and their log-sum-exp combine, for
// batches where each block serves one query (decode). Query q's kept ranks
// (inv[h, q, r] >= 0, block selected[q, h, r]) are dealt to the eight waves;
// each wave streams its blocks through the same 16-key pieces as k_fwd_small
// (the next piece in flight, the next block's key offsets fetched a block
// ahead) and keeps a running (M, L, O) per row, rescaled when a block raises
// the maximum: the merge the combine applies. The waves' (M, L, O) meet in
// LDS and one merge writes the output. Every kept block is read once, as in
// the KV-outer path when each slot holds one edge.
constexpr int kFusedWaves = 8;
constexpr int kFusedRanksPerWave = 64;           // topk <= 8 * 64

struct FusedWaveLds {
  int32_t blk[kFusedRanksPerWave];               // block ids of the wave's kept ranks
  int64_t ko[2][kMaxKeys];                       // key offsets of the current / next block, or -1
  uint64_t vm[2];                                // bit t: key t has a row
};

template <int NCH, int KVF>
__global__ __launch_bounds__(kFusedWaves * 64) __attribute__((amdgpu_waves_per_eu(2))) void k_fwd_fused(
    IndexPtrs P, FwdArgs A, const int32_t* __restrict__ selected, float* __restrict__ out,
    float* __restrict__ lse, int32_t tq, int32_t topk) {
  using Piece = PieceT<KVF>;
  __shared__ FusedWaveLds s_wave[kFusedWaves];
  __shared__ float s_m[kFusedWaves][kRows], s_l[kFusedWaves][kRows];
  __shared__ __align__(16) float s_o[kFusedWaves][kRows][kD];

  const int32_t qhead = A.qhead;
  // head-major workgroups: neighbours read the same head of neighbouring sequences
  const int32_t h = (int32_t)(blockIdx.x / (uint32_t)tq);
  const int32_t q = (int32_t)(blockIdx.x - (uint32_t)h * (uint32_t)tq);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int li = lane & 15, g = lane >> 4;
  const int64_t orow0 = (int64_t)q * A.hq + (int64_t)h * qhead;    // first output row

  if (P.hdr->status != SA_OK) {
    // a failed build: the output gets a defined value, as sa_combine gives it
    for (int x = threadIdx.x; x < qhead * kD; x += kFusedWaves * 64) out[orow0 * kD + x] = NAN;
    if (lse != nullptr && (int)threadIdx.x < qhead) lse[orow0 + threadIdx.x] = NAN;
    return;
  }
  FusedWaveLds& S = s_wave[w];
  const int64_t page_stride = (int64_t)A.hkv * A.page_size * kD;
  const int64_t head_off = (int64_t)h * A.page_size * kD;

  // ---- the query's sequence: b = q when cu[q] <= q < cu[q + 1] (a decode
  // batch), else the search of batch_of; its kv length and causal offset
  int32_t b;
  {
    const int32_t qq = q < A.batch ? q : A.batch - 1;
    const int64_t c0 = A.cu[qq], c1 = A.cu[qq + 1];
    b = (c0 <= q && q < c1) ? qq : batch_of_dev(A.cu, A.batch, q);
  }
  const int64_t cb0 = A.cu[b];
  const int64_t qo_len = A.cu[b + 1] - cb0;
  const int64_t lk = kv_len_dev(A.used, b, A.msb, A.block_size);
  const int64_t delta = (lk >= qo_len ? lk - qo_len : 0) - cb0;
  const int64_t bt_row = (int64_t)b * A.max_pages;

  // ---- this wave's kept ranks r = w + 8 i (lane i): their block ids, in rank order
  int32_t n_blk;
  {
    const int32_t r = w + kFusedWaves * lane;
    const bool in = r < topk;
    const int64_t at = ((int64_t)q * A.hkv + h) * topk + (in ? r : 0);
    const int32_t e = P.inv[((int64_t)h * tq + q) * topk + (in ? r : 0)];
    const int32_t v = selected[at];
    const bool kept = in && e >= 0;
    const uint64_t bal = __ballot(kept);
    const int32_t pos = (int32_t)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    if (kept) S.blk[pos] = v;
    n_blk = (int32_t)__popcll(bal);
  }
  // key offsets of the wave's k-th block into slot ks (lane = key)
  auto block_meta = [&](int32_t k, int ks) {
    int64_t ko = -1;
    if (k < n_blk) {
      const int32_t v = S.blk[k];
      const int64_t start = (int64_t)v * A.block_size;
      int64_t end = start + A.block_size;
      end = end < lk ? end : lk;
      if (start + lane < end) {
        const int32_t pl = (int32_t)div_magic((uint32_t)lane, A.ps_magic);
        const int32_t page = A.block_tables[bt_row + (int64_t)v * A.ppb + pl];
        if (page >= 0 && page < A.num_pages)
          ko = (int64_t)page * page_stride + head_off + (int64_t)(lane - pl * A.page_size) * kD;
      }
    }
    S.ko[ks][lane] = ko;
    const uint64_t vm = __ballot(ko >= 0);
    if (lane == 0) S.vm[ks] = vm;
  };
  auto load_piece = [&](auto pkc, int ks, bool live, Piece& pc) __attribute__((always_inline)) {
    constexpr int pk = decltype(pkc)::value;
    if constexpr (KVF == kKvF32) {
      if constexpr (pk < NCH) {
        const int64_t kb = S.ko[ks][kPiece * pk + li];
        gfloat* kp = (live && kb >= 0 ? (gfloat*)(A.k + kb) : zero_line()) + 8 * g;
#pragma unroll
        for (int i = 0; i < 8; ++i) pc.x[i] = *(gfloatx4*)(kp + 32 * (i >> 1) + 4 * (i & 1));
      } else {
        constexpr int c = pk - NCH;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t kb = S.ko[ks][kPiece * c + 4 * g + r];
          gfloat* vp = (live && kb >= 0 ? (gfloat*)(A.v + kb) : zero_line()) + 8 * li;
          pc.x[2 * r] = *(gfloatx4*)vp;
          pc.x[2 * r + 1] = *(gfloatx4*)(vp + 4);
        }
      }
    } else {
      gu16* kbase = (gu16*)A.k;
      gu16* vbase = (gu16*)A.v;
      gu16* zero = (gu16*)zero_line();
      if constexpr (pk < NCH) {
        const int64_t kb = S.ko[ks][kPiece * pk + li];
        gu16* kp = (live && kb >= 0 ? kbase + kb : zero) + 8 * g;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uintx4 x = *(guint4*)(kp + 32 * t);
          pc.x[2 * t] = uintx2{x.x, x.y};
          pc.x[2 * t + 1] = uintx2{x.z, x.w};
        }
      } else {
        constexpr int c = pk - NCH;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t kb = S.ko[ks][kPiece * c + 4 * g + r];
          gu16* vp = (live && kb >= 0 ? vbase + kb : zero) + 8 * li;
          const uintx4 x = *(guint4*)vp;
          pc.x[2 * r] = uintx2{x.x, x.y};
          pc.x[2 * r + 1] = uintx2{x.z, x.w};
        }
      }
    }
  };

  // the query's rows as the B operand: row li (lane group g takes
  // d = 32 (i >> 1) + 8g + 4 (i & 1) .. +3 in qreg[i]); zero past qhead
  floatx4 qreg[8];
  {
    gfloat* src = (li < qhead ? (gfloat*)(A.q + (orow0 + li) * kD) : zero_line()) + 8 * g;
#pragma unroll
    for (int i = 0; i < 8; ++i) qreg[i] = *(gfloatx4*)(src + 32 * (i >> 1) + 4 * (i & 1));
  }
  // bf16 pages: the q row as three bf16 terms; word 4t + m of term k holds
  // d = 32t + 8g + 2m and 2m + 1, the elements of the K words it meets
  uint32_t qw[KVF != kKvF32 ? 3 : 1][16];
  float c2q = A.scale_log2;          // the factor of the raw scores
  if constexpr (KVF != kKvF32) c2q = split_q16<KVF>(qreg, qw, A.scale_log2);
  block_meta(0, 0);
  Piece bufA, bufB;
  load_piece(IC<0>{}, 0, n_blk > 0, bufA);

  // running merge of this wave's blocks for row li (base-2 units)
  float M = -INFINITY, L = 0.f;
  floatx4 oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = zero4();
  const bool row_ok = li < qhead;

  for (int32_t k = 0; k < n_blk; ++k) {
    const int ks = k & 1, ks1 = ks ^ 1;
    const bool more = k + 1 < n_blk;
    const int32_t v = S.blk[k];
    const int64_t block_start = (int64_t)v * A.block_size;
    int64_t block_end = block_start + A.block_size;
    block_end = block_end < lk ? block_end : lk;
    const int32_t nkeys = block_end > block_start ? (int32_t)(block_end - block_start) : 0;
    const uint64_t vm = S.vm[ks];
    int64_t klim = A.causal ? (int64_t)q + delta - block_start : (int64_t)nkeys - 1;
    klim = klim < (int64_t)nkeys - 1 ? klim : (int64_t)nkeys - 1;
    const int32_t kmax = (int32_t)(klim < -1 ? -1 : klim);
    float sreg[NCH][4];
    float resc = 1.f;

    auto step = [&](auto kc) __attribute__((always_inline)) {
      constexpr int j = decltype(kc)::value;
      if constexpr (j < 2 * NCH) {
        Piece& cur = (j & 1) ? bufB : bufA;
        Piece& nxt = (j & 1) ? bufA : bufB;
        if constexpr (j == 0) block_meta(k + 1, ks1);     // the next block's key offsets
        if constexpr (j + 1 < 2 * NCH) load_piece(IC<j + 1>{}, ks, true, nxt);
        else load_piece(IC<0>{}, ks1, more, nxt);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (j < NCH) {
          floatx4 s;                      // lane (li, g), reg r: key 16j + 4g + r, row li
          if constexpr (KVF != kKvF32) {
            s = scores16<KVF>(cur, qw);
          } else {
            floatx4 sa0 = zero4(), sa1 = zero4();
#pragma unroll
            for (int t = 0; t < 8; t += 2) {
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                sa0 = __builtin_amdgcn_mfma_f32_16x16x4f32(kv_elem(cur, t, c), qreg[t][c], sa0, 0, 0, 0);
                sa1 = __builtin_amdgcn_mfma_f32_16x16x4f32(kv_elem(cur, t + 1, c), qreg[t + 1][c], sa1,
                                                           0, 0, 0);
              }
            }
            s = sa0 + sa1;
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = kPiece * j + 4 * g + r;
            const bool alive = row_ok && ((vm >> key) & 1ull) && key <= kmax;
            sreg[j][r] = alive ? s[r] * c2q : -INFINITY;
          }
          if constexpr (j == NCH - 1) {
            // ---- the block's maximum joins the running one; rescale O and L
            float mx = -INFINITY;
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
              for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sreg[c][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float m_new = fmaxf(M, mx);
            resc = (M == -INFINITY) ? 0.f : exp2f(M - m_new);
            float ls = 0.f;
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float p = sreg[c][r] == -INFINITY ? 0.f : exp2f(sreg[c][r] - m_new);
                sreg[c][r] = p;
                ls += p;
              }
            ls += __shfl_xor(ls, 16, 64);
            ls += __shfl_xor(ls, 32, 64);
            if (m_new != -INFINITY) {
              L = L * resc + ls;
              M = m_new;
            }
#pragma unroll
            for (int db = 0; db < 8; ++db) oacc[db] *= resc == 0.f ? 0.f : resc;
          }
        } else {
          constexpr int c = j - NCH;
          if constexpr (KVF != kKvF32) {
            pv16<KVF>(cur, sreg[c], oacc, false);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
#pragma unroll
              for (int db = 0; db < 8; ++db)
                oacc[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(kv_elem(cur, 2 * r + (db >> 2), db & 3),
                                                                sreg[c][r], oacc[db], 0, 0, 0);
            }
          }
        }
      }
    };
    step(IC<0>{}); step(IC<1>{}); step(IC<2>{}); step(IC<3>{});
    step(IC<4>{}); step(IC<5>{}); step(IC<6>{}); step(IC<7>{});
  }

  // ---- the waves' (M, L, O) into LDS: lane (li, g) holds row li,
  // d = 32g + 8v + db in oacc[db][v]
  if (row_ok) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      *reinterpret_cast<floatx4*>(&s_o[w][li][32 * g + 8 * v]) =
          floatx4{oacc[0][v], oacc[1][v], oacc[2][v], oacc[3][v]};
      *reinterpret_cast<floatx4*>(&s_o[w][li][32 * g + 8 * v + 4]) =
          floatx4{oacc[4][v], oacc[5][v], oacc[6][v], oacc[7][v]};
    }
    if (g == 0) {
      s_m[w][li] = M;
      s_l[w][li] = L;
    }
  }
  __syncthreads();
  // ---- final merge: item x covers row x / 32 and float4 column x % 32
  for (int x = threadIdx.x; x < qhead * (kD / 4); x += kFusedWaves * 64) {
    const int row = x >> 5, c4 = x & 31;
    float mt = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kFusedWaves; ++ww) mt = fmaxf(mt, s_m[ww][row]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float lt = 0.f;
    if (mt != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < kFusedWaves; ++ww) {
        const float mw = s_m[ww][row];
        const float f = mw == -INFINITY ? 0.f : exp2f(mw - mt);
        const float4 o4 = *reinterpret_cast<const float4*>(&s_o[ww][row][4 * c4]);
        acc = make_float4(fmaf(o4.x, f, acc.x), fmaf(o4.y, f, acc.y), fmaf(o4.z, f, acc.z),
                          fmaf(o4.w, f, acc.w));
        lt = fmaf(s_l[ww][row], f, lt);
      }
      const float il = 1.f / lt;
      acc = make_float4(acc.x * il, acc.y * il, acc.z * il, acc.w * il);
    }
    *reinterpret_cast<float4*>(out + (orow0 + row) * kD + 4 * c4) = acc;
    if (lse != nullptr && c4 == 0)
      lse[orow0 + row] = mt == -INFINITY ? -INFINITY : mt * kLn2 + logf(lt);
  }
}

template <int NCH, int KVF>
hipError_t launch_fused_nch(const sa_index* idx, const FwdArgs& a, const int32_t* selected,
                            float* out, float* lse, hipStream_t s) {
  const int64_t grid = idx->tq * (int64_t)idx->hkv;
  hipLaunchKernelGGL((k_fwd_fused<NCH, KVF>), dim3((unsigned)grid), dim3(kFusedWaves * 64), 0, s,
                     index_ptrs(idx), a, selected, out, lse, (int32_t)idx->tq, idx->topk);
  return hipGetLastError();
}

}  // namespace

bool small_kernel_fits(int head_dim, int block_size, int page_size, int qhead) {
  (void)page_size;
  return head_dim == kD && block_size <= kMaxKeys && qhead <= kRows;
}

int small_kernel_rows() { return kRows; }

bool fused_kernel_fits(int head_dim, int block_size, int page_size, int qhead, int topk) {
  return small_kernel_fits(head_dim, block_size, page_size, qhead) &&
         topk <= kFusedWaves * kFusedRanksPerWave;
}

hipError_t launch_forward_fused(const sa_index* idx, const FwdArgs& a, const int32_t* selected,
                                float* out, float* lse, hipStream_t s) {
  const int nch = (a.block_size + kPiece - 1) / kPiece;
  switch (a.kv_format) {
    case kKvBf16:
      switch (nch) {
        case 1: return launch_fused_nch<1, kKvBf16>(idx, a, selected, out, lse, s);
        case 2: return launch_fused_nch<2, kKvBf16>(idx, a, selected, out, lse, s);
        case 3: return launch_fused_nch<3, kKvBf16>(idx, a, selected, out, lse, s);
        default: return launch_fused_nch<4, kKvBf16>(idx, a, selected, out, lse, s);
      }
    case kKvF16:
      switch (nch) {
        case 1: return launch_fused_nch<1, kKvF16>(idx, a, selected, out, lse, s);
        case 2: return launch_fused_nch<2, kKvF16>(idx, a, selected, out, lse, s);
        case 3: return launch_fused_nch<3, kKvF16>(idx, a, selected, out, lse, s);
        default: return launch_fused_nch<4, kKvF16>(idx, a, selected, out, lse, s);
      }
    default:
      switch (nch) {
        case 1: return launch_fused_nch<1, kKvF32>(idx, a, selected, out, lse, s);
        case 2: return launch_fused_nch<2, kKvF32>(idx, a, selected, out, lse, s);
        case 3: return launch_fused_nch<3, kKvF32>(idx, a, selected, out, lse, s);
        default: return launch_fused_nch<4, kKvF32>(idx, a, selected, out, lse, s);
      }
  }
}

hipError_t launch_forward_small(const sa_index* idx, const FwdArgs& a, hipStream_t s,
                                unsigned max_units) {
  const int nch = (a.block_size + kPiece - 1) / kPiece;
  switch (a.kv_format) {
    case kKvBf16:
      switch (nch) {
        case 1: return launch_nch<1, kKvBf16>(idx, a, s, max_units);
        case 2: return launch_nch<2, kKvBf16>(idx, a, s, max_units);
        case 3: return launch_nch<3, kKvBf16>(idx, a, s, max_units);
        default: return launch_nch<4, kKvBf16>(idx, a, s, max_units);
      }
    case kKvF16:
      switch (nch) {
        case 1: return launch_nch<1, kKvF16>(idx, a, s, max_units);
        case 2: return launch_nch<2, kKvF16>(idx, a, s, max_units);
        case 3: return launch_nch<3, kKvF16>(idx, a, s, max_units);
        default: return launch_nch<4, kKvF16>(idx, a, s, max_units);
      }
    default:
      switch (nch) {
        case 1: return launch_nch<1, kKvF32>(idx, a, s, max_units);
        case 2: return launch_nch<2, kKvF32>(idx, a, s, max_units);
        case 3: return launch_nch<3, kKvF32>(idx, a, s, max_units);
        default: return launch_nch<4, kKvF32>(idx, a, s, max_units);
      }
  }
}

}  // namespace sa
