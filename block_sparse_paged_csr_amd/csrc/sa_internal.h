// Internal definitions shared by the library's translation units (not part
// of the public ABI): the device-side index header, kernel argument packs,
// tuning constants and launcher prototypes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sa.h"

namespace sa {

// ---------------------------------------------------------------- tuning
// Most rows (edges * qhead) in one work unit. A slot with more edges is split
// into near-equal units so that one hot block does not serialise the grid.
constexpr int kCapRows = 2048;
constexpr int kCapUnitEdges = 512;   // most edges in one MFMA unit
// Smallest unit (in rows) that goes to the MFMA kernel. Smaller ones use the
// wavefront-reduction kernel.
constexpr int kMfmaMinRows = 32;
// Head dims the MFMA kernel is built for; others always take the wave path.
constexpr int kMfmaHeadDim = 128;
constexpr int kMfmaMaxBlock = 128;

// ---------------------------------------------------------------- errors
// Device errors are ranked. The build keeps the smallest (rank, position)
// key with one atomicMin, so the report does not depend on thread timing.
enum ErrRank : uint64_t {
  kRankCuContent = 1,   // cu[0] != 0 or decreasing
  kRankCuTotal = 2,     // cu[batch] != tq
  kRankSelected = 3,    // id outside [-1, msb), position = flat index
  kRankPage = 4,        // page id >= num_pages, position = block-table index
};
__host__ __device__ inline unsigned long long err_key(uint64_t rank, uint64_t pos) {
  return (rank << 56) | (pos & ((1ull << 56) - 1));
}

enum WhatCode : int32_t {
  kWhatNone = 0,
  kWhatCuTotal = 1,
  kWhatPageId = 2,
};

// One work unit: a sub-range [e0, e1) of compact slot j of head h (the
// WorkSplit fields of forward.rs), plus what the forward needs without
// further lookups: the slot's sequence b and block blk, the resolved KV length
// lk_b, and delta such that the causal limit of query q is q + delta.
struct alignas(16) Unit {
  int32_t h, j, e0, e1;
  int32_t b, blk, lk, delta;
};
static_assert(sizeof(Unit) == 32, "unit record is 32 bytes");

// Device-resident header at the start of the index buffer (256 bytes).
struct alignas(256) DevHeader {
  unsigned long long err_key;   // ~0ull = no error
  int32_t status;               // sa_status, filled by the last build kernel
  int32_t what_code;            // WhatCode
  int64_t err_expected;
  int64_t err_got;
  int64_t total_edges;
  int32_t num_units_wave;
  int32_t num_units_mfma;
  int64_t num_slots;
  int32_t geom[8];              // planned geometry fingerprint
};
static_assert(sizeof(DevHeader) == 256, "header is one 256-byte block");

// Scratch region inside the index buffer (after the public arrays).
struct ScratchLayout {
  size_t cnt;        // int32 [hkv*nbs]   counts, then scatter cursors
  size_t slot_uw;    // int32 [hkv*nbs]   wave-unit offset of compact slot (head-local)
  size_t slot_um;    // int32 [hkv*nbs]   mfma-unit offset of compact slot (head-local)
  size_t head_e;     // int32 [hkv]       E_h
  size_t head_uw;    // int32 [hkv]
  size_t head_um;    // int32 [hkv]
  size_t keys;       // int32 [max_edges] scattered (q*topk + r), unordered per slot
  size_t qinfo;      // int2  [tq]        (sequence b, resolved kv length lk_b) per query
  size_t agg;        // HeadAgg [hkv]     per-head totals published by the fused build
  size_t chunk_agg;  // ChunkAgg [hkv * scan_chunks(nbs)]  per-chunk sums of the slot scan
  size_t units_sorted;  // Unit [max_units]  the MFMA units, largest first (unit sort)
  size_t sort_hist;  // int32 [kSortHistInts]: the unit sort's counts, counter and group offsets
  size_t end;
};

// Totals of one head, published by the fused build's workgroup for that head
// (flag == that build's epoch once the fields are written).
struct alignas(64) HeadAgg {
  int64_t e;                  // edges
  int32_t ns, uw, um, pad;    // nonempty slots, wavefront units, MFMA units
  unsigned long long err;     // smallest error key seen by the head (~0ull: none)
  uint64_t flag;
};

// The MFMA unit sort: a counting sort over (group, size) buckets in up to
// kSortGrid workgroups. A unit's group is (b * hkv + h) % kSortGroups, one
// group for each XCD; its size bucket counts 32-row tiles, largest first
// (units hold at most 2048 rows = 64 tiles). The sort array holds the
// per-(bucket, workgroup) counts, then offsets [kSortBuckets * kSortGrid];
// the workgroups' counter [1]; and what the forward reads [kSortGroups +
// 2]: whether the list is in groups, then the groups' first units
// (kSortGroups + 1 offsets).
constexpr int kSortGrid = 64;
constexpr int kSortSizes = 64;
constexpr int kSortGroups = 8;
constexpr int kSortBuckets = kSortSizes * kSortGroups;
constexpr int kSortHistCounter = kSortBuckets * kSortGrid;
constexpr int kSortHistInfo = kSortHistCounter + 1;
constexpr int kSortHistInts = kSortHistInfo + kSortGroups + 2;

// Slots scanned by one workgroup of the multi-kernel build.
constexpr int kScanChunkSlots = 2048;
// Chunks of one head's slots (at least one, which writes the head's totals).
__host__ __device__ inline int64_t scan_chunks(int64_t nbs) {
  return nbs > kScanChunkSlots ? (nbs + kScanChunkSlots - 1) / kScanChunkSlots : 1;
}

// Sums over one chunk of a head's slots (edges, nonempty slots, wavefront
// units, MFMA units), published for the chunks after it: `agg` with flag ==
// that build's epoch, then also `incl` (the sums over this chunk and all
// before it) with flag == epoch + 1.
struct alignas(64) ChunkAgg {
  int4 agg;
  int4 incl;
  uint64_t flag;
};

// Plain pointers into one index buffer.
struct IndexPtrs {
  DevHeader* hdr;
  int32_t* sel_slots;
  int32_t* sel_offsets;
  int32_t* num_sel;
  int64_t* edge_head_base;
  int32_t* edges;
  int32_t* inv;
  Unit* units_wave;
  Unit* units_mfma;
  int32_t* cnt;
  int32_t* slot_uw;
  int32_t* slot_um;
  int32_t* head_e;
  int32_t* head_uw;
  int32_t* head_um;
  int32_t* keys;
  int2* qinfo;
  HeadAgg* agg;
  ChunkAgg* chunk_agg;
  Unit* units_sorted;
  int32_t* sort_hist;
};

struct BuildArgs {
  const int32_t* selected;
  const int32_t* block_tables;
  const int64_t* cu;
  const int32_t* used;       // may be null
  int64_t tq;
  int64_t nbs;
  int64_t num_pages;
  int32_t hkv, topk, batch, max_pages, block_size, page_size, ppb, msb;
  int32_t qhead, cap_edges, wave_cap_edges, mfma_min_rows;
  uint64_t epoch;            // distinct per build call, odd; tags HeadAgg / ChunkAgg flags
  uint64_t cap_magic;        // make_div_magic(cap_edges)
  uint64_t wave_cap_magic;   // make_div_magic(wave_cap_edges)
  int32_t rank_bitmap_words; // words of the rank kernel's key bitmap (tq*topk bits, capped)
};

struct FwdArgs {
  const float* q;
  const float* k;
  const float* v;
  const int32_t* block_tables;
  const int64_t* cu;
  const int32_t* used;       // may be null
  float* o;
  float* m;
  float* l;
  int64_t nbs;
  int64_t num_pages;
  int32_t hq, hkv, qhead, head_dim, block_size, page_size, ppb, msb, max_pages, batch;
  int32_t causal;
  float scale_log2;          // softmax_scale * log2(e)
  uint64_t ps_magic;         // ceil(2^40 / page_size): n / page_size == (n * ps_magic) >> 40
                             // for n * page_size < 2^40
  int32_t kv_format;         // SA_KV_F32, SA_KV_BF16 or SA_KV_F16 (k, v then point at 16-bit words)
};

struct CombineArgs {
  const float* o;
  const float* m;
  const float* l;
  float* out;
  float* lse;
  int64_t tq;
  int32_t hq, hkv, qhead, head_dim, topk;
};

IndexPtrs index_ptrs(const sa_index* idx);
ScratchLayout scratch_layout(const sa_index* idx);

// Whether the MFMA forward kernel is part of the library.
bool mfma_enabled();
// The chunked MFMA kernel: head_dim 64, 128 or 256 and blocks the fixed
// kernels do not take (head_dim 128 with blocks of up to 128 keys); rows of
// one tile a wave (the unit cap for blocks of more than one chunk) and keys
// a chunk.
bool mfma_general_fits(int head_dim, int block_size);
int mfma_general_tile_rows(int head_dim);
int mfma_general_chunk_keys(int head_dim, int block_size);
// Compute units of the current device (cached per host thread).
unsigned cu_count();

// Launchers (enqueue only; return hipSuccess or the launch error).
hipError_t launch_build(const sa_index* idx, const BuildArgs& a, hipStream_t s);
hipError_t launch_forward(const sa_index* idx, const FwdArgs& a, hipStream_t s);
// True when one workgroup per head can build the index in LDS (k_index_fused).
bool fused_build_fits(int64_t tq, int32_t topk, int64_t nbs, int32_t batch, int32_t hkv);
hipError_t launch_combine(const sa_index* idx, const CombineArgs& a, hipStream_t s);
hipError_t launch_forward_wave(const sa_index* idx, const FwdArgs& a, hipStream_t s,
                               unsigned max_grid);
hipError_t launch_forward_mfma(const sa_index* idx, const FwdArgs& a, hipStream_t s,
                               unsigned grid);
hipError_t launch_forward_small(const sa_index* idx, const FwdArgs& a, hipStream_t s,
                                unsigned max_grid);
// The small-unit kernel: head_dim 128, blocks of <= 64 keys, qhead <= 16;
// its units hold at most small_kernel_rows() rows.
bool small_kernel_fits(int head_dim, int block_size, int page_size, int qhead);
int small_kernel_rows();
// The fused forward + combine (one workgroup per (query, KV head)): the
// one-wave kernel's geometry and at most 512 ranks a row.
bool fused_kernel_fits(int head_dim, int block_size, int page_size, int qhead, int topk);
hipError_t launch_forward_fused(const sa_index* idx, const FwdArgs& a, const int32_t* selected,
                                float* out, float* lse, hipStream_t s);

// Exact n / d for n * d < 2^40 with magic = ceil(2^40 / d).
__host__ __device__ inline uint32_t div_magic(uint32_t n, uint64_t magic) {
  return (uint32_t)(((uint64_t)n * magic) >> 40);
}
inline uint64_t make_div_magic(uint32_t d) { return ((1ull << 40) + d - 1) / d; }

// ---------------------------------------------------------------- device helpers
// Four consecutive K/V elements at element offset `off` as fp32: a float4 for
// fp32 pages; for 16-bit pages (KVF = SA_KV_BF16 / SA_KV_F16, `base` then
// points at uint16 words) 8 bytes, each word converted exactly.
template <int KVF>
__device__ inline float kv16_to_f32(uint32_t w) {
  if constexpr (KVF == SA_KV_BF16) return __uint_as_float(w << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)w);
}
template <int KVF>
__device__ inline float4 load_kv4(const float* base, int64_t off) {
  if constexpr (KVF == SA_KV_F32) {
    return *reinterpret_cast<const float4*>(base + off);
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + off);
    return make_float4(kv16_to_f32<KVF>(w.x & 0xffffu), kv16_to_f32<KVF>(w.x >> 16),
                       kv16_to_f32<KVF>(w.y & 0xffffu), kv16_to_f32<KVF>(w.y >> 16));
  }
}

// Last b in [0, batch) with cu[b] <= q (types.rs CuSeqlensQ::batch_of).
__device__ inline int32_t batch_of_dev(const int64_t* __restrict__ cu, int32_t batch, int64_t q) {
  int32_t lo = 0, hi = batch + 1;      // first index with cu[i] > q lies in [lo, hi]
  while (lo < hi) {
    int32_t mid = (lo + hi) >> 1;
    if (cu[mid] <= q) lo = mid + 1; else hi = mid;
  }
  int32_t b = lo - 1;
  b = b < 0 ? 0 : b;
  return b >= batch ? batch - 1 : b;
}

__device__ inline int64_t kv_len_dev(const int32_t* __restrict__ used, int32_t b, int32_t msb,
                                     int32_t block_size) {
  if (used == nullptr) return (int64_t)msb * block_size;
  int32_t u = used[b];
  return u > 0 ? (int64_t)u : 0;
}

}  // namespace sa
