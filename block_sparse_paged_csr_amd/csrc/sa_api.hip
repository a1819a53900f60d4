// Host side of the C ABI declared in include/sa.h: index planning, argument
// checks in the order of the pages' kvouter_forward (alice-llm 2.0.0
// forward.rs) and of the builder's field docs (types.rs), dispatch of the
// kernels on the caller's stream, and the device-status readback.
#include <atomic>
#include <chrono>
#include <climits>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "sa_internal.h"

namespace {

thread_local sa_error_detail g_last = {SA_OK, "", 0, 0};

// Build epochs: distinct per build call in this process, started at a value
// mixed from the clock and an address so that flags left in a reused buffer
// by another process do not match.
uint64_t next_epoch() {
  static std::atomic<uint64_t> counter{[] {
    uint64_t x = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
    x ^= (uint64_t)(uintptr_t)&g_last * 0x9E3779B97F4A7C15ull;
    x ^= x >> 31;
    x *= 0xBF58476D1CE4E5B9ull;
    x ^= x >> 29;
    return x | 1ull;
  }()};
  uint64_t e = counter.fetch_add(2, std::memory_order_relaxed);
  return e == 0 ? 1 : e;
}

sa_status fail(sa_status st, const char* what = "", int64_t expected = 0, int64_t got = 0) {
  g_last.status = st;
  std::snprintf(g_last.what, sizeof(g_last.what), "%s", what ? what : "");
  g_last.expected = expected;
  g_last.got = got;
  return st;
}

sa_status ok() {
  g_last.status = SA_OK;
  g_last.what[0] = '\0';
  g_last.expected = 0;
  g_last.got = 0;
  return SA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
  return true;
}

sa_status runtime_error(hipError_t e, const char* where) {
  return fail(SA_ERR_GPU_RUNTIME, where, (int64_t)e, 0);
}

// The pages' forward checks on scalars: HeadCountMismatch, then
// BlockPageMismatch (forward.rs kvouter_forward, argument sanity).
sa_status check_heads_blocks(int32_t hq, int32_t hkv, int32_t head_dim, int32_t block_size,
                             int32_t page_size) {
  if (hkv <= 0 || hq <= 0 || hq % hkv != 0) return fail(SA_ERR_HEAD_COUNT, "", hq, hkv);
  if (head_dim <= 0 || block_size <= 0 || page_size <= 0 || block_size % page_size != 0)
    return fail(SA_ERR_BLOCK_PAGE, "", block_size, page_size);
  return SA_OK;
}

// Build-side length checks, in the order the oracle's builder uses.
sa_status check_build_lengths(int64_t selected_len, int64_t block_tables_len, int64_t cu_len,
                              const int32_t* used, int64_t used_len, int64_t tq, int32_t hkv,
                              int32_t topk, int32_t batch, int32_t max_pages,
                              int32_t block_size, int32_t page_size) {
  if (cu_len < 2) return fail(SA_ERR_CU_SEQLENS);
  if (block_size <= 0 || page_size <= 0 || block_size % page_size != 0)
    return fail(SA_ERR_BLOCK_PAGE, "", block_size, page_size);
  const int64_t want_sel = tq * (int64_t)hkv * topk;
  if (selected_len != want_sel) return fail(SA_ERR_SHAPE, "selected", want_sel, selected_len);
  const int64_t want_tbl = (int64_t)batch * max_pages;
  if (block_tables_len != want_tbl)
    return fail(SA_ERR_SHAPE, "block_tables", want_tbl, block_tables_len);
  if (cu_len - 1 != batch) return fail(SA_ERR_SHAPE, "block_tables rows", cu_len - 1, batch);
  if (used != nullptr && used_len != batch)
    return fail(SA_ERR_SHAPE, "used_kv_lens", batch, used_len);
  if (tq == 0 || hkv == 0 || topk == 0) return fail(SA_ERR_EMPTY);
  return SA_OK;
}

sa::BuildArgs build_args(const sa_index* idx, const int32_t* selected, const int32_t* bt,
                         const int64_t* cu, const int32_t* used) {
  sa::BuildArgs a{};
  a.selected = selected;
  a.block_tables = bt;
  a.cu = cu;
  a.used = used;
  a.tq = idx->tq;
  a.nbs = idx->nbs;
  a.num_pages = idx->num_pages;
  a.hkv = idx->hkv;
  a.topk = idx->topk;
  a.batch = idx->batch;
  a.max_pages = idx->max_pages;
  a.block_size = idx->block_size;
  a.page_size = idx->page_size;
  a.ppb = idx->pages_per_block;
  a.msb = idx->msb;
  a.qhead = idx->hq / idx->hkv;
  a.cap_edges = idx->cap_edges;
  a.wave_cap_edges = idx->wave_cap_edges;
  a.mfma_min_rows = idx->mfma_min_rows;
  a.epoch = next_epoch();
  a.cap_magic = sa::make_div_magic((uint32_t)(a.cap_edges > 0 ? a.cap_edges : 1));
  a.wave_cap_magic = sa::make_div_magic((uint32_t)(a.wave_cap_edges > 0 ? a.wave_cap_edges : 1));
  return a;
}

}  // namespace

namespace sa {

ScratchLayout scratch_layout(const sa_index* idx) {
  ScratchLayout L{};
  const size_t slots = (size_t)idx->hkv * (size_t)idx->nbs;
  size_t o = idx->off_scratch;
  L.cnt = o;     o = align256(o + 4 * slots);
  L.slot_uw = o; o = align256(o + 4 * slots);
  L.slot_um = o; o = align256(o + 4 * slots);
  L.head_e = o;  o = align256(o + 4 * (size_t)idx->hkv);
  L.head_uw = o; o = align256(o + 4 * (size_t)idx->hkv);
  L.head_um = o; o = align256(o + 4 * (size_t)idx->hkv);
  L.keys = o;    o = align256(o + 4 * (size_t)idx->max_edges);
  L.qinfo = o;   o = align256(o + 8 * (size_t)idx->tq);
  L.agg = o;     o = align256(o + sizeof(HeadAgg) * (size_t)idx->hkv);
  L.chunk_agg = o;
  o = align256(o + sizeof(ChunkAgg) * (size_t)idx->hkv * (size_t)scan_chunks(idx->nbs));
  L.units_sorted = o;
  o = align256(o + sizeof(Unit) * (size_t)idx->max_units);
  L.sort_hist = o;
  o = align256(o + sizeof(int32_t) * (size_t)kSortHistInts);
  L.end = o;
  return L;
}

IndexPtrs index_ptrs(const sa_index* idx) {
  char* b = static_cast<char*>(idx->buffer);
  const ScratchLayout L = scratch_layout(idx);
  IndexPtrs P{};
  P.hdr = reinterpret_cast<DevHeader*>(b + idx->off_header);
  P.sel_slots = reinterpret_cast<int32_t*>(b + idx->off_sel_slots);
  P.sel_offsets = reinterpret_cast<int32_t*>(b + idx->off_sel_offsets);
  P.num_sel = reinterpret_cast<int32_t*>(b + idx->off_num_sel);
  P.edge_head_base = reinterpret_cast<int64_t*>(b + idx->off_edge_head_base);
  P.edges = reinterpret_cast<int32_t*>(b + idx->off_edges);
  P.inv = reinterpret_cast<int32_t*>(b + idx->off_inv);
  P.units_wave = reinterpret_cast<Unit*>(b + idx->off_units_wave);
  P.units_mfma = reinterpret_cast<Unit*>(b + idx->off_units_mfma);
  P.cnt = reinterpret_cast<int32_t*>(b + L.cnt);
  P.slot_uw = reinterpret_cast<int32_t*>(b + L.slot_uw);
  P.slot_um = reinterpret_cast<int32_t*>(b + L.slot_um);
  P.head_e = reinterpret_cast<int32_t*>(b + L.head_e);
  P.head_uw = reinterpret_cast<int32_t*>(b + L.head_uw);
  P.head_um = reinterpret_cast<int32_t*>(b + L.head_um);
  P.keys = reinterpret_cast<int32_t*>(b + L.keys);
  P.qinfo = reinterpret_cast<int2*>(b + L.qinfo);
  P.agg = reinterpret_cast<HeadAgg*>(b + L.agg);
  P.chunk_agg = reinterpret_cast<ChunkAgg*>(b + L.chunk_agg);
  P.units_sorted = reinterpret_cast<Unit*>(b + L.units_sorted);
  P.sort_hist = reinterpret_cast<int32_t*>(b + L.sort_hist);
  return P;
}

}  // namespace sa

extern "C" {

const char* sa_status_string(sa_status st) {
  switch (st) {
    case SA_OK: return "ok";
    case SA_ERR_HEAD_COUNT: return "HeadCountMismatch";
    case SA_ERR_BLOCK_PAGE: return "BlockPageMismatch";
    case SA_ERR_CU_SEQLENS: return "CuSeqlensInvalid";
    case SA_ERR_SHAPE: return "ShapeMismatch";
    case SA_ERR_SELECTED_RANGE: return "SelectedOutOfRange";
    case SA_ERR_HEAD_DIM: return "HeadDimMismatch";
    case SA_ERR_EMPTY: return "EmptyInput";
    case SA_ERR_GPU_INIT: return "GpuInitFailed";
    case SA_ERR_GPU_RUNTIME: return "GpuRuntimeError";
    case SA_ERR_UNSUPPORTED: return "Unsupported";
  }
  return "unknown";
}

sa_status sa_last_error(sa_error_detail* out) {
  if (out) *out = g_last;
  return (sa_status)g_last.status;
}

sa_status sa_index_plan(int64_t tq, int32_t hkv, int32_t topk, int32_t batch, int32_t max_pages,
                        int32_t block_size, int32_t page_size, int32_t hq, int32_t head_dim,
                        int64_t num_pages, sa_index* idx) {
  if (idx == nullptr) return fail(SA_ERR_SHAPE, "idx (null)", 1, 0);
  if (batch < 1) return fail(SA_ERR_CU_SEQLENS);
  if (block_size <= 0 || page_size <= 0 || block_size % page_size != 0)
    return fail(SA_ERR_BLOCK_PAGE, "", block_size, page_size);
  if (tq <= 0 || hkv <= 0 || topk <= 0) return fail(SA_ERR_EMPTY);
  if (hq <= 0 || hq % hkv != 0) return fail(SA_ERR_HEAD_COUNT, "", hq, hkv);
  if (head_dim <= 0) return fail(SA_ERR_BLOCK_PAGE, "", block_size, page_size);
  if (max_pages < 0) return fail(SA_ERR_SHAPE, "block_tables", 0, max_pages);
  if (head_dim % 4 != 0 || head_dim > 256)
    return fail(SA_ERR_UNSUPPORTED, "head_dim must be a multiple of 4, at most 256", 256, head_dim);
  const int32_t qhead = hq / hkv;
  if ((int64_t)qhead * head_dim > 4096)
    return fail(SA_ERR_UNSUPPORTED, "(hq/hkv)*head_dim must be at most 4096", 4096,
                (int64_t)qhead * head_dim);
  const int64_t max_edges = tq * (int64_t)hkv * topk;
  if (max_edges * (int64_t)qhead >= INT32_MAX || tq * (int64_t)topk >= INT32_MAX)
    return fail(SA_ERR_UNSUPPORTED, "tq*hkv*topk*qhead must stay below 2^31", INT32_MAX,
                max_edges * qhead);
  const int64_t kv_cap = (int64_t)(max_pages / (block_size / page_size)) * block_size;
  if (block_size >= (1 << 20) || kv_cap >= INT32_MAX)
    return fail(SA_ERR_UNSUPPORTED, "block_size < 2^20 and msb*block_size < 2^31",
                1 << 20, block_size);
  std::memset(idx, 0, sizeof(*idx));
  idx->tq = tq;
  idx->hkv = hkv;
  idx->topk = topk;
  idx->batch = batch;
  idx->max_pages = max_pages;
  idx->block_size = block_size;
  idx->page_size = page_size;
  idx->hq = hq;
  idx->head_dim = head_dim;
  idx->num_pages = num_pages;
  idx->pages_per_block = block_size / page_size;
  idx->msb = max_pages / idx->pages_per_block;
  idx->nbs = (int64_t)batch * idx->msb;
  idx->max_edges = max_edges;
  idx->cap_edges = sa::kCapRows / qhead > 0 ? sa::kCapRows / qhead : 1;
  if (idx->cap_edges > sa::kCapUnitEdges) idx->cap_edges = sa::kCapUnitEdges;
  const bool mfma_ok = ((head_dim == sa::kMfmaHeadDim && block_size <= sa::kMfmaMaxBlock) ||
                        sa::mfma_general_fits(head_dim, block_size)) &&
                       sa::mfma_enabled();
  // The chunked kernel holds one 32-row tile a wave across a block's chunks:
  // for blocks of more than one chunk a unit takes at most a workgroup's
  // tiles, so that each chunk is gathered once a unit.
  if (mfma_ok && sa::mfma_general_fits(head_dim, block_size) &&
      block_size > sa::mfma_general_chunk_keys(head_dim, block_size)) {
    const int32_t cap = sa::mfma_general_tile_rows(head_dim) / qhead;
    idx->cap_edges = cap < 1 ? 1 : (cap < idx->cap_edges ? cap : idx->cap_edges);
  }
  // Where the one-wave-per-unit kernel fits (head_dim 128, blocks of at most
  // 64 keys, qhead <= 16) it takes every slot: a slot with more than 16 rows
  // becomes several 16-row units that read the same block close together in
  // time, so the repeat reads mostly hit L2 / MALL. Measured on MI355X this
  // beats the LDS-staged MFMA kernel on the ragged mixed batch (forward 446 ->
  // 382 us) and on slots shared by hundreds of queries; the MFMA kernels
  // take the other geometries, from kMfmaMinRows rows a slot.
  const bool small_fit = sa::small_kernel_fits(head_dim, block_size, page_size, qhead);
  idx->mfma_min_rows = (mfma_ok && !small_fit) ? sa::kMfmaMinRows : INT32_MAX;
  idx->wave_cap_edges = small_fit
                            ? (sa::small_kernel_rows() / qhead > 0 ? sa::small_kernel_rows() / qhead : 1)
                            : idx->cap_edges;
  const int64_t slots = (int64_t)hkv * idx->nbs;
  const int32_t min_cap = idx->wave_cap_edges < idx->cap_edges ? idx->wave_cap_edges : idx->cap_edges;
  idx->max_units = (slots < max_edges ? slots : max_edges) + max_edges / min_cap + 1;
  size_t o = 0;
  idx->off_header = o;          o = align256(o + sizeof(sa::DevHeader));
  idx->off_sel_slots = o;       o = align256(o + 4 * (size_t)slots);
  idx->off_sel_offsets = o;     o = align256(o + 4 * (size_t)hkv * (size_t)(idx->nbs + 1));
  idx->off_num_sel = o;         o = align256(o + 4 * (size_t)hkv);
  idx->off_edge_head_base = o;  o = align256(o + 8 * (size_t)(hkv + 1));
  idx->off_edges = o;           o = align256(o + 8 * (size_t)max_edges);
  idx->off_inv = o;             o = align256(o + 4 * (size_t)max_edges);
  idx->off_units_wave = o;      o = align256(o + sizeof(sa::Unit) * (size_t)idx->max_units);
  idx->off_units_mfma = o;      o = align256(o + sizeof(sa::Unit) * (size_t)idx->max_units);
  idx->off_scratch = o;
  idx->index_bytes = sa::scratch_layout(idx).end;
  idx->buffer = nullptr;
  return ok();
}

sa_status sa_build_index(const int32_t* selected, int64_t selected_len,
                         const int32_t* block_tables, int64_t block_tables_len,
                         const int64_t* cu_seqlens_q, int64_t cu_len,
                         const int32_t* used_kv_lens, int64_t used_len,
                         sa_index* idx, hipStream_t stream) {
  if (idx == nullptr) return fail(SA_ERR_SHAPE, "idx (null)", 1, 0);
  sa_status st = check_build_lengths(selected_len, block_tables_len, cu_len, used_kv_lens,
                                     used_len, idx->tq, idx->hkv, idx->topk, idx->batch,
                                     idx->max_pages, idx->block_size, idx->page_size);
  if (st != SA_OK) return st;
  if (idx->buffer == nullptr || (reinterpret_cast<uintptr_t>(idx->buffer) & 255) != 0)
    return fail(SA_ERR_SHAPE, "index buffer (null or not 256-byte aligned)", 256, 0);
  sa_index chk;
  if (sa_index_plan(idx->tq, idx->hkv, idx->topk, idx->batch, idx->max_pages, idx->block_size,
                    idx->page_size, idx->hq, idx->head_dim, idx->num_pages, &chk) != SA_OK)
    return (sa_status)g_last.status;
  if (chk.index_bytes > idx->index_bytes)
    return fail(SA_ERR_SHAPE, "index buffer", (int64_t)chk.index_bytes, (int64_t)idx->index_bytes);
  if (!check_device()) return fail(SA_ERR_GPU_INIT, "no HIP device");
  const sa::BuildArgs a = build_args(idx, selected, block_tables, cu_seqlens_q, used_kv_lens);
  hipError_t e = sa::launch_build(idx, a, stream);
  if (e != hipSuccess) return runtime_error(e, "index build launch");
  return ok();
}

sa_status sa_index_status(const sa_index* idx, sa_index_info* out, hipStream_t stream) {
  if (idx == nullptr || idx->buffer == nullptr) return fail(SA_ERR_SHAPE, "idx (null)", 1, 0);
  sa::DevHeader h;
  hipError_t e = hipMemcpyAsync(&h, static_cast<char*>(idx->buffer) + idx->off_header,
                                sizeof(h), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return runtime_error(e, "index status readback");
  sa_index_info info{};
  info.status = h.status;
  const char* what = h.what_code == sa::kWhatCuTotal ? "cu_seqlens_q total"
                     : h.what_code == sa::kWhatPageId ? "block_tables page id" : "";
  std::snprintf(info.what, sizeof(info.what), "%s", what);
  info.expected = h.err_expected;
  info.got = h.err_got;
  info.total_edges = h.total_edges;
  info.num_units_wave = h.num_units_wave;
  info.num_units_mfma = h.num_units_mfma;
  info.num_slots = h.num_slots;
  if (out) *out = info;
  if (h.status != SA_OK) return fail((sa_status)h.status, info.what, info.expected, info.got);
  return ok();
}

}  // extern "C"

namespace {

// sa_forward's checks (in the page's order) and launch, for K/V pages stored
// as fp32 or, with `kv16`, as 16-bit words of `kv_format` (`k`, `v` then
// hold uint16 elements; formats and geometry are checked after the others).
sa_status forward_checks(const sa_index* idx, const float* q, int64_t q_len, const void* k_pages,
                         int64_t k_len, const void* v_pages, int64_t v_len,
                         const int32_t* block_tables, const int64_t* cu_seqlens_q,
                         const int32_t* used_kv_lens, int32_t hq, int32_t hkv, int32_t head_dim,
                         int32_t block_size, int32_t page_size, float softmax_scale,
                         int32_t causal, bool kv16, int32_t kv_format, float* o_partial,
                         float* m_partial, float* l_partial, sa::FwdArgs* args) {
  sa_status st = check_heads_blocks(hq, hkv, head_dim, block_size, page_size);
  if (st != SA_OK) return st;
  if (idx == nullptr || idx->buffer == nullptr) return fail(SA_ERR_SHAPE, "idx (null)", 1, 0);
  if (idx->hkv != hkv || idx->pages_per_block != block_size / page_size)
    return fail(SA_ERR_SHAPE, "idx (hkv or pages_per_block)", hkv, idx->hkv);
  if (idx->hq != hq || idx->head_dim != head_dim || idx->block_size != block_size)
    return fail(SA_ERR_SHAPE, "idx (planned hq/head_dim)", hq, idx->hq);
  const int64_t want_q = idx->tq * hq * (int64_t)head_dim;
  if (q_len != want_q) return fail(SA_ERR_SHAPE, "q", want_q, q_len);
  const int64_t page_stride = (int64_t)hkv * page_size * head_dim;
  if (k_len % page_stride != 0 || v_len != k_len)
    return fail(SA_ERR_SHAPE, "k_pages / v_pages page stride", page_stride, k_len);
  const int64_t num_pages = k_len / page_stride;
  if (idx->num_pages < 0 || num_pages < idx->num_pages)
    return fail(SA_ERR_SHAPE, "k_pages / v_pages pages", idx->num_pages, num_pages);
  if (kv16 && kv_format != SA_KV_BF16 && kv_format != SA_KV_F16)
    return fail(SA_ERR_UNSUPPORTED, "kv_format", SA_KV_BF16, kv_format);
  if (!check_device()) return fail(SA_ERR_GPU_INIT, "no HIP device");
  sa::FwdArgs a{};
  a.q = q;
  a.k = static_cast<const float*>(k_pages);
  a.v = static_cast<const float*>(v_pages);
  a.kv_format = kv_format;
  a.block_tables = block_tables;
  a.cu = cu_seqlens_q;
  a.used = used_kv_lens;
  a.o = o_partial;
  a.m = m_partial;
  a.l = l_partial;
  a.nbs = idx->nbs;
  a.num_pages = num_pages;
  a.hq = hq;
  a.hkv = hkv;
  a.qhead = hq / hkv;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.page_size = page_size;
  a.ppb = block_size / page_size;
  a.msb = idx->msb;
  a.max_pages = idx->max_pages;
  a.batch = idx->batch;
  a.causal = causal != 0;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.ps_magic = sa::make_div_magic((uint32_t)page_size);
  *args = a;
  return SA_OK;
}

sa_status forward_common(const sa_index* idx, const float* q, int64_t q_len, const void* k_pages,
                         int64_t k_len, const void* v_pages, int64_t v_len,
                         const int32_t* block_tables, const int64_t* cu_seqlens_q,
                         const int32_t* used_kv_lens, int32_t hq, int32_t hkv, int32_t head_dim,
                         int32_t block_size, int32_t page_size, float softmax_scale,
                         int32_t causal, bool kv16, int32_t kv_format, float* o_partial,
                         float* m_partial, float* l_partial, hipStream_t stream) {
  sa::FwdArgs a{};
  sa_status st = forward_checks(idx, q, q_len, k_pages, k_len, v_pages, v_len, block_tables,
                                cu_seqlens_q, used_kv_lens, hq, hkv, head_dim, block_size,
                                page_size, softmax_scale, causal, kv16, kv_format, o_partial,
                                m_partial, l_partial, &a);
  if (st != SA_OK) return st;
  hipError_t e = sa::launch_forward(idx, a, stream);
  if (e != hipSuccess) return runtime_error(e, "forward launch");
  return ok();
}

// sa_attention's host checks, in its order (the forward's, then the
// build's, then the plan's): fills the plan and the workspace size.
sa_status attention_host_checks(int64_t q_len, int64_t k_len, int64_t v_len,
                                int64_t selected_len, int64_t block_tables_len, int64_t cu_len,
                                const int32_t* used_kv_lens, int64_t used_len, int64_t tq,
                                int32_t hq, int32_t hkv, int32_t head_dim, int32_t topk,
                                int32_t batch, int32_t max_pages, int32_t block_size,
                                int32_t page_size, sa_index* idx, size_t* need);

}  // namespace

extern "C" {

sa_status sa_forward(const sa_index* idx, const float* q, int64_t q_len, const float* k_pages,
                     int64_t k_len, const float* v_pages, int64_t v_len,
                     const int32_t* block_tables,
                     const int64_t* cu_seqlens_q, const int32_t* used_kv_lens, int32_t hq,
                     int32_t hkv, int32_t head_dim, int32_t block_size, int32_t page_size,
                     float softmax_scale, int32_t causal, float* o_partial, float* m_partial,
                     float* l_partial, hipStream_t stream) {
  return forward_common(idx, q, q_len, k_pages, k_len, v_pages, v_len, block_tables, cu_seqlens_q,
                        used_kv_lens, hq, hkv, head_dim, block_size, page_size, softmax_scale,
                        causal, false, SA_KV_F32, o_partial, m_partial, l_partial, stream);
}

sa_status sa_forward_kv16(const sa_index* idx, const float* q, int64_t q_len,
                          const uint16_t* k_pages, int64_t k_len, const uint16_t* v_pages,
                          int64_t v_len, int32_t kv_format, const int32_t* block_tables,
                          const int64_t* cu_seqlens_q, const int32_t* used_kv_lens, int32_t hq,
                          int32_t hkv, int32_t head_dim, int32_t block_size, int32_t page_size,
                          float softmax_scale, int32_t causal, float* o_partial,
                          float* m_partial, float* l_partial, hipStream_t stream) {
  return forward_common(idx, q, q_len, k_pages, k_len, v_pages, v_len, block_tables, cu_seqlens_q,
                        used_kv_lens, hq, hkv, head_dim, block_size, page_size, softmax_scale,
                        causal, true, kv_format, o_partial, m_partial, l_partial, stream);
}

sa_status sa_combine(const sa_index* idx, const float* o_partial, const float* m_partial,
                     const float* l_partial, int32_t hq, int32_t head_dim, float* out,
                     float* lse, hipStream_t stream) {
  if (idx == nullptr || idx->buffer == nullptr) return fail(SA_ERR_SHAPE, "idx (null)", 1, 0);
  if (hq != idx->hq || head_dim != idx->head_dim)
    return fail(SA_ERR_SHAPE, "idx (planned hq/head_dim)", hq, idx->hq);
  if (!check_device()) return fail(SA_ERR_GPU_INIT, "no HIP device");
  sa::CombineArgs a{};
  a.o = o_partial;
  a.m = m_partial;
  a.l = l_partial;
  a.out = out;
  a.lse = lse;
  a.tq = idx->tq;
  a.hq = hq;
  a.hkv = idx->hkv;
  a.qhead = hq / idx->hkv;
  a.head_dim = head_dim;
  a.topk = idx->topk;
  hipError_t e = sa::launch_combine(idx, a, stream);
  if (e != hipSuccess) return runtime_error(e, "combine launch");
  return ok();
}

namespace {

// sa_forward_combine's checks (sa_forward's, then the selections and the
// fused geometry) and launch, for fp32 or 16-bit pages
sa_status forward_combine_impl(const sa_index* idx, const int32_t* selected, int64_t selected_len,
                               const float* q, int64_t q_len, const void* k_pages, int64_t k_len,
                               const void* v_pages, int64_t v_len, bool kv16, int32_t kv_format,
                               const int32_t* block_tables, const int64_t* cu_seqlens_q,
                               const int32_t* used_kv_lens, int32_t hq, int32_t hkv,
                               int32_t head_dim, int32_t block_size, int32_t page_size,
                               float softmax_scale, int32_t causal, float* out, float* lse,
                               hipStream_t stream) {
  sa::FwdArgs a{};
  sa_status st = forward_checks(idx, q, q_len, k_pages, k_len, v_pages, v_len, block_tables,
                                cu_seqlens_q, used_kv_lens, hq, hkv, head_dim, block_size,
                                page_size, softmax_scale, causal, kv16, kv_format, nullptr,
                                nullptr, nullptr, &a);
  if (st != SA_OK) return st;
  const int64_t want_sel = idx->tq * (int64_t)idx->hkv * idx->topk;
  if (selected_len != want_sel) return fail(SA_ERR_SHAPE, "selected", want_sel, selected_len);
  if (!sa::fused_kernel_fits(head_dim, block_size, page_size, hq / hkv, idx->topk))
    return fail(SA_ERR_UNSUPPORTED,
                "fused forward: head_dim 128, blocks of at most 64 keys, hq/hkv <= 16, topk <= 512",
                128, head_dim);
  hipError_t e = sa::launch_forward_fused(idx, a, selected, out, lse, stream);
  if (e != hipSuccess) return runtime_error(e, "fused forward launch");
  return ok();
}

}  // namespace

sa_status sa_forward_combine(const sa_index* idx, const int32_t* selected, int64_t selected_len,
                             const float* q, int64_t q_len, const float* k_pages, int64_t k_len,
                             const float* v_pages, int64_t v_len, const int32_t* block_tables,
                             const int64_t* cu_seqlens_q, const int32_t* used_kv_lens,
                             int32_t hq, int32_t hkv, int32_t head_dim, int32_t block_size,
                             int32_t page_size, float softmax_scale, int32_t causal, float* out,
                             float* lse, hipStream_t stream) {
  return forward_combine_impl(idx, selected, selected_len, q, q_len, k_pages, k_len, v_pages,
                              v_len, false, SA_KV_F32, block_tables, cu_seqlens_q, used_kv_lens,
                              hq, hkv, head_dim, block_size, page_size, softmax_scale, causal,
                              out, lse, stream);
}

sa_status sa_forward_combine_kv16(const sa_index* idx, const int32_t* selected,
                                  int64_t selected_len, const float* q, int64_t q_len,
                                  const uint16_t* k_pages, int64_t k_len,
                                  const uint16_t* v_pages, int64_t v_len, int32_t kv_format,
                                  const int32_t* block_tables, const int64_t* cu_seqlens_q,
                                  const int32_t* used_kv_lens, int32_t hq, int32_t hkv,
                                  int32_t head_dim, int32_t block_size, int32_t page_size,
                                  float softmax_scale, int32_t causal, float* out, float* lse,
                                  hipStream_t stream) {
  return forward_combine_impl(idx, selected, selected_len, q, q_len, k_pages, k_len, v_pages,
                              v_len, true, kv_format, block_tables, cu_seqlens_q, used_kv_lens,
                              hq, hkv, head_dim, block_size, page_size, softmax_scale, causal,
                              out, lse, stream);
}

sa_status sa_attention_workspace_bytes(int64_t tq, int32_t hkv, int32_t topk, int32_t batch,
                                       int32_t max_pages, int32_t block_size, int32_t page_size,
                                       int32_t hq, int32_t head_dim, size_t* bytes) {
  sa_index idx;
  sa_status st = sa_index_plan(tq, hkv, topk, batch, max_pages, block_size, page_size, hq,
                               head_dim, 0, &idx);
  if (st != SA_OK) return st;
  const size_t rows = (size_t)idx.max_edges * (size_t)(hq / hkv);
  size_t o = align256(idx.index_bytes);
  o = align256(o + rows * (size_t)head_dim * 4);   // o_partial
  o = align256(o + rows * 4);                      // m_partial
  o = align256(o + rows * 4);                      // l_partial
  if (bytes) *bytes = o;
  return ok();
}

}  // extern "C"

namespace {

sa_status attention_host_checks(int64_t q_len, int64_t k_len, int64_t v_len,
                                int64_t selected_len, int64_t block_tables_len, int64_t cu_len,
                                const int32_t* used_kv_lens, int64_t used_len, int64_t tq,
                                int32_t hq, int32_t hkv, int32_t head_dim, int32_t topk,
                                int32_t batch, int32_t max_pages, int32_t block_size,
                                int32_t page_size, sa_index* idx, size_t* need) {
  sa_status st = check_heads_blocks(hq, hkv, head_dim, block_size, page_size);
  if (st != SA_OK) return st;
  st = check_build_lengths(selected_len, block_tables_len, cu_len, used_kv_lens, used_len, tq,
                           hkv, topk, batch, max_pages, block_size, page_size);
  if (st != SA_OK) return st;
  const int64_t want_q = tq * hq * (int64_t)head_dim;
  if (q_len != want_q) return fail(SA_ERR_SHAPE, "q", want_q, q_len);
  const int64_t page_stride = (int64_t)hkv * page_size * head_dim;
  if (k_len % page_stride != 0 || v_len != k_len)
    return fail(SA_ERR_SHAPE, "k_pages / v_pages page stride", page_stride, k_len);
  const int64_t num_pages = k_len / page_stride;
  st = sa_index_plan(tq, hkv, topk, batch, max_pages, block_size, page_size, hq, head_dim,
                     num_pages, idx);
  if (st != SA_OK) return st;
  return sa_attention_workspace_bytes(tq, hkv, topk, batch, max_pages, block_size, page_size,
                                      hq, head_dim, need);
}

}  // namespace

extern "C" {

sa_status sa_attention(const float* q, int64_t q_len, const float* k_pages, int64_t k_len,
                       const float* v_pages, int64_t v_len, const int32_t* selected,
                       int64_t selected_len,
                       const int32_t* block_tables, int64_t block_tables_len,
                       const int64_t* cu_seqlens_q, int64_t cu_len, const int32_t* used_kv_lens,
                       int64_t used_len, int64_t tq, int32_t hq, int32_t hkv, int32_t head_dim,
                       int32_t topk, int32_t batch, int32_t max_pages, int32_t block_size,
                       int32_t page_size, float softmax_scale, int32_t causal, void* workspace,
                       size_t workspace_bytes, float* out, float* lse, sa_index* idx_out,
                       hipStream_t stream) {
  sa_index idx;
  size_t need = 0;
  sa_status st = attention_host_checks(q_len, k_len, v_len, selected_len, block_tables_len,
                                       cu_len, used_kv_lens, used_len, tq, hq, hkv, head_dim,
                                       topk, batch, max_pages, block_size, page_size, &idx,
                                       &need);
  if (st != SA_OK) return st;
  if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 255) != 0 ||
      workspace_bytes < need)
    return fail(SA_ERR_SHAPE, "workspace", (int64_t)need, (int64_t)workspace_bytes);
  idx.buffer = workspace;
  const size_t rows = (size_t)idx.max_edges * (size_t)(hq / hkv);
  char* w = static_cast<char*>(workspace);
  size_t o = align256(idx.index_bytes);
  float* o_part = reinterpret_cast<float*>(w + o);
  o = align256(o + rows * (size_t)head_dim * 4);
  float* m_part = reinterpret_cast<float*>(w + o);
  o = align256(o + rows * 4);
  float* l_part = reinterpret_cast<float*>(w + o);
  st = sa_build_index(selected, selected_len, block_tables, block_tables_len, cu_seqlens_q,
                      cu_len, used_kv_lens, used_len, &idx, stream);
  if (st != SA_OK) return st;
  if (tq == batch && sa::fused_kernel_fits(head_dim, block_size, page_size, hq / hkv, topk)) {
    // one query per sequence on average (decode): forward and combine in one
    // launch, no partials in memory
    st = sa_forward_combine(&idx, selected, selected_len, q, q_len, k_pages, k_len, v_pages,
                            v_len, block_tables, cu_seqlens_q, used_kv_lens, hq, hkv, head_dim,
                            block_size, page_size, softmax_scale, causal, out, lse, stream);
    if (st != SA_OK) return st;
  } else {
    st = sa_forward(&idx, q, q_len, k_pages, k_len, v_pages, v_len, block_tables, cu_seqlens_q,
                    used_kv_lens, hq, hkv, head_dim, block_size, page_size, softmax_scale, causal,
                    o_part, m_part, l_part, stream);
    if (st != SA_OK) return st;
    st = sa_combine(&idx, o_part, m_part, l_part, hq, head_dim, out, lse, stream);
    if (st != SA_OK) return st;
  }
  if (idx_out) *idx_out = idx;
  return ok();
}

}  // extern "C"

// ------------------------------------------------------------ allocation-free entry
// Workspace of sa_attention_noalloc: a file-scope device array that the code
// object's loader places on every GPU the library runs on (each GPU has its
// own copy at its own address). In host code `scratch` names a host-side
// stand-in, never the device memory: every host use goes through the device
// address that hipGetSymbolAddress returns, looked up once per device.
static __device__ __align__(256) unsigned char scratch[SA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (first call on a device:
// looked up with that device current), or null with the failure recorded.
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    fail(SA_ERR_GPU_INIT, "no HIP device");
    return nullptr;
  }
  if (dev >= kMaxDevices) {
    fail(SA_ERR_UNSUPPORTED, "device ordinal", kMaxDevices, dev);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      runtime_error(e, "scratch symbol address");
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

sa_status sa_attention_noalloc(const float* q, int64_t q_len, const float* k_pages,
                               int64_t k_len, const float* v_pages, int64_t v_len,
                               const int32_t* selected, int64_t selected_len,
                               const int32_t* block_tables, int64_t block_tables_len,
                               const int64_t* cu_seqlens_q, int64_t cu_len,
                               const int32_t* used_kv_lens, int64_t used_len, int64_t tq,
                               int32_t hq, int32_t hkv, int32_t head_dim, int32_t topk,
                               int32_t batch, int32_t max_pages, int32_t block_size,
                               int32_t page_size, float softmax_scale, int32_t causal,
                               float* out, float* lse, sa_index* idx_out,
                               hipStream_t stream) {
  // the host checks of sa_attention come first, in its order
  sa_index plan;
  size_t need = 0;
  sa_status st = attention_host_checks(q_len, k_len, v_len, selected_len, block_tables_len,
                                       cu_len, used_kv_lens, used_len, tq, hq, hkv, head_dim,
                                       topk, batch, max_pages, block_size, page_size, &plan,
                                       &need);
  if (st != SA_OK) return st;
  if (need > (size_t)SA_NOALLOC_SCRATCH_BYTES)
    return fail(SA_ERR_UNSUPPORTED, "workspace exceeds the no-alloc scratch",
                (int64_t)SA_NOALLOC_SCRATCH_BYTES, (int64_t)need);
  void* ws = scratch_for_current_device();
  if (ws == nullptr) return (sa_status)g_last.status;
  return sa_attention(q, q_len, k_pages, k_len, v_pages, v_len, selected, selected_len,
                      block_tables, block_tables_len, cu_seqlens_q, cu_len, used_kv_lens,
                      used_len, tq, hq, hkv, head_dim, topk, batch, max_pages, block_size,
                      page_size, softmax_scale, causal, ws, (size_t)SA_NOALLOC_SCRATCH_BYTES,
                      out, lse, idx_out, stream);
}

}  // extern "C"
