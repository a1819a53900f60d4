/*
 * sa.h: C ABI of the KV-outer block-sparse paged attention library (gfx950).
 *
 * The operation follows the alice-llm 2.0.0 `sparse_attention` pages
 * (docs.rs source view): types.rs (SparseSelection, BlockTables,
 * CuSeqlensQ, KvOuterIndex, SparseAttentionError) and forward.rs
 * (kvouter_forward, ForwardPartials, process_work_unit). gpu.rs shows the
 * builder call `build_kvouter_index(&sel, &tbl, &cu, Some(&used),
 * block_size, page_size)`.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless the comment says "host". The caller
 *    allocates and owns every buffer; the library allocates no memory and
 *    keeps no data between calls (a process-wide build counter aside, which
 *    tags the device-side handshake of one build).
 *  - All GPU work is enqueued on `stream` and runs asynchronously. Only
 *    sa_index_status() waits for the stream.
 *  - Scalar and length checks run on the host before anything is enqueued.
 *    They run in the order the pages use and return a non-zero sa_status.
 *    The detail is then available from sa_last_error() on the same host thread.
 *  - Checks that need device data (cu_seqlens_q content, selected ids,
 *    block-table page ids) run inside the build kernels. They record the
 *    first failure in the index's device header. On an index whose header
 *    holds an error, sa_forward writes nothing and sa_combine writes NaN to
 *    every element of `out` (and `lse`), so that a caller who does not wait
 *    for the status never reads stale memory as a result. The pages' forward
 *    returns the error instead; reporting it here would need a host wait.
 *    Call sa_index_status() to read the error.
 *  - Layouts are row-major and element types are as stated: float32 for
 *    q/K/V/partials/outputs, int32 for ids, int64 for cu_seqlens_q.
 */
#ifndef SA_H
#define SA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes: the SparseAttentionError variants of types.rs, plus the
 * limits of this library. */
typedef enum sa_status {
  SA_OK = 0,
  SA_ERR_HEAD_COUNT = 1,     /* HeadCountMismatch: hq, hkv > 0 and hq % hkv == 0 */
  SA_ERR_BLOCK_PAGE = 2,     /* BlockPageMismatch: head_dim, block_size, page_size > 0,
                                block_size % page_size == 0 */
  SA_ERR_CU_SEQLENS = 3,     /* CuSeqlensInvalid: len >= 2, cu[0] == 0, non-decreasing */
  SA_ERR_SHAPE = 4,          /* ShapeMismatch {what, expected, got} */
  SA_ERR_SELECTED_RANGE = 5, /* SelectedOutOfRange {got, msb}: id outside [-1, msb) */
  SA_ERR_HEAD_DIM = 6,       /* HeadDimMismatch (raised by the Python binding) */
  SA_ERR_EMPTY = 7,          /* EmptyInput: tq == 0 || hkv == 0 || topk == 0 */
  SA_ERR_GPU_INIT = 8,       /* GpuInitFailed: no usable gfx950 device */
  SA_ERR_GPU_RUNTIME = 9,    /* GpuRuntimeError: a HIP call failed */
  SA_ERR_UNSUPPORTED = 10    /* outside this library's limits (see sa_index_plan) */
} sa_status;

/* Host-side detail of the last failed call on this host thread. */
typedef struct sa_error_detail {
  int32_t status;      /* sa_status */
  char what[64];       /* the ShapeMismatch `what`, or a short reason */
  int64_t expected;    /* ShapeMismatch expected / SelectedOutOfRange msb */
  int64_t got;         /* ShapeMismatch got / SelectedOutOfRange id */
} sa_error_detail;

/* Index handle. It is a host struct that sa_index_plan() fills. It mirrors
 * the scalars of KvOuterIndex (types.rs) and points at one caller-owned
 * device buffer holding every index array:
 *
 *   sel_slots      int32 [hkv, nbs]    compact rank -> raw slot b*msb+blk, -1 tail
 *   sel_offsets    int32 [hkv, nbs+1]  head-local CSR offsets, plateau at E_h
 *   num_sel        int32 [hkv]         nonempty compact slots per head
 *   edge_head_base int64 [hkv+1]       exclusive prefix of E_h over heads
 *   edges          int32 [E, 2]        (query, rank) in CSR order across heads
 *   inv            int32 [hkv, tq, topk]  head-local edge position, or -1
 *   units          int32 [U, 8]        work units: head, compact slot, e0, e1 (the
 *                                      WorkSplit fields of forward.rs), then the
 *                                      slot's batch b and block blk, lk_b, and d with
 *                                      causal limit(q) = q + d
 *
 * E (kept edges) is known only on the device. Buffers are sized for the
 * worst case max_edges = tq*hkv*topk. The offsets below are byte offsets
 * into `buffer`. */
typedef struct sa_index {
  void* buffer;              /* device, caller-owned, >= index_bytes, 256-B aligned */
  size_t index_bytes;
  int64_t tq;
  int32_t hkv, topk, batch, max_pages, block_size, page_size;
  int32_t hq, head_dim;      /* forward geometry the work units were planned for */
  int64_t num_pages;         /* page ids >= num_pages are rejected by the build */
  int32_t pages_per_block, msb;
  int64_t nbs;               /* batch * msb */
  int64_t max_edges;         /* tq * hkv * topk */
  int64_t max_units;
  int32_t cap_edges;         /* most edges in one MFMA work unit */
  int32_t wave_cap_edges;    /* most edges in one wavefront-path work unit */
  int32_t mfma_min_rows;     /* slots with at least this many rows use MFMA */
  size_t off_header, off_sel_slots, off_sel_offsets, off_num_sel, off_edge_head_base,
         off_edges, off_inv, off_units_wave, off_units_mfma, off_scratch;
} sa_index;

/* Device-side outcome of a build, read back by sa_index_status(). */
typedef struct sa_index_info {
  int32_t status;            /* sa_status of the first device-detected error, or SA_OK */
  char what[64];
  int64_t expected, got;
  int64_t total_edges;       /* E */
  int32_t num_units_wave;    /* units on the wavefront-reduction path */
  int32_t num_units_mfma;    /* units on the MFMA path */
  int64_t num_slots;         /* sum over heads of num_sel */
} sa_index_info;

/* sa_index_plan: fill `idx` (host) with the geometry and layout for one build.
 * Computes msb = max_pages / (block_size / page_size), nbs = batch * msb and
 * the buffer size (types.rs, KvOuterIndex field docs). No GPU call. `buffer`
 * is left NULL. Set it to a device allocation of idx->index_bytes before
 * sa_build_index.
 * Checks, in order: batch >= 1 (else CU_SEQLENS); block/page (BLOCK_PAGE);
 * tq, hkv, topk > 0 (EMPTY); hq > 0 and hq % hkv == 0 (HEAD_COUNT);
 * head_dim > 0 (BLOCK_PAGE); max_pages >= 0 (SHAPE "block_tables");
 * head_dim % 4 == 0 and <= 256, (hq/hkv)*head_dim <= 4096,
 * tq*hkv*topk*(hq/hkv) < 2^31, block_size < 2^20 and msb*block_size < 2^31
 * (UNSUPPORTED). */
sa_status sa_index_plan(int64_t tq, int32_t hkv, int32_t topk, int32_t batch,
                        int32_t max_pages, int32_t block_size, int32_t page_size,
                        int32_t hq, int32_t head_dim, int64_t num_pages,
                        sa_index* idx /* host, out */);

/* sa_build_index: build the KV-outer CSR index (types.rs KvOuterIndex; the
 * builder call in gpu.rs's tests) and the work units on the device.
 *   selected      int32 [tq, hkv, topk], -1 = padding rank (SparseSelection)
 *   block_tables  int32 [batch, max_pages], -1 = no page (BlockTables)
 *   cu_seqlens_q  int64 [batch+1] (CuSeqlensQ)
 *   used_kv_lens  int32 [batch] or NULL. lk_b = max(used[b], 0), or msb*block_size
 * A rank is dropped (inv = -1) if it is -1 or its block starts at or past
 * lk_b. Within a slot, edges are in ascending (query, rank) order.
 * Host checks, in order: cu_len >= 2 (CU_SEQLENS); block/page (BLOCK_PAGE);
 * selected_len == tq*hkv*topk (SHAPE "selected"); block_tables_len ==
 * batch*max_pages (SHAPE "block_tables"); cu_len-1 == batch (SHAPE
 * "block_tables rows"); used_len == batch when used is given (SHAPE
 * "used_kv_lens"); EMPTY; idx->buffer set, 256-byte aligned and
 * index_bytes large enough (SHAPE "index buffer"). The geometry (tq, hkv,
 * topk, batch, max_pages, block_size, page_size, num_pages) is the one
 * sa_index_plan() stored in `idx`.
 * Device checks, reported by sa_index_status in this priority:
 * cu[0] != 0 or decreasing (CU_SEQLENS); cu[batch] != tq (SHAPE
 * "cu_seqlens_q total"); the first id outside [-1, msb) in memory order
 * (SELECTED_RANGE); the first block-table entry >= num_pages, in memory
 * order, among pages that a kept block's valid range touches (SHAPE
 * "block_tables page id").
 * Work units split each slot of n edges into near-equal, consecutive ranges:
 * ceil(n / cap_edges) units for the MFMA kernel if n*(hq/hkv) >= mfma_min_rows,
 * else ceil(n / wave_cap_edges) units for the wavefront kernels.
 * The kernels are chosen from the sizes; two environment variables, read at
 * each call, override the choice for testing and leave the index unchanged:
 * SA_BUILD_MULTIKERNEL=1 keeps small problems off the one-kernel build, and
 * SA_BUILD_AGG=1 / 0 turns the multi-kernel build's per-workgroup (LDS)
 * counting on / off where hkv*msb <= 8192. */
sa_status sa_build_index(const int32_t* selected, int64_t selected_len,
                         const int32_t* block_tables, int64_t block_tables_len,
                         const int64_t* cu_seqlens_q, int64_t cu_len,
                         const int32_t* used_kv_lens, int64_t used_len,
                         sa_index* idx, hipStream_t stream);

/* sa_index_status: wait for `stream`, then copy the device header of `idx`
 * to `out` (host). The return value equals out->status. */
sa_status sa_index_status(const sa_index* idx, sa_index_info* out, hipStream_t stream);

/* sa_forward: KV-outer forward (forward.rs, kvouter_forward and
 * process_work_unit). For every kept edge e = (q, r) of head h, and every
 * GQA lane qh (query head h*qhead + qh), it writes the partial row
 * e*qhead + qh:
 *   o_partial float32 [E*qhead, head_dim]  sum_t exp(s_t - m) v_t (unnormalised)
 *   m_partial float32 [E*qhead]            m = max_t s_t
 *   l_partial float32 [E*qhead]            sum_t exp(s_t - m)
 * s_t = dot(q, k_t) * softmax_scale over the block's positions t in
 * [blk*bs, min((blk+1)*bs, lk_b)) whose page is >= 0. With causal, a
 * position is alive iff t <= lk_b - qo_len_b + q_local (or t <= q_local
 * when lk_b < qo_len_b). No alive position gives (0, -inf, 0).
 *   q        float32 [tq, hq, head_dim], q_len elements
 *   k_pages, v_pages float32 [num_pages, hkv, page_size, head_dim], k_len / v_len elements
 * Buffers must hold idx->max_edges * qhead rows.
 * Host checks, in the page's order: HEAD_COUNT; BLOCK_PAGE; SHAPE "idx
 * (hkv or pages_per_block)"; SHAPE "idx (planned hq/head_dim)"; SHAPE "q";
 * SHAPE "k_pages / v_pages page stride" (k_len not a multiple of
 * hkv*page_size*head_dim, or v_len != k_len); SHAPE "k_pages / v_pages pages"
 * (fewer pages than the index was checked against). */
sa_status sa_forward(const sa_index* idx,
                     const float* q, int64_t q_len,
                     const float* k_pages, int64_t k_len,
                     const float* v_pages, int64_t v_len,
                     const int32_t* block_tables, const int64_t* cu_seqlens_q,
                     const int32_t* used_kv_lens,
                     int32_t hq, int32_t hkv, int32_t head_dim,
                     int32_t block_size, int32_t page_size,
                     float softmax_scale, int32_t causal,
                     float* o_partial, float* m_partial, float* l_partial,
                     hipStream_t stream);

/* Storage formats of K/V pages for sa_forward_kv16 and
 * sa_forward_combine_kv16. The pages define fp32 pages only. Where head_dim
 * is 128 and blocks hold at most 128 keys (the one-wave, fused and
 * direct-to-LDS kernels) the 16-bit words are multiplied on the 16-bit
 * matrix cores as stored, with q written as three terms of the format (fp16:
 * after a power-of-two scale of its row) and the probabilities as two;
 * elsewhere each word is converted exactly to fp32. Either way the
 * tolerance is the fp32 path's on the stored values. */
typedef enum sa_kv_format {
  SA_KV_F32 = 0,   /* float32 (sa_forward) */
  SA_KV_BF16 = 1,  /* bfloat16: the top 16 bits of an IEEE binary32 */
  SA_KV_F16 = 2    /* IEEE binary16 */
} sa_kv_format;

/* sa_forward_kv16: sa_forward with K/V pages stored as 16-bit words
 * (`kv_format` SA_KV_BF16 or SA_KV_F16; k_len / v_len count elements, as in
 * sa_forward). Every other argument, the partials written and the host
 * checks (in sa_forward's order) are sa_forward's. Then SA_ERR_UNSUPPORTED
 * "kv_format" for another format. Every geometry that sa_forward takes is
 * supported: each forward kernel converts the words as it loads them. */
sa_status sa_forward_kv16(const sa_index* idx,
                          const float* q, int64_t q_len,
                          const uint16_t* k_pages, int64_t k_len,
                          const uint16_t* v_pages, int64_t v_len,
                          int32_t kv_format,
                          const int32_t* block_tables, const int64_t* cu_seqlens_q,
                          const int32_t* used_kv_lens,
                          int32_t hq, int32_t hkv, int32_t head_dim,
                          int32_t block_size, int32_t page_size,
                          float softmax_scale, int32_t causal,
                          float* o_partial, float* m_partial, float* l_partial,
                          hipStream_t stream);

/* sa_combine: log-sum-exp merge of the partials (the combine pass that
 * forward.rs's module doc describes as the FlashAttention update). For every
 * (q, hq = h*qhead + qh), over ranks r with inv[h,q,r] >= 0 at partial row
 * p = (edge_head_base[h] + inv)*qhead + qh:
 *   M = max m_p;  L = sum l_p exp(m_p - M);  O = sum o_p exp(m_p - M) / L
 *   out float32 [tq, hq, head_dim];  lse float32 [tq, hq] = M + log L, or NULL
 * No rank with finite m gives O = 0, lse = -inf. If the index's build found
 * an input error (sa_index_status), every element of out and lse is NaN. */
sa_status sa_combine(const sa_index* idx,
                     const float* o_partial, const float* m_partial, const float* l_partial,
                     int32_t hq, int32_t head_dim,
                     float* out, float* lse, hipStream_t stream);

/* sa_forward_combine: sa_forward followed by sa_combine in one launch, with
 * no partials in memory (forward.rs module doc: the forward's persistent
 * outer loop and the log-sum-exp combine of its partials). One workgroup per
 * (query, KV head) reads the query's kept blocks (inv >= 0; block ids from
 * `selected`, int32 [tq, hkv, topk], the array the index was built from),
 * merges the blocks' softmax pieces as they come, and writes `out` and `lse`
 * exactly as sa_combine defines them. Meant for batches where each block
 * serves one query (decode: one query per sequence); with shared blocks it is
 * still exact but reads a shared block once per query. Host checks: those of
 * sa_forward, then SHAPE "selected" (selected_len != tq*hkv*topk), then
 * UNSUPPORTED outside head_dim 128, blocks of at most 64 keys, hq/hkv <= 16
 * and topk <= 512. On an index whose build failed, out and lse are NaN.
 * sa_attention takes this path itself when tq == batch and the geometry fits. */
sa_status sa_forward_combine(const sa_index* idx,
                             const int32_t* selected, int64_t selected_len,
                             const float* q, int64_t q_len,
                             const float* k_pages, int64_t k_len,
                             const float* v_pages, int64_t v_len,
                             const int32_t* block_tables, const int64_t* cu_seqlens_q,
                             const int32_t* used_kv_lens,
                             int32_t hq, int32_t hkv, int32_t head_dim,
                             int32_t block_size, int32_t page_size,
                             float softmax_scale, int32_t causal,
                             float* out, float* lse, hipStream_t stream);

/* sa_forward_combine_kv16: sa_forward_combine with K/V pages stored as
 * 16-bit words (`kv_format` SA_KV_BF16 or SA_KV_F16; k_len / v_len count
 * elements), as sa_forward_kv16 takes them. Every other argument, what is
 * written and the host checks are sa_forward_combine's, with UNSUPPORTED
 * "kv_format" for another format after sa_forward's SHAPE checks (its place
 * in sa_forward_kv16). */
sa_status sa_forward_combine_kv16(const sa_index* idx,
                                  const int32_t* selected, int64_t selected_len,
                                  const float* q, int64_t q_len,
                                  const uint16_t* k_pages, int64_t k_len,
                                  const uint16_t* v_pages, int64_t v_len,
                                  int32_t kv_format,
                                  const int32_t* block_tables, const int64_t* cu_seqlens_q,
                                  const int32_t* used_kv_lens,
                                  int32_t hq, int32_t hkv, int32_t head_dim,
                                  int32_t block_size, int32_t page_size,
                                  float softmax_scale, int32_t causal,
                                  float* out, float* lse, hipStream_t stream);

/* sa_attention_workspace_bytes: bytes of the workspace that sa_attention
 * needs: the index buffer plus the worst-case partials, 256-B aligned. */
sa_status sa_attention_workspace_bytes(int64_t tq, int32_t hkv, int32_t topk, int32_t batch,
                                       int32_t max_pages, int32_t block_size,
                                       int32_t page_size, int32_t hq, int32_t head_dim,
                                       size_t* bytes /* host, out */);

/* sa_attention: sa_build_index -> sa_forward -> sa_combine on one stream,
 * with the index and partials inside `workspace`. num_pages is
 * k_len / (hkv*page_size*head_dim). Arguments mean what they mean in the
 * three calls above (build -> sa_forward_combine when tq == batch and its
 * geometry fits). Host checks run before anything is enqueued, in the
 * forward's order and then the build's. `idx_out` (host, may be NULL)
 * receives the index handle, so that sa_index_status() can read the
 * device-side outcome; when the build found an input error, out and lse
 * hold NaN (see sa_combine). */
sa_status sa_attention(const float* q, int64_t q_len,
                       const float* k_pages, int64_t k_len,
                       const float* v_pages, int64_t v_len,
                       const int32_t* selected, int64_t selected_len,
                       const int32_t* block_tables, int64_t block_tables_len,
                       const int64_t* cu_seqlens_q, int64_t cu_len,
                       const int32_t* used_kv_lens, int64_t used_len,
                       int64_t tq, int32_t hq, int32_t hkv, int32_t head_dim, int32_t topk,
                       int32_t batch, int32_t max_pages,
                       int32_t block_size, int32_t page_size,
                       float softmax_scale, int32_t causal,
                       void* workspace, size_t workspace_bytes,
                       float* out, float* lse,
                       sa_index* idx_out, hipStream_t stream);

/* Size of the library's own workspace for sa_attention_noalloc (bytes, per
 * GPU). */
#define SA_NOALLOC_SCRATCH_BYTES (32u << 20)

/* sa_attention_noalloc: sa_attention without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP stream capture,
 * tight serving loops, harnesses that forbid hipMalloc). The index and the
 * partials live in a device array of SA_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends. The first
 * call on a GPU looks the array up there (the runtime then loads it with the
 * library's device code for that GPU); no call allocates anything. Arguments, outputs, host checks (in
 * sa_attention's order) and the device-side error behaviour are
 * sa_attention's. Then SA_ERR_UNSUPPORTED "workspace exceeds the no-alloc
 * scratch" (expected = the limit, got = sa_attention_workspace_bytes) when
 * the problem needs more than the array holds. Every call on one GPU uses
 * the same array and leaves its contents there; calls that overlap on one
 * GPU (several streams or host threads) race, so serialise them. `idx_out`
 * (host, may be NULL) receives the index handle, whose buffer is that array,
 * valid until the next call on the same GPU. */
sa_status sa_attention_noalloc(const float* q, int64_t q_len,
                               const float* k_pages, int64_t k_len,
                               const float* v_pages, int64_t v_len,
                               const int32_t* selected, int64_t selected_len,
                               const int32_t* block_tables, int64_t block_tables_len,
                               const int64_t* cu_seqlens_q, int64_t cu_len,
                               const int32_t* used_kv_lens, int64_t used_len,
                               int64_t tq, int32_t hq, int32_t hkv, int32_t head_dim,
                               int32_t topk, int32_t batch, int32_t max_pages,
                               int32_t block_size, int32_t page_size,
                               float softmax_scale, int32_t causal,
                               float* out, float* lse,
                               sa_index* idx_out, hipStream_t stream);

/* Name of a status code (static string). */
const char* sa_status_string(sa_status status);

/* Detail of the last host-side failure on the calling thread (host out). */
sa_status sa_last_error(sa_error_detail* out);

#ifdef __cplusplus
}
#endif

#endif /* SA_H */
