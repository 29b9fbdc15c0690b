/*
 * fp8idx — fp8 MQA indexer logits + top-k for AMD Instinct MI355X (gfx950).
 *
 * C ABI of the sparse-attention indexer hot path:
 *
 *   logits[i, j] = sum_h weights[i, h] * max(dot(q[i, h, :], kv[j, :]) * kv_scale[j], 0)
 *                  for ks[i] <= j < ke[i]  (-inf elsewhere when `clean` is set)
 *
 * followed by the per-row indices of the k largest logits inside [ks, ke),
 * mapped through a page table.  The operations are the two library calls of
 * the indexer loop on the bench_mqa_logits_chunking.py page
 * (`fp8_mqa_logits(q, (kv, kv_scales), weights, ks, ke, clean_logits)` and
 * `fast_topk_transform_fused(score, lengths, page_table_size_1, cu_seqlens_q,
 * topk, row_starts)`), the paged-decode logits named on the vessl-ai/sglang
 * PR #87 page, and the row-chunked loop of the chunking page that bounds the
 * rows x keys float32 logits buffer by a byte cap.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Shapes: q has H = 32 heads of D = 128 fp8 e4m3fn (OCP "fn" flavour) bytes.
 *   Other H or D return FP8IDX_EUNSUPPORTED.
 * - Pointers: every array pointer is a DEVICE pointer (HIP device memory or
 *   memory the device can read) unless marked "host".  The caller owns all
 *   memory.  The library never allocates, frees or keeps device memory between
 *   calls, and keeps no state that one call leaves for another: scratch
 *   (work-queue counters, top-k candidates, chunk logits) comes only from the
 *   caller's `ws` buffer, whose contents on entry do not matter.
 * - Layouts: row-major, contiguous in the last dimension; leading dimensions
 *   (in elements) are explicit where a buffer may be wider than its content.
 *   q, kv and kv pools must be 16-byte aligned; float and int32 arrays 4-byte
 *   aligned; `ws` 256-byte aligned.
 * - Execution: work is enqueued on `stream` (a hipStream_t; NULL = the legacy
 *   default stream) and the call returns without waiting.  No call allocates,
 *   synchronises the host, or copies host memory to the device, so every entry
 *   point can be captured in a HIP graph.
 * - Errors: arguments are validated on the host before anything is enqueued.
 *   On any status other than FP8IDX_OK nothing was enqueued and no output was
 *   written.  FP8IDX_EHIP means a HIP call failed (the HIP error is reported
 *   by fp8idx_last_hip_error()).
 * - Device-side contents (ks, ke, row lengths, table entries) are not read by
 *   the host.  Kernels clamp them so that no access leaves the buffers the
 *   sizes describe: ke is clamped to the key count, ks to [0, ke], row lengths
 *   to the logits width, and table entries outside their range map to -1 (or,
 *   for kv pages, make the affected keys' logits -inf).  Results for such
 *   out-of-contract inputs are otherwise unspecified.
 * - kv_scale must be >= 0 (quantisation scales); NaN or infinite inputs give
 *   unspecified results.
 * - Determinism: identical inputs give identical output bytes.  Concurrent
 *   calls (on different streams, from different threads, or as replays of
 *   captured graphs) are safe when their outputs and workspaces do not
 *   overlap; a call's workspace must not be used by any other work while the
 *   call's kernels run.
 * - Top-k output: each row holds the selected keys (a set: positions within
 *   the row are not part of the contract; this library writes them in
 *   ascending key order) followed by -1 padding when the row's window holds
 *   fewer than k keys.  A tie at the k-th value is broken toward the lower key
 *   index, so the selected set is unique.
 */
#ifndef FP8IDX_H
#define FP8IDX_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define FP8IDX_API __attribute__((visibility("default")))
#else
#define FP8IDX_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fp8idx_status {
  FP8IDX_OK = 0,
  FP8IDX_EINVAL = 1,       /* null pointer, bad size, stride or alignment */
  FP8IDX_EUNSUPPORTED = 2, /* H != 32, D != 128, k out of range, page size not 64 */
  FP8IDX_EWORKSPACE = 3,   /* ws_bytes smaller than the matching *_workspace_bytes() */
  FP8IDX_EDEVICE = 4,      /* no device, or the current device is not gfx950 */
  FP8IDX_EHIP = 5          /* a HIP launch or query failed */
} fp8idx_status;

/* Index map applied by the top-k stage (the "transform" of the chunking page's
 * fast_topk_transform_fused). */
typedef enum fp8idx_map_kind {
  FP8IDX_MAP_NONE = 0,        /* output the raw key index j */
  FP8IDX_MAP_TOKEN_TABLE = 1, /* page size 1: table[req(i) * ld + (j - ks[i])] */
  FP8IDX_MAP_BLOCK_TABLE = 2  /* table[b * ld + j / page_size] * page_size + j % page_size,
                                 b = i / rows_per_req (paged decode: physical slot id) */
} fp8idx_map_kind;

/* Host struct; the pointers inside are device pointers. */
typedef struct fp8idx_map {
  int32_t kind;            /* fp8idx_map_kind */
  const int32_t* table;    /* [num_req, ld] int32; unused for FP8IDX_MAP_NONE */
  int64_t ld;              /* table row stride in elements (>= 1) */
  int32_t num_req;         /* rows of `table` */
  const int32_t* cu_rows;  /* token table: [num_req + 1] row offsets of each request
                              (like cu_seqlens_q); NULL puts every row in request 0 */
  int32_t rows_per_req;    /* block table: consecutive rows per request (next_n) */
  int32_t page_size;       /* block table: keys per page */
  int64_t num_pages;       /* block table: pages in the pool (>= 1); a page id outside
                              [0, num_pages) maps its keys to -1 */
} fp8idx_map;

/* Operation selector for fp8idx_workspace_bytes(). */
typedef enum fp8idx_op {
  FP8IDX_OP_TOPK = 0,              /* indexer_topk */
  FP8IDX_OP_LOGITS_TOPK_RAGGED = 1, /* indexer_logits_topk_ragged */
  FP8IDX_OP_LOGITS_TOPK_RAGGED_OVERLAP = 2, /* indexer_logits_topk_ragged_overlap */
  FP8IDX_OP_LOGITS_RAGGED = 3      /* indexer_logits_ragged (work-queue counters) */
} fp8idx_op;

/*
 * Ragged-prefill fp8 MQA logits (the chunking page's
 * `fp8_mqa_logits(q, (kv, kv_scales), weights, ks, ke, clean_logits)`).
 *
 *   q        [m, H, D] uint8 e4m3fn      kv       [n, D] uint8 e4m3fn
 *   kv_scale [n] float32 (>= 0)          weights  [m, H] float32
 *   ks, ke   [m] int32: row i's key window is [ks[i], ke[i])
 *   logits   [m, ld_logits] float32 output, ld_logits >= n.  Columns
 *            [0, n) of every row are written when clean != 0 (-inf outside
 *            the window); when clean == 0 only the window is guaranteed and
 *            other columns < n hold unspecified values.  Columns >= n are
 *            never touched.
 *   ws       device scratch of at least fp8idx_workspace_bytes(
 *            FP8IDX_OP_LOGITS_RAGGED, m, n, 1, 0) bytes (256), 256-byte
 *            aligned: the work-queue counters the kernel's workgroups claim
 *            their items from.  The call clears them on `stream` before the
 *            logits kernel, so their contents on entry do not matter; calls
 *            that may run at the same time need distinct `ws` buffers.
 * m == 0 is a no-op (ws may then be NULL).  Requires n >= 1, m >= 0.
 */
FP8IDX_API fp8idx_status indexer_logits_ragged(const uint8_t* q, const uint8_t* kv, const float* kv_scale,
                                    const float* weights, const int32_t* ks, const int32_t* ke,
                                    int32_t m, int32_t n, int32_t H, int32_t D,
                                    float* logits, int64_t ld_logits, int32_t clean,
                                    void* ws, size_t ws_bytes, void* stream);

/*
 * indexer_logits_ragged without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, layouts and
 * results as indexer_logits_ragged, minus ws / ws_bytes.
 * The work-queue counters live in a static device array of the library
 * (256 bytes per device, held until the process ends), cleared on `stream`
 * by each call that needs them; nothing is allocated and no size is too
 * large for it, since the counters do not grow with m or n.  Every call of
 * this entry on one GPU shares that array: calls that may overlap in time
 * on one GPU (different streams, threads, or concurrent graph replays)
 * race and must use indexer_logits_ragged with distinct workspaces.
 */
FP8IDX_API fp8idx_status indexer_logits_ragged_noalloc(const uint8_t* q, const uint8_t* kv, const float* kv_scale,
                                                       const float* weights, const int32_t* ks, const int32_t* ke,
                                                       int32_t m, int32_t n, int32_t H, int32_t D,
                                                       float* logits, int64_t ld_logits, int32_t clean,
                                                       void* stream);

/*
 * Paged-decode fp8 MQA logits (the paged form of the indexer named on the
 * vessl-ai/sglang PR #87 page).  B requests of next_n query rows each; row
 * r = b * next_n + t belongs to request b and sees keys [0, row_len[r]).
 * Key j of request b lives in physical page block_table[b * max_pages + j / page_size],
 * slot j % page_size.  The work split over keys is derived on the device from
 * row_len; nothing is read back to the host.
 *
 *   q           [B, next_n, H, D] uint8     kv_pool    [num_pages, page_size, D] uint8
 *   scale_pool  [num_pages, page_size] f32  weights    [B * next_n, H] float32
 *   row_len     [B * next_n] int32          block_table [B, max_pages] int32
 *   logits      [B * next_n, ld_logits] float32, width <= ld_logits columns
 *               are owned by the call: row r's window [0, min(row_len[r], width))
 *               is written, and with clean != 0 the rest of [0, width) is -inf.
 *               Keys of the window whose page id lies outside [0, num_pages)
 *               get -inf whatever `clean` says.
 * page_size must be 64.
 */
FP8IDX_API fp8idx_status indexer_logits_paged(const uint8_t* q, const uint8_t* kv_pool,
                                   const float* scale_pool, const float* weights,
                                   const int32_t* row_len, const int32_t* block_table,
                                   int32_t B, int32_t next_n, int32_t H, int32_t D,
                                   int32_t page_size, int32_t max_pages, int64_t num_pages,
                                   float* logits, int64_t ld_logits, int32_t width,
                                   int32_t clean, void* stream);

/*
 * Per-row top-k over float32 logits with the index map (the chunking page's
 * `fast_topk_transform_fused(score, lengths=ke, page_table, cu_seqlens_q, topk,
 * row_starts=ks)`).
 *
 *   logits [rows, ld] float32; row i's candidates are columns [ks[i], ke[i])
 *          (ks NULL means 0; ke is clamped to `width` <= ld)
 *   row0   global id of logits row 0, used by the map (request lookup)
 *   map    host pointer; NULL means FP8IDX_MAP_NONE.  For the token table
 *          ks must be indexed like the logits rows.
 *   out    [rows, ld_out] int32, ld_out >= k: columns [0, k) are written
 *   ws     device scratch of at least fp8idx_workspace_bytes(FP8IDX_OP_TOPK,
 *          rows, width, k, 0) bytes (rows longer than one selection segment,
 *          or few rows, are split into segments whose candidates live there;
 *          the size may be 0, and ws may then be NULL)
 * 1 <= k <= 16384.  Rows so long that the candidate merge would need more
 * than 8 selection levels (width above about 2^30 at k = 16384) return
 * FP8IDX_EUNSUPPORTED.
 */
FP8IDX_API fp8idx_status indexer_topk(const float* logits, int64_t ld, int32_t rows, int32_t width,
                           const int32_t* ks, const int32_t* ke, int32_t k, int32_t row0,
                           const fp8idx_map* map, int32_t* out, int64_t ld_out,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * Fused ragged logits + top-k under a logits byte cap (the row-chunked loop
 * of the chunking page: at most fp8idx_rows_per_chunk rows per chunk, i.e.
 * max(1, floor(cap / (n * 4)))).  The rows are spread evenly over that many
 * chunks, ceil(m / fp8idx_rows_per_chunk), so the last one is not short.  Per
 * chunk: logits into the workspace, then top-k into `out`, on one stream.
 * The full rows x n buffer is never materialised unless the cap allows it.
 *
 *   logits_cap_bytes   0 = one chunk holding every row
 *   ws, ws_bytes       >= fp8idx_workspace_bytes(FP8IDX_OP_LOGITS_TOPK_RAGGED,
 *                        m, n, k, logits_cap_bytes)
 * The workspace holds the logits kernel's work-queue counters (first 256
 * bytes), one chunk of logits and the top-k candidates.
 * Other arguments as indexer_logits_ragged and indexer_topk (row0 = 0).
 */
FP8IDX_API fp8idx_status indexer_logits_topk_ragged(const uint8_t* q, const uint8_t* kv,
                                         const float* kv_scale, const float* weights,
                                         const int32_t* ks, const int32_t* ke,
                                         int32_t m, int32_t n, int32_t H, int32_t D,
                                         int32_t k, const fp8idx_map* map,
                                         int32_t* out, int64_t ld_out,
                                         size_t logits_cap_bytes, void* ws, size_t ws_bytes,
                                         void* stream);

/*
 * The same row-chunked loop with the top-k of chunk N - 1 running on
 * `side_stream` while the logits of chunk N run on `stream` (the chunking
 * page's `_run_chunked_pipelined`, which asks whether small chunks cost
 * through serialisation or through small-M inefficiency).  Two chunk logits
 * buffers alternate in the workspace; device events order each buffer's
 * writes, its top-k read and its reuse, and `stream` waits for the last
 * top-k before the call returns, so work enqueued on `stream` afterwards
 * sees every output.  Output is identical to indexer_logits_topk_ragged.
 *
 *   side_stream   a stream other than `stream` (else FP8IDX_EINVAL)
 *   ws_bytes      >= fp8idx_workspace_bytes(FP8IDX_OP_LOGITS_TOPK_RAGGED_OVERLAP,
 *                    m, n, k, logits_cap_bytes)
 * The ordering uses four events that the call creates (without timing) and
 * destroys before it returns; a wait enqueued on a stream keeps the state
 * the event had when the wait was enqueued, so nothing outlives the call and
 * concurrent calls share nothing.  Stream capture works as a fork (the side
 * stream joins through the first event) and a join (the final wait).
 */
FP8IDX_API fp8idx_status indexer_logits_topk_ragged_overlap(const uint8_t* q, const uint8_t* kv,
                                                 const float* kv_scale, const float* weights,
                                                 const int32_t* ks, const int32_t* ke,
                                                 int32_t m, int32_t n, int32_t H, int32_t D,
                                                 int32_t k, const fp8idx_map* map,
                                                 int32_t* out, int64_t ld_out,
                                                 size_t logits_cap_bytes, void* ws, size_t ws_bytes,
                                                 void* stream, void* side_stream);

/*
 * Fused paged logits + top-k.  Output indices are physical kv slots
 * (block_table[b, j / 64] * 64 + j % 64) when map_to_slots != 0, else raw key
 * positions j.  `width` bounds every row length (the logits row stride used in
 * the workspace).  Requests are chunked so that at most logits_cap_bytes of
 * logits exist at once (0 = all rows at once), spread evenly over the chunks.
 *   ws_bytes >= fp8idx_workspace_bytes_paged(B, next_n, width, k, logits_cap_bytes)
 * Chunks hold whole requests: at least one request per chunk even when one
 * request's next_n rows exceed the cap.  When a chunk's top-k takes one
 * workgroup per row (at most 512 rows of at most 131072 keys, k up to about
 * 2300), the logits kernel also writes each row's largest logit per 16-key
 * fragment into the workspace (one word per fragment of the width, rounded up
 * to whole 1024-key blocks, per row slot: min(4, next_n) slots per group of 4
 * rows; fp8idx_workspace_bytes_paged includes them), and the top-k
 * takes its threshold from those maxima: the kk-th largest of them is at most
 * the row's kk-th largest logit, and only fragments that reach it are read.
 * The result is the same exact selection either way.
 */
FP8IDX_API fp8idx_status indexer_logits_topk_paged(const uint8_t* q, const uint8_t* kv_pool,
                                        const float* scale_pool, const float* weights,
                                        const int32_t* row_len, const int32_t* block_table,
                                        int32_t B, int32_t next_n, int32_t H, int32_t D,
                                        int32_t page_size, int32_t max_pages, int64_t num_pages,
                                        int32_t width, int32_t k, int32_t map_to_slots,
                                        int32_t* out, int64_t ld_out,
                                        size_t logits_cap_bytes, void* ws, size_t ws_bytes,
                                        void* stream);

/*
 * Per-row fp8 e4m3fn quantisation (the `act_quant` step named on the
 * vessl-ai/sglang PR #87 page, which also pins its encoder: nearest with
 * ties to even, subnormals, saturation to +-448).  It produces this path's
 * fp8 inputs: kv codes with the per-token kv_scale, or q codes (one row per
 * query row and head).  For each row r:
 *
 *   amax     = max_d |x[r, d]|   (a row of zeros takes amax = 448)
 *   codes[r, d] = e4m3fn(float32(x[r, d] * float32(448 / amax)))
 *   scale[r] = float32(amax / 448)            so x ~ decode(code) * scale
 *
 *   x      [rows, ld_x] float32, ld_x >= D, ld_x % 4 == 0, 16-byte aligned
 *   codes  [rows, ld_codes] uint8 output, ld_codes >= D, ld_codes % 4 == 0,
 *          4-byte aligned; columns [0, D) are written
 *   scale  [rows] float32 output
 * 4 <= D <= 2048 with D % 4 == 0 (else FP8IDX_EUNSUPPORTED).  Inputs must be
 * finite, with every nonzero row's amax at least 2^-100.  rows == 0 is a
 * no-op.  Allocates nothing; runs on `stream`.
 */
FP8IDX_API fp8idx_status indexer_quant_fp8(const float* x, int64_t ld_x, int64_t rows, int32_t D,
                                           uint8_t* codes, int64_t ld_codes, float* scale, void* stream);

/*
 * Ragged prefill index preparation (the `gen_nsa_ks_ke` step on the lightllm
 * "parallel NSA ragged index copies" PR page).  Request b holds seq_len[b]
 * tokens whose last q_len[b] are this step's queries (q_len clamped to
 * [0, seq_len]); the keys of all requests lie back to back in the ragged key
 * space, request b's first at cu_seq[b]:
 *
 *   cu_seq [B+1], cu_q [B+1] int32   prefix sums of seq_len and q_len
 *   ks, ke [max_q] int32             query t of request b, at cu_q[b] + t, sees ragged
 *                                    keys [cu_seq[b], cu_seq[b] + seq_len[b] - q_len[b] + t + 1)
 *   ragged_mem [max_keys] int32      ragged key cu_seq[b] + p -> table[req_idx[b], p], the
 *                                    kv slot (-1 past the table row or for an out-of-range
 *                                    req_idx); NULL skips the copy
 *   table [num_table_rows, ld_table] int32, the request -> token-slot table
 *
 * ks/ke and ragged_mem are written up to the totals or the capacities
 * (max_q, max_keys), whichever is smaller; nothing past the totals is
 * touched.  The totals must stay below 2^31.  B <= 4096 (else
 * FP8IDX_EUNSUPPORTED); B == 0 is a no-op.  One launch, no host
 * synchronisation, graph capturable.  Allocates nothing.
 */
FP8IDX_API fp8idx_status indexer_prepare_ragged(const int32_t* seq_len, const int32_t* q_len,
                                                const int32_t* req_idx, const int32_t* table,
                                                int64_t ld_table, int32_t num_table_rows, int32_t B,
                                                int32_t* cu_seq, int32_t* cu_q, int32_t* ks, int32_t* ke,
                                                int64_t max_q, int32_t* ragged_mem, int64_t max_keys,
                                                void* stream);

/*
 * Paged decode / MTP index preparation.  Request b's next_n query rows are
 * its last next_n tokens:
 *   row_len [B * next_n] int32       row t of request b sees keys
 *                                    [0, max(0, seq_len[b] - next_n + t + 1))
 *   block_table [B, max_pages] int32 row b = req_to_page[req_idx[b], 0:max_pages]
 *                                    (-1 for an out-of-range req_idx)
 *   req_to_page [num_table_rows, ld_req_to_page] int32, ld_req_to_page >= max_pages
 * The outputs feed indexer_logits_paged / indexer_logits_topk_paged.
 */
FP8IDX_API fp8idx_status indexer_prepare_decode(const int32_t* seq_len, const int32_t* req_idx,
                                                const int32_t* req_to_page, int64_t ld_req_to_page,
                                                int32_t num_table_rows, int32_t B, int32_t next_n,
                                                int32_t* row_len, int32_t* block_table, int32_t max_pages,
                                                void* stream);

/*
 * Sparse MLA attention over the top-k slots: the step after the indexer on
 * the vessl-ai/sglang PR #87 page (sparse MLA prefill / decode kernels over an
 * MLA KV pool kept in fp8 e4m3 and widened to bf16 inside the kernel, with
 * few-token decode run as split-K partials plus a combine).  The page does
 * not write the attention out; this is softmax attention of every query
 * token over the pool rows its top-k list selects.  For token t, head h and
 * the valid slots j of indices[t, 0:topk] (0 <= j < num_slots; other entries,
 * such as the -1 padding of the top-k output, are skipped, and a repeated
 * slot counts each time):
 *
 *   s_j     = sm_scale * dot(q[t, h, :], kv_scale[j] * e4m3(kv[j, :]))   (all 576 values)
 *   out[t, h, :] = sum_j softmax(s)_j * kv_scale[j] * e4m3(kv[j, 0:512])  (the latent values)
 *   lse[t, h]    = log sum_j exp(s_j)
 *
 * A token with no valid slot gets out = 0 and lse = -inf.
 *   q        [T, H, 576] bf16 (uint16 bit patterns), 16-byte aligned
 *   kv       [num_slots, 576] e4m3fn codes, 16-byte aligned; num_slots >= 1
 *   kv_scale [num_slots] float32, kv_scale >= 0 (the value weights fold it in)
 *   indices  [T, ld_indices] int32 slot ids, ld_indices >= topk
 *   out      [T, H, 512] float32 output, 16-byte aligned
 *   lse      [T, H] float32 output, or NULL
 *   ws       fp8idx_sparse_mla_workspace_bytes(T, H, topk) bytes of device
 *            scratch, 256-byte aligned (NULL allowed when that is 0)
 * D must be 576, Dv 512 and H a multiple of 16 (else FP8IDX_EUNSUPPORTED);
 * 1 <= topk.  q is rounded nowhere: the scores use its bf16 values, the fp8
 * rows widened exactly, and fp32 accumulation; the probabilities enter the
 * value product in bf16.  T == 0 is a no-op.  Allocates nothing; runs on
 * `stream`.
 */
FP8IDX_API fp8idx_status indexer_sparse_mla(const uint16_t* q, const uint8_t* kv, const float* kv_scale,
                                            int64_t num_slots, const int32_t* indices, int64_t ld_indices,
                                            int32_t T, int32_t H, int32_t D, int32_t Dv, int32_t topk,
                                            float sm_scale, float* out, float* lse, void* ws, size_t ws_bytes,
                                            void* stream);

/* Entry points whose arguments fp8idx_validate_only() checks. */
typedef enum fp8idx_entry {
  FP8IDX_ENTRY_LOGITS_RAGGED = 0,             /* indexer_logits_ragged */
  FP8IDX_ENTRY_LOGITS_PAGED = 1,              /* indexer_logits_paged */
  FP8IDX_ENTRY_TOPK = 2,                      /* indexer_topk */
  FP8IDX_ENTRY_LOGITS_TOPK_RAGGED = 3,        /* indexer_logits_topk_ragged */
  FP8IDX_ENTRY_LOGITS_TOPK_RAGGED_OVERLAP = 4, /* indexer_logits_topk_ragged_overlap */
  FP8IDX_ENTRY_LOGITS_TOPK_PAGED = 5          /* indexer_logits_topk_paged */
} fp8idx_entry;

/* The arguments of one call of an indexer entry point, field for field under
 * the parameter names of the declarations above (indexer_topk's `logits`
 * input is `scores` here, its `ld` is `ld_logits`).  Fields the entry does not
 * take are ignored.  Host struct; pointers are only compared with NULL and
 * tested for alignment, never dereferenced. */
typedef struct fp8idx_call_args {
  const uint8_t* q;
  const uint8_t* kv;            /* kv, or kv_pool for the paged entries */
  const float* kv_scale;        /* kv_scale, or scale_pool for the paged entries */
  const float* weights;
  const int32_t* ks;
  const int32_t* ke;
  const int32_t* row_len;
  const int32_t* block_table;
  int32_t m, n, H, D;
  int32_t B, next_n, page_size, max_pages;
  int64_t num_pages;
  int32_t width;
  float* logits;                /* output of the logits entries */
  const float* scores;          /* input of indexer_topk */
  int64_t ld_logits;
  int32_t clean;
  int32_t rows, k, row0, map_to_slots;
  const fp8idx_map* map;
  int32_t* out;
  int64_t ld_out;
  size_t logits_cap_bytes;
  void* ws;
  size_t ws_bytes;
  void* stream;
  void* side_stream;
} fp8idx_call_args;

/*
 * Host-only argument check: the status `entry` would return for `args`
 * before it looks for a device, i.e. every FP8IDX_EINVAL, FP8IDX_EUNSUPPORTED
 * and FP8IDX_EWORKSPACE case, and FP8IDX_OK when the call would go on to the
 * device.  The entry points run this same check first.  Touches no device
 * and needs none (for tests and for callers that vet a configuration on a
 * host without a GPU).  A NULL args or an unknown entry gives FP8IDX_EINVAL.
 */
FP8IDX_API fp8idx_status fp8idx_validate_only(int32_t entry, const fp8idx_call_args* args);

/* Bytes of workspace indexer_sparse_mla needs (0 when it runs without
 * splitting the top-k lists).  Pure host arithmetic. */
FP8IDX_API size_t fp8idx_sparse_mla_workspace_bytes(int32_t T, int32_t H, int32_t topk);

/* Bytes of device workspace an operation needs (0 when it needs none, or
 * for arguments the operation rejects).  rows = logits rows (m or
 * B * next_n), width = keys per row (n or the paged width); k is ignored for
 * FP8IDX_OP_LOGITS_RAGGED.  Pure host arithmetic. */
FP8IDX_API size_t fp8idx_workspace_bytes(int32_t op, int32_t rows, int64_t width, int32_t k,
                              size_t logits_cap_bytes);

/* Bytes of workspace indexer_logits_topk_paged needs.  Pure host arithmetic.
 * Returns 0 for arguments the entry rejects (B or next_n < 1, width < 0, k
 * outside [1, 16384], B * next_n past INT32_MAX). */
FP8IDX_API size_t fp8idx_workspace_bytes_paged(int32_t B, int32_t next_n, int32_t width, int32_t k,
                                    size_t logits_cap_bytes);

/* Largest chunk of the fused ragged entry: max(1, floor(cap / (ld * 4))),
 * capped at rows, where ld = width rounded up to a multiple of 4 (the row
 * stride of the workspace logits); cap 0 gives rows.  The entry runs
 * ceil(rows / this) chunks of ceil(rows / chunks) rows (the last one takes the
 * remainder).  Pure host arithmetic. */
FP8IDX_API int32_t fp8idx_rows_per_chunk(size_t logits_cap_bytes, int64_t width, int32_t rows);

/*
 * Measurement helper, not a step of the indexer: a sustained fp8 MFMA
 * throughput probe, the measured peak that the logits kernel's MFMA rate is
 * reported against next to the published dense fp8 figure.  Launches
 * `blocks` workgroups of 256 threads; each wave issues iters x 4
 * back-to-back v_mfma_f32_16x16x128_f8f6f4 on four independent accumulators
 * with register operands.  out: device float32 [blocks * 256], written (one
 * value per thread, which keeps the work live; its value means nothing).
 * *flops (if non-NULL) receives the flops of the launch:
 * blocks * 4 waves * iters * 4 * 65536.  blocks > 0 and iters > 0, else
 * FP8IDX_EINVAL.  Allocates nothing; runs on `stream`; the caller times it.
 */
FP8IDX_API fp8idx_status fp8idx_probe_mfma_fp8(int32_t blocks, int32_t iters, float* out, double* flops,
                                               void* stream);

/*
 * Measurement helper, not a step of the indexer: the logits kernels' per-fragment
 * core without memory traffic.  Launches `blocks` workgroups of 256 threads;
 * each wave runs iters x one 16-key fragment of the logits core (eight
 * v_mfma_f32_16x16x128_f8f6f4 for 4 query rows x 32 heads, then ReLU, the head
 * weights and the cross-lane head reduction, the same code as the logits
 * kernels) on register operands.  With as many workgroups per CU as the ragged
 * logits kernel keeps resident, its rate is the issue-bound ceiling of that
 * kernel.  out: device float32 [blocks * 256], written (keeps the work live;
 * its value means nothing).  *flops (if non-NULL) receives blocks * 4 waves *
 * iters * 8 * 65536.  blocks > 0 and iters > 0, else FP8IDX_EINVAL.
 * Allocates nothing; runs on `stream`; the caller times it.
 */
FP8IDX_API fp8idx_status fp8idx_probe_logits_core(int32_t blocks, int32_t iters, float* out, double* flops,
                                                  void* stream);

/* Static string naming a status. */
FP8IDX_API const char* fp8idx_status_string(int32_t status);

/* The hipError_t of the last FP8IDX_EHIP returned on this thread (0 if none). */
FP8IDX_API int32_t fp8idx_last_hip_error(void);

/* Library version, e.g. "fp8idx 0.1.0 gfx950". */
FP8IDX_API const char* fp8idx_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8IDX_H */
