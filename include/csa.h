/*
 * csa.h - C ABI of the CSA / HCA compressed-attention library for MI355X
 * (gfx950).
 *
 * The calls follow the method described on the page "DeepSeek V4 深度解析"
 * (section 2, "核心技術創新": the three CSA steps and the HCA paragraph) and
 * the page at wmrh.cn/news/726125 ("V4 改进一", and the FP4 paragraph):
 *
 *   csa_kv_compress      CSA step 1: every m raw tokens' KV -> one entry,
 *                        softmax weights from per-token logits plus per-slot
 *                        position biases over an overlapping window.
 *   csa_indexer_score    CSA step 2: low-rank lightning-indexer scores of each
 *                        query against the visible entries (BF16 scores).
 *   csa_topk_select      CSA step 2: the top-k entries of each query.
 *   csa_indexer_topk     the two together, without writing the scores.
 *   csa_sparse_mqa_attn  CSA step 3 / HCA: shared-KV multi-query attention over
 *                        the selected (CSA) or all visible (HCA) entries
 *                        together with the sliding window of raw tokens.
 *   csa_swa_merge        the exact log-sum-exp combination of two partial
 *                        attentions, so the window branch and the compressed
 *                        branch can run separately.
 *   csa_kv_compress_append
 *                        decode-time compression through a per-request state
 *                        (page "DeepSeek V4 深度解析", section 4, KV-cache
 *                        management): one token per request and call.
 *   csa_quantize, csa_dequantize, csa_mxfp4_to_fp8
 *                        the storage formats: mixed-precision KV entries
 *                        (RoPE dims BF16, the rest FP8) and the FP4 indexer
 *                        operands with their lossless FP4 -> FP8 regrouping.
 *
 * Conventions
 *  - Every pointer passed to a compute call is a DEVICE pointer unless stated,
 *    and the structs themselves (csa_tensor, csa_batch) live in host memory.
 *  - Calls are stream ordered and asynchronous: they enqueue kernels on
 *    `stream` and return.  The library never synchronises the host, never
 *    allocates device memory and keeps no pointer after a call returns.  The
 *    caller owns every buffer.
 *  - Arguments are validated on the host before anything is launched; on any
 *    error nothing is enqueued and the call returns a non-zero csa_status.
 *    csa_last_error() gives a thread-local description.  Device-resident
 *    metadata (offsets, positions, top-k indices) cannot be checked on the
 *    host: kernels clamp every such value to the extents of the tensors they
 *    were given, so bad metadata gives wrong results but never an
 *    out-of-bounds access.
 *  - Results are deterministic: the same inputs give the same bits, and a
 *    request's results do not depend on its position in the batch or on the
 *    other requests (no atomics in value reductions).
 *  - Layouts are dense and row major.
 *
 * Readings where the pages are silent (fixed here; see the individual calls):
 *  - entry i covers raw positions (i+1)m-w .. (i+1)m-1; slots before position 0
 *    are left out of the softmax;
 *  - entry i is visible to the query at position t iff (i+1)m-1 <= t, i.e.
 *    n_c(t) = floor((t+1)/m) entries;
 *  - the window of the query at t is positions max(0, t-W+1) .. t;
 *  - one softmax over the union of entries and window tokens, key = value.
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 5

typedef enum csa_status {
  CSA_OK = 0,
  CSA_ERR_INVALID_ARGUMENT = 1, /* a null pointer, bad size or bad format      */
  CSA_ERR_UNSUPPORTED = 2,      /* valid but not implemented (e.g. a dim)       */
  CSA_ERR_WORKSPACE = 3,        /* workspace missing or too small               */
  CSA_ERR_HIP = 4               /* a HIP launch failed; see csa_last_error()    */
} csa_status;

typedef enum csa_format {
  CSA_F32 = 0,       /* float32                                                */
  CSA_BF16 = 1,      /* bfloat16 bit patterns (uint16)                          */
  CSA_FP8_MIXED = 2, /* 512-dim KV entry: [448 e4m3fn | 64 bf16] with 4 e8m0
                        scales for the e4m3 blocks [0,128) [128,256) [256,384)
                        [384,448); scale = smallest 2^e with amax <= 448*2^e    */
  CSA_MXFP4 = 3      /* OCP MX: e2m1 elements, two per byte (element 2i in the
                        low nibble of byte i), one e8m0 scale per 32 elements,
                        X = 2^(floor(log2 amax) - 2), saturating to +-6          */
} csa_format;

/* A matrix of `rows` vectors of `dim` logical elements (device memory).
 *   CSA_F32      data  = float   [rows][dim]
 *   CSA_BF16     data  = uint16  [rows][dim]
 *   CSA_FP8_MIXED dim = 512;  data = uint8 e4m3fn [rows][448],
 *                scale = uint8 e8m0 [rows][4],  rope = uint16 bf16 [rows][64]
 *   CSA_MXFP4    data  = uint8 [rows][dim/2],   scale = uint8 e8m0 [rows][dim/32]
 * Unused pointers must be NULL. */
typedef struct csa_tensor {
  int32_t fmt;
  int32_t dim;
  int64_t rows;
  void* data;
  void* scale;
  void* rope;
} csa_tensor;

/* A batch of requests (host struct; the arrays are DEVICE memory, int64).
 *   queries of request r      : rows q_off[r] .. q_off[r+1]-1 of the query
 *                               tensors; query i of r sits at position
 *                               q_pos[r] + i
 *   compressed entries of r   : rows kv_off[r] .. kv_off[r+1]-1 of the entry
 *                               (and indexer-key) tensor; local entry j is row
 *                               kv_off[r] + j
 *   raw (window) rows of r    : rows raw_off[r] .. raw_off[r+1]-1 of the raw
 *                               tensor, holding positions raw_pos[r] ..
 *                               (may be NULL when no window is used)
 *   window_ring               : 0: the raw rows of r hold positions raw_pos[r],
 *                               raw_pos[r] + 1, ... in order.  1: they are a
 *                               ring of C = raw_off[r+1]-raw_off[r] rows,
 *                               position p at row raw_off[r] + p mod C,
 *                               holding the positions from raw_pos[r] up to
 *                               the request's last query, at most C of them
 *                               (as csa_kv_compress_append writes them); C
 *                               must be at least the window plus the
 *                               request's queries minus one
 *   kv_block_table            : NULL, or the paged compressed cache (page
 *                               "DeepSeek V4 深度解析", section 4, KV-cache
 *                               management: compressed entries kept in blocks
 *                               that each cover LCM of the compression ratios
 *                               raw tokens, i.e. 128 raw tokens = 32 CSA
 *                               entries or 1 HCA entry).  int32 DEVICE array
 *                               [n_req][kv_block_stride] of block ids; entry j
 *                               of r is row table[r*stride + j/P]*P + j%P of
 *                               the entry and indexer-key tensors, with P =
 *                               kv_block_rows (a power of two, 1 .. 2^20).
 *                               kv_off[r+1]-kv_off[r] still counts r's entries
 *                               (at most stride*P are used).  A block id whose
 *                               rows fall outside a tensor reads row 0 there
 *                               (reads stay in bounds; that entry's value is
 *                               unspecified).
 * n_q = q_off[n_req] and max_kv >= every kv_off[r+1]-kv_off[r] are host-side
 * copies used to size launch grids. */
typedef struct csa_batch {
  int32_t n_req;
  int32_t window_ring;
  int64_t n_q;
  int64_t max_kv;
  const int64_t* q_off;
  const int64_t* q_pos;
  const int64_t* kv_off;
  const int64_t* raw_off;
  const int64_t* raw_pos;
  const int32_t* kv_block_table;
  int64_t kv_block_stride;
  int32_t kv_block_rows;
  int32_t reserved;
} csa_batch;

/* ---------------------------------------------------------------------------
 * csa_kv_compress - CSA step 1 (and HCA at m' = 128).
 * Page "DeepSeek V4 深度解析", section 2, CSA step 1: m raw tokens -> one entry
 * by a softmax-weighted sum with one learned weight per raw token plus a
 * position bias, adjacent blocks overlapping.
 *
 * Computes entries entry_begin .. entry_begin+n_entries-1 of one sequence into
 * rows 0 .. n_entries-1 of `out`.  Entry i, slot s in [0, w): p = (i+1)m-w+s;
 * slots with p < 0 are dropped; weights = softmax over the valid slots of
 * logits[p - x_pos0] + slot_bias[s] (fp32); entry = sum weight_s * x[p - x_pos0]
 * accumulated in fp32, then stored as F32, BF16 (round to nearest-even) or
 * FP8_MIXED (dim 512).
 *   x          raw rows, F32 or BF16, positions x_pos0 .. x_pos0 + x->rows - 1;
 *              must hold every valid slot of the requested entries
 *   logits     float [x->rows], aligned with x
 *   slot_bias  float [w]
 *   1 <= m <= w <= 1024; out->rows >= n_entries; out->dim == x->dim
 * ------------------------------------------------------------------------- */
csa_status csa_kv_compress(const csa_tensor* x, const float* logits, int64_t x_pos0,
                           const float* slot_bias, int32_t m, int32_t w,
                           int64_t entry_begin, int64_t n_entries, const csa_tensor* out,
                           hipStream_t stream);

/* ---------------------------------------------------------------------------
 * csa_kv_compress_paged - csa_kv_compress into a paged compressed cache (page
 * "DeepSeek V4 深度解析", section 4, KV-cache management: entries kept in
 * blocks of LCM(compression ratios) raw tokens; see csa_batch.kv_block_table).
 *
 * As csa_kv_compress, except that entry j (entry_begin <= j < entry_begin +
 * n_entries, counted from the request's first entry) goes to row
 * blocks[j / block_rows] * block_rows + j % block_rows of `out`, the cache's
 * block pool:
 *   blocks      device int32, the request's block ids in order (at least
 *               (entry_begin + n_entries + block_rows - 1) / block_rows of them)
 *   block_rows  entries per block, a power of two in [1, 2^20]
 * An entry whose block id is negative or whose row falls outside `out` is not
 * written.  out->rows is the pool's size (no relation to n_entries).
 * ------------------------------------------------------------------------- */
csa_status csa_kv_compress_paged(const csa_tensor* x, const float* logits, int64_t x_pos0,
                                 const float* slot_bias, int32_t m, int32_t w,
                                 int64_t entry_begin, int64_t n_entries, const int32_t* blocks,
                                 int32_t block_rows, const csa_tensor* out, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * csa_kv_compress_batch - csa_kv_compress for a batch of prefill chunks in one
 * launch (page "DeepSeek V4 深度解析", section 2, CSA step 1, applied to every
 * request of a ragged batch).
 *
 * For each request r of `batch`: its chunk covers positions q_pos[r] ..
 * q_pos[r] + T_r - 1, T_r = q_off[r+1] - q_off[r], and completes entries
 * floor(q_pos[r] / m) .. floor((q_pos[r] + T_r) / m) - 1 (an entry is
 * complete once its last raw token, position (i+1)m - 1, is in).  Each is
 * computed as csa_kv_compress computes entry i, from r's raw rows x[raw_off[r]
 * .. raw_off[r+1]) at positions raw_pos[r] .. (logits aligned with x), and
 * written to r's cache row kv_off[r] + i, or through batch->kv_block_table
 * when it is set (row table[r*stride + i/P]*P + i%P).
 *   x, logits  raw rows of all requests (F32 or BF16) and their logits
 *   slot_bias  float [w]; 1 <= m <= w <= 1024
 *   batch      q_off, q_pos, kv_off, raw_off, raw_pos (device); window_ring 0
 *   out        the entry tensor (F32, BF16 or FP8_MIXED at dim 512)
 * Each chunk's raw rows must start at position (floor(q_pos[r] / m) + 1) m - w
 * (the first slot of its first new entry) or at 0: a slot at a position >= 0
 * outside r's raw rows is left out of that entry's softmax, as a slot at a
 * negative position is.
 * An entry past r's cache rows (i >= kv_off[r+1] - kv_off[r]) or whose block
 * id is negative or out of the tensor is not written.  Sizes and formats are
 * checked on the host; offsets are read on the device.
 * ------------------------------------------------------------------------- */
csa_status csa_kv_compress_batch(const csa_tensor* x, const float* logits, const float* slot_bias,
                                 int32_t m, int32_t w, const csa_batch* batch, const csa_tensor* out,
                                 hipStream_t stream);

/* ---------------------------------------------------------------------------
 * csa_kv_compress_channel - CSA step 1 with a learned weight per raw token and
 * channel.  Page "DeepSeek V4 深度解析", section 2, CSA step 1, read with one
 * compression logit per token and channel (and a position bias per slot and
 * channel) instead of one per token: each channel has its own softmax.
 *
 * As csa_kv_compress, except:
 *   logits     float [x->rows][dim], aligned with x
 *   slot_bias  float [w][dim]
 * Entry i, channel d: weights = softmax over the valid slots s of
 * logits[p - x_pos0][d] + slot_bias[s][d]; channel d of the entry = sum of
 * weight * x[p - x_pos0][d], fp32, stored as F32, BF16 or FP8_MIXED (dim 512).
 * ------------------------------------------------------------------------- */
csa_status csa_kv_compress_channel(const csa_tensor* x, const float* logits, int64_t x_pos0,
                                   const float* slot_bias, int32_t m, int32_t w,
                                   int64_t entry_begin, int64_t n_entries,
                                   const csa_tensor* out, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * csa_kv_compress_append - decode-time compression through a state cache.
 * Page "DeepSeek V4 深度解析", section 4, the paragraph on KV-cache management
 * for the hybrid attention: a fixed per-request state holds the window and the
 * tail of tokens not yet compressed, finished entries go to the compressed
 * cache.  The entries are those of csa_kv_compress (same reading: entry i
 * covers positions (i+1)m-w .. (i+1)m-1, slots before 0 left out), computed
 * one token at a time.
 *
 * Appends one raw token to each of the n_req = x->rows requests:
 *   x          [n_req, dim] F32 or BF16, request r's new raw row, at position
 *              pos[r] (device int64; a negative position skips the request)
 *   logits     float [n_req], its compression logit; slot_bias float [w]
 *   1 <= m <= w <= 2m (so a token lies in at most two entries' windows), w <= 1024
 *   state      device float, csa_kv_append_state_size(n_req, dim) bytes,
 *              owned by the caller: per request the two open entries (online
 *              softmax: running max, sum and weighted row, fp32).  An entry's
 *              accumulator is reset at the first valid position of its window,
 *              so no initialisation is needed when a request's tokens are
 *              appended in order from a window start (position 0, or the first
 *              position of the oldest entry still open after a prefill);
 *              replaying such a tail re-emits the entries it completes
 *   entry_off  device int64 [n_req]: entry i of request r goes to row
 *              entry_off[r] + i of `cache` when position (i+1)m-1 is appended
 *              (rows outside the cache are skipped); ignored (may be NULL)
 *              when block_table is given
 *   block_table  NULL, or the paged compressed cache (as csa_batch's
 *              kv_block_table): device int32 [n_req][block_stride] block ids,
 *              entry i of request r goes to row table[r*block_stride + i/P]*P
 *              + i%P with P = block_rows (a power of two, 1 .. 2^20); an entry
 *              past the request's slots, a negative block id or a row outside
 *              the cache is not written
 *   cache      F32, BF16 or FP8_MIXED (dim 512) entries of dim = x->dim, dim in
 *              {64, 128, 256, 512}
 *   window     NULL, or F32 / BF16 rows of dim: the raw row also goes to row
 *              window_off[r] + pos[r] mod window_rows (a ring of window_rows
 *              rows per request, read by csa_sparse_mqa_attn with
 *              csa_batch.window_ring = 1)
 * Requests must be distinct (each owns its state and rows); calls on one
 * stream see each other's writes in order.
 * ------------------------------------------------------------------------- */
size_t csa_kv_append_state_size(int64_t n_req, int32_t dim);
csa_status csa_kv_compress_append(const csa_tensor* x, const float* logits,
                                  const float* slot_bias, int32_t m, int32_t w,
                                  const int64_t* pos, float* state, const int64_t* entry_off,
                                  const int32_t* block_table, int64_t block_stride,
                                  int32_t block_rows, const csa_tensor* cache,
                                  const csa_tensor* window, const int64_t* window_off,
                                  int32_t window_rows, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * csa_indexer_score - CSA step 2, the lightning indexer.
 * Page "DeepSeek V4 深度解析", section 2, CSA step 2 (a light low-rank
 * relevance score per query and compressed entry) and the FP4 paragraph
 * (indexer QK in FP4; BF16 scores).
 *
 * For query row q (request r, position t) and local entry j < n_vis =
 * min(floor((t+1)/m), kv_off[r+1]-kv_off[r]):
 *   S[q][j] = sum_h w[q][h] * ReLU(qi[q*n_heads+h] . ki[kv_off[r]+j])
 * (relu = 0 drops the ReLU), accumulated in fp32 and stored as F32 or
 * BF16 (round to nearest-even) at scores + q*ld + j.  Columns j >= n_vis are
 * not written.
 *   qi        rows = n_q * n_heads, fmt F32 | BF16 | MXFP4 (dim % 32 == 0)
 *   ki        entry keys, same fmt and dim as qi
 *   head_w    float [n_q][n_heads] or NULL (all weights 1)
 *   scores    [n_q][ld] of score_fmt (F32 | BF16), ld >= batch->max_kv
 * ------------------------------------------------------------------------- */
csa_status csa_indexer_score(const csa_tensor* qi, int32_t n_heads, const float* head_w,
                             const csa_tensor* ki, const csa_batch* batch, int32_t m,
                             int32_t relu, void* scores, int32_t score_fmt, int64_t ld,
                             hipStream_t stream);

/* ---------------------------------------------------------------------------
 * csa_topk_select - CSA step 2, top-k selection.
 * Page "DeepSeek V4 深度解析", section 2, CSA step 2 (each query keeps the k
 * most relevant entries: 1024 Pro, 512 Flash).
 *
 * Row q's candidates are its n_vis visible entries (as in csa_indexer_score).
 * Keeps the min(k, n_vis) largest scores, ties broken by the lower entry
 * index, and writes them in ascending index order to idx[q][0..], padding
 * the row with -1.  Exact (radix select on the order-preserving integer image
 * of the scores); scores must not be NaN.
 *   scores  [n_q][ld] F32 | BF16;  idx int32 [n_q][k];  1 <= k <= 4096
 * ------------------------------------------------------------------------- */
csa_status csa_topk_select(const void* scores, int32_t score_fmt, int64_t ld,
                           const csa_batch* batch, int32_t m, int32_t k, int32_t* idx,
                           hipStream_t stream);

/* ---------------------------------------------------------------------------
 * csa_indexer_topk - CSA step 2 fused: indexer scores and top-k selection.
 * Page "DeepSeek V4 深度解析", section 2, CSA step 2 (light indexer scores,
 * then the k most relevant entries per query) and the FP4 paragraph.
 *
 * Same result, bit for bit, as csa_indexer_score (same qi, ki, head_w, m,
 * relu, score_fmt; ld >= max_kv) followed by csa_topk_select (same k): the
 * min(k, n_vis) best entries of each query by the score rounded to score_fmt,
 * ties to the lower index, ascending, -1 padded.  The score matrix is never
 * written: each query keeps a list of candidates in `workspace`, sized by
 * csa_indexer_topk_workspace_size(n_q, k) and owned by the caller (16-byte
 * aligned; its contents are scratch, nothing needs clearing between calls).
 * Candidates are the entries at or above an estimated threshold (sampled per
 * query for a single request's query groups, chosen by each filter workgroup
 * for its own entries when every request has one query); rows whose list
 * misses (more than it holds, fewer than k, or a k-th key below a threshold)
 * are redone exactly from recomputed scores, so the result never depends on
 * the estimate.
 *   qi, ki, head_w, batch, m, relu, score_fmt   as csa_indexer_score
 *   idx    int32 [n_q][k];  1 <= k <= 4096;  rows of at most 2^20 entries
 * Errors: CSA_ERR_WORKSPACE if workspace is NULL or short; CSA_ERR_UNSUPPORTED
 * for max_kv > 2^20 or the formats csa_indexer_score refuses.
 * ------------------------------------------------------------------------- */
size_t csa_indexer_topk_workspace_size(int64_t n_q, int32_t k);
csa_status csa_indexer_topk(const csa_tensor* qi, int32_t n_heads, const float* head_w,
                            const csa_tensor* ki, const csa_batch* batch, int32_t m,
                            int32_t relu, int32_t score_fmt, int32_t k, int32_t* idx,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * csa_indexer_topk_noalloc - csa_indexer_topk for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same result, bit for bit, with the
 * candidate lists in a static device array of the library instead of a
 * caller workspace.  Nothing is allocated by the call.
 *   arguments   as csa_indexer_topk, without workspace / workspace_bytes
 *   limit       csa_indexer_topk_workspace_size(n_q, k) must not exceed
 *               csa_indexer_topk_noalloc_max_bytes() (16 MiB: e.g. 256 decode
 *               queries at k = 1024); larger calls return CSA_ERR_WORKSPACE
 *               before anything is launched
 *   sharing     each GPU holds one such array for the life of the process,
 *               shared by every call on that GPU: calls on one GPU that may
 *               overlap in time (different streams, threads) race and must
 *               be ordered by the caller; calls on one stream are ordered
 *   first call  on a device resolves the array's device address once
 *               (hipGetSymbolAddress); a failure there is CSA_ERR_HIP
 * ------------------------------------------------------------------------- */
size_t csa_indexer_topk_noalloc_max_bytes(void);
csa_status csa_indexer_topk_noalloc(const csa_tensor* qi, int32_t n_heads, const float* head_w,
                                    const csa_tensor* ki, const csa_batch* batch, int32_t m,
                                    int32_t relu, int32_t score_fmt, int32_t k, int32_t* idx,
                                    hipStream_t stream);

/* ---------------------------------------------------------------------------
 * csa_sparse_mqa_attn - CSA step 3 / HCA dense attention.
 * Page "DeepSeek V4 深度解析", section 2: CSA step 3 (a sliding-window branch
 * of the latest 128 uncompressed tokens, attended together with the selected
 * entries) and the HCA paragraph (no selection, dense attention, same window,
 * shared-KV multi-query attention).
 *
 * Query row q of request r at position t has heads q_rows[q*n_heads + h].
 * Key set: the entries idx[q][0..k) that are >= 0 (CSA), or, when idx is NULL,
 * every visible entry j < n_vis (HCA); plus, when raw != NULL and window > 0,
 * the raw rows of positions max(0, t-window+1) .. t that request r holds.
 * Each key is also its value.  One softmax over the union:
 *   o[q][h] = sum_key softmax(scale * q_h . key) * key,
 *   lse[q][h] = natural log-sum-exp of the scaled logits (optional).
 * A row whose key set is empty gets o = 0 and lse = -inf.
 *   q         rows = n_q*n_heads, dim D (128 | 512), F32 or BF16; or
 *             FP8_MIXED (fp8 queries, stored like KV entries: the same
 *             section's mixed-precision paragraph read for the query side;
 *             D 512, FP8_MIXED kv (not NULL), BF16 raw, 64 or 128 heads, at
 *             most 4096 keys per query without a split)
 *   kv        entries: F32 (D 128), BF16, or FP8_MIXED (D 512); may be NULL
 *             for a window-only call
 *   raw       window rows, F32 or BF16 (q's format; BF16 for fp8 queries),
 *             dim D; may be NULL
 *   compute   F32 q, kv and raw use fp32 matrix cores; otherwise all operands
 *             are bf16 (FP8_MIXED rows dequantised to bf16 exactly) with
 *             fp32 accumulation and bf16 probabilities.  With fp8 queries
 *             the logits' non-RoPE products over entries run on the fp8
 *             matrix cores with both block scales (exact products, fp32
 *             sums); tiles holding window rows, the RoPE dims and the
 *             values as above
 *   scale     > 0 (the pages fix none; 1/sqrt(D) is the usual choice)
 *   out       [n_q*n_heads][D] F32 or BF16;  lse float [n_q*n_heads] or NULL
 *   n_heads   8, 16 or a multiple of 32 up to 128 (8 and 16 need a single
 *             request and no split)
 *   split_keys 0: each query's keys are processed by one workgroup.  > 0
 *             (decode): a query's key list of n keys (its entries, then its
 *             window rows) is cut into p = min(32, ceil(n/split_keys))
 *             parts of ceil(n/p) keys rounded up to a multiple of 32 (the
 *             last takes the rest), processed in parallel and merged in
 *             order by log-sum-exp (with D = 512, 64 or 128 heads and a BF16
 *             out, each part's normalised output is kept in bf16 before the
 *             merge).  The parts depend on n and split_keys alone, so a
 *             request's result does not depend on the other requests.  With D = 512 a part
 *             holds at most 2048 keys with 64 heads and 4096 with 128
 *             (CSA_ERR_UNSUPPORTED otherwise).  Needs `workspace` (device
 *             memory, caller-owned, contents not preserved) of at least
 *             csa_attn_workspace_size(n_q, n_heads, D, max_keys, split_keys)
 *             bytes, where max_keys = (k if idx else batch->max_kv) + window.
 *             Calls sharing one workspace must not overlap.
 * ------------------------------------------------------------------------- */
csa_status csa_sparse_mqa_attn(const csa_tensor* q, int32_t n_heads, const csa_tensor* kv,
                               const int32_t* idx, int32_t k, const csa_tensor* raw,
                               int32_t window, const csa_batch* batch, int32_t m, float scale,
                               void* out, int32_t out_fmt, float* lse, int32_t split_keys,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes csa_sparse_mqa_attn needs for split_keys > 0 (0 otherwise). */
size_t csa_attn_workspace_size(int64_t n_q, int32_t n_heads, int32_t dim, int64_t max_keys,
                               int32_t split_keys);

/* ---------------------------------------------------------------------------
 * csa_swa_merge - combination of the window branch and the compressed branch.
 * Page "DeepSeek V4 深度解析", section 2, CSA step 3 (the two are attended
 * together): a softmax over the union of two disjoint key sets equals
 *   M = max(a, b),  o = (e^(a-M) o_a + e^(b-M) o_b) / (e^(a-M) + e^(b-M)),
 *   lse = M + log(e^(a-M) + e^(b-M))
 * with a = lse_a[r], b = lse_b[r] (fp32 arithmetic).  A side with lse = -inf
 * contributes nothing; both -inf gives o = 0, lse = -inf.
 *   o_a, o_b  float [rows][dim];  lse_a, lse_b float [rows]
 *   out       [rows][dim] F32 or BF16;  lse_out float [rows] or NULL
 * ------------------------------------------------------------------------- */
csa_status csa_swa_merge(const float* o_a, const float* lse_a, const float* o_b,
                         const float* lse_b, int64_t rows, int32_t dim, void* out,
                         int32_t out_fmt, float* lse_out, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Storage formats.  Page "DeepSeek V4 深度解析", section 2 (KV cache: RoPE
 * dims BF16, the rest FP8) and the FP4 quantisation paragraph of section 4
 * (FP4 -> FP8 is lossless while the block max/min ratio is bounded).
 *
 * csa_quantize: src (F32 | BF16) -> dst of the same rows and dim:
 *   BF16 (from F32, nearest-even), FP8_MIXED (dim 512), MXFP4 (dim % 32 == 0).
 * csa_dequantize: src of any format -> float [rows][dim] (exact).
 * csa_mxfp4_to_fp8: MXFP4 rows -> e4m3fn codes uint8 [rows][dim] with one
 *   power-of-two group scale per row, g = max block exponent - 6, stored as an
 *   e8m0 byte in group_scale[rows]; lossless[r] = 1 iff the row's block
 *   exponents span at most 14 (then the conversion is exact).
 * ------------------------------------------------------------------------- */
csa_status csa_quantize(const csa_tensor* src, const csa_tensor* dst, hipStream_t stream);
csa_status csa_dequantize(const csa_tensor* src, float* dst, hipStream_t stream);
csa_status csa_mxfp4_to_fp8(const csa_tensor* src, uint8_t* fp8, uint8_t* group_scale,
                            uint8_t* lossless, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Projections around the path.  Page "DeepSeek V4 深度解析", section 2, HCA
 * paragraph (CSA and HCA both project their outputs in groups to cut
 * compute); page "wmrh.cn/news/726125", "V4 改进一" (the output side projected
 * in groups; before it, the MLA passage: a low-rank query side, the key/value
 * up-projections absorbed into the query and output projections).  The pages
 * give no sizes: these calls take any that meet the alignment rules below.
 *
 * csa_linear: y_b = x_b W_b^T for b < batch (the q, KV, indexer and output
 *   projections), bf16 operands, fp32 accumulation, y F32 or BF16 (nearest
 *   even).  Element strides:
 *     x  bf16 [batch][M][K] at x + b*x_bstride + m*ldx + k
 *     w  bf16 [batch][N][K] at w + b*w_bstride + n*ldw + k  (weights [out][in])
 *     y  [batch][M][N]      at y + b*y_bstride + m*ldy + n
 *   K a positive multiple of 64; ldx, ldw >= K and ldy >= N; x and w 16-byte
 *   aligned with ldx, ldw, x_bstride, w_bstride multiples of 8; M, N >= 0
 *   (0: nothing to do); 1 <= batch <= 65535.  Caller-owned device memory; y
 *   must not overlap x or w.  Errors: CSA_ERR_INVALID_ARGUMENT (null pointer,
 *   short leading dimension, misalignment), CSA_ERR_UNSUPPORTED (K not a
 *   multiple of 64, a size beyond 2^31, y format).
 *
 * csa_grouped_out_proj: out[n] = W_out . concat_g(W_g . o[n, heads of g]):
 *     o       bf16 [n_q][n_heads][dim] (the attention outputs)
 *     w_group bf16 [groups][d_group][(n_heads/groups)*dim]: group g takes
 *             heads g*n_heads/groups .. (g+1)*n_heads/groups - 1, flattened
 *             in head order
 *     w_out   bf16 [d_model][groups*d_group]
 *     out     [n_q][d_model] F32 or BF16
 *   The group results are rounded to bf16 (nearest even) into `workspace`
 *   (caller-owned device memory of csa_grouped_out_proj_workspace_size bytes,
 *   contents not preserved; calls sharing one must not overlap).  groups must
 *   divide n_heads; (n_heads/groups)*dim and groups*d_group multiples of 64.
 *   Errors as csa_linear, and CSA_ERR_WORKSPACE for a missing or short
 *   workspace.
 * ------------------------------------------------------------------------- */
csa_status csa_linear(const void* x, int64_t ldx, int64_t x_bstride, const void* w, int64_t ldw,
                      int64_t w_bstride, void* y, int32_t y_fmt, int64_t ldy, int64_t y_bstride,
                      int64_t M, int64_t N, int64_t K, int32_t batch, hipStream_t stream);
size_t csa_grouped_out_proj_workspace_size(int64_t n_q, int32_t groups, int32_t d_group);
csa_status csa_grouped_out_proj(const void* o, int64_t n_q, int32_t n_heads, int32_t dim,
                                int32_t groups, const void* w_group, int32_t d_group,
                                const void* w_out, int32_t d_model, void* out, int32_t out_fmt,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Introspection (host only).
 * ------------------------------------------------------------------------- */
int csa_abi_version(void);
const char* csa_status_string(csa_status s);
/* Description of the last error on the calling thread ("" if none). */
const char* csa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H_ */
