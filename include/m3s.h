/*
 * m3s.h - C ABI of the decode hot path for block-sparse attention over
 * NVFP4 / MXFP4 paged caches (MiniMax-M3 indexed sparse-attention layers),
 * built for MI355X (gfx950).
 *
 * Four calls make one decode step, issued in this order on one stream:
 *
 *   m3s_store          quantize the step's new K, V and index-K rows and write
 *                      them into the paged uint8 planes at their slots
 *   m3s_decode_rows    map every decode / verify row to (request, causal length)
 *   m3s_index_topk     score every causal 128-token block of every row against
 *                      the FP4 index cache, keep each row's top-k block ids
 *   m3s_sparse_attend  GQA softmax attention of each row over only its top-k
 *                      blocks of the FP4 K/V cache
 *
 * Sources (web pages; sections named, not quoted):
 *   [ATOM-2746]  ROCm/ATOM PR "NVFP4 sparse KV", Summary and Tests.
 *   [ATOM-2744]  ROCm/ATOM PR "[MiniMax-M3.1] FP4 index cache and NVFP4 sparse
 *                KV cache", Design (Kernels, Write path, Index, Decode score
 *                grid, Attention, Fused verify top-k), Follow-up: MXFP4
 *                caches, Tests, and the review notes on ties, ascending ids,
 *                page size and invalid block ids.
 *   [VLLM-64198] vllm-project/vllm PR "MXFP4 KV + indexer cache for
 *                MiniMax-M3.1", Claims and Design.
 *
 * Conventions shared by every call:
 *   - All tensor pointers are DEVICE pointers unless a comment says "host".
 *     The caller owns every buffer; the library never allocates, frees or
 *     synchronizes inside these calls. Every call is asynchronous on `stream`
 *     and may be captured into a HIP graph (all counts that depend on device
 *     data are read on the device; nothing is read back to the host).
 *   - bf16 tensors are passed as `const uint16_t*` (raw bfloat16 bits).
 *   - Host-side validation runs first and is synchronous. It returns
 *     M3S_ERR_INVALID_ARG (null pointer, negative count, too-small stride) or
 *     M3S_ERR_UNSUPPORTED (a shape the kernels do not implement) or
 *     M3S_ERR_WORKSPACE (workspace null or smaller than m3s_workspace_bytes)
 *     without touching the GPU. M3S_ERR_HIP reports a failed launch.
 *   - Device-side problems (an out-of-range page or block id, a bad length)
 *     never wrap and never fault: the kernel ORs an M3S_DEV_* bit into
 *     `*dev_status` (one uint32 on the device, optional: may be NULL) and the
 *     affected row produces -1 ids / zero output. The bits are sticky; the
 *     caller clears the word.
 *   - No C++ exception crosses this boundary.
 *
 * Geometry (fixed): page = sparse block = 128 tokens ([ATOM-2744] review:
 * the block size must equal the page size), head_dim = 128, one KV head and
 * one index head per GPU (one rank of a TP4 deployment).
 */
#ifndef M3S_H
#define M3S_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define M3S_VERSION 1

#define M3S_PAGE 128
#define M3S_HEAD_DIM 128
#define M3S_MAX_Q_LEN 16     /* rows per request (1 target + up to 15 drafts) */
#define M3S_MAX_HEADS 16     /* query heads per KV head (G) */
#define M3S_MAX_TOPK 64
#define M3S_MAX_REQS 4096
#define M3S_MAX_GROUPS 4096  /* scan work groups (requests, or 64-row prefill groups) */
#define M3S_MAX_ROWS 65536
#define M3S_MAX_BLOCKS 8192  /* causal blocks per request: 1,048,576 tokens */

typedef int32_t m3s_status;
enum {
  M3S_OK = 0,
  M3S_ERR_INVALID_ARG = 1,
  M3S_ERR_UNSUPPORTED = 2,
  M3S_ERR_WORKSPACE = 3,
  M3S_ERR_HIP = 4
};

/* Cache formats ([ATOM-2746] Summary; [ATOM-2744] Follow-up: MXFP4 caches;
 * [VLLM-64198] Claims). */
enum {
  M3S_FMT_NVFP4 = 1, /* e2m1 codes + one E4M3FN scale per 16 elements: 64 + 8 B per token */
  M3S_FMT_MXFP4 = 2  /* e2m1 codes + one E8M0 scale per 32 elements:   64 + 4 B per token */
};

/* Sticky device status bits (ORed into *dev_status). */
enum {
  M3S_DEV_BAD_SLOT = 1u << 0,     /* store: slot >= num_pages * 128 */
  M3S_DEV_BAD_ROWS = 1u << 1,     /* decode_rows / prefill_rows: q_len outside its range, seq_len < q_len,
                                     cu_q not non-decreasing, or cu_q[B] > num_rows */
  M3S_DEV_BAD_LENGTH = 1u << 2,   /* a live row needs more than max_blocks blocks */
  M3S_DEV_BAD_PAGE = 1u << 3,     /* block table entry outside [0, num_pages) */
  M3S_DEV_BAD_BLOCK_ID = 1u << 4, /* attend: top-k id outside the row's causal blocks */
  M3S_DEV_INEXACT = 1u << 5,      /* index_topk: an exact rescore could not prove its
                                     float64 sum exact (ids may then differ from exact
                                     arithmetic in a near tie) */
  M3S_DEV_BAND_OVERFLOW = 1u << 6, /* index_topk: more than 1024 blocks inside a row's
                                      uncertainty band; that row fell back to the
                                      approximate scores */
  M3S_DEV_BAD_POSITION = 1u << 7,  /* qknorm_rope_store: position outside [0, max_pos);
                                      that token's outputs are left unwritten */
  M3S_DEV_RANGE = 1u << 8,         /* attend: an output element was not finite in fp32 (logits
                                      or sums beyond the fp32 range; MXFP4 scale bytes 253
                                      and 254, which no store writes, decode to infinity);
                                      that element is written as 0 */
  M3S_DEV_STEP_SLOT = 1u << 9      /* decode_step: a new token's slot is not its position in its
                                      own request's block table; the step's results are then
                                      not defined */
};

/* Flags of m3s_index_topk. */
enum {
  M3S_TOPK_TIE_HIGH_ID = 1 /* equal scores rank the higher block id first (the rule of
                              the [ATOM-2744] review notes); default: lower id first */
};

/*
 * One KV head's paged cache (host struct; the plane pointers are device
 * pointers). Reading of [ATOM-2746] Summary (K, V and their scales are
 * separate uint8 planes) and [VLLM-64198] Claims (an MXFP4 page holds 128
 * rows of 64 B of codes, then 128 rows of 4 B of scales):
 * each tensor (K, V, index K) has a payload plane and a scale plane, page
 * major; slot s = page * 128 + offset lives at
 *     payload[page][offset][0..64)   byte j = code(2j) | code(2j+1) << 4
 *     scale  [page][offset][0..SB)   SB = 8 (NVFP4) or 4 (MXFP4)
 * page_size must be 128, head_dim 128, num_kv_heads 1.
 */
typedef struct m3s_cache {
  int32_t format;       /* M3S_FMT_NVFP4 or M3S_FMT_MXFP4 */
  int32_t num_pages;
  int32_t page_size;    /* = 128 */
  int32_t head_dim;     /* = 128 */
  int32_t num_kv_heads; /* = 1 */
  uint8_t* k_data;
  uint8_t* k_scale;
  uint8_t* v_data;
  uint8_t* v_scale;
  uint8_t* idx_data;
  uint8_t* idx_scale;
} m3s_cache;

/*
 * The row map of one step (host struct of device pointers), filled by
 * m3s_decode_rows or m3s_prefill_rows and shared by m3s_index_topk and
 * m3s_sparse_attend ([ATOM-2744] Design, Attention: one row-map launch,
 * shared by the attention and the fused top-k).
 *
 * The index scan scores one page against a work group of consecutive rows of
 * one request at a time. With grp_req = NULL (m3s_decode_rows: each request
 * is one group, grp_row = cu_q) a group holds at most 16 rows; with grp_req
 * set (m3s_prefill_rows: each request's rows cut into groups of 64) at most
 * 64. Rows past that in a group are not scored and set M3S_DEV_BAD_ROWS.
 */
typedef struct m3s_rows {
  const int32_t* grp_row; /* [num_groups + 1] first row of each work group; grp_row[num_groups] ends the rows */
  const int32_t* grp_req; /* [num_groups] request of each group (-1: empty), or NULL: group g is request g */
  const int32_t* grp_blk; /* [num_groups + 1] exclusive prefix sum of each group's causal block count */
  const int32_t* row_req; /* [num_rows] request of each row, -1 for a pad row */
  const int32_t* row_len; /* [num_rows] causal length of each row, 0 for a pad row */
  int32_t num_groups;     /* <= M3S_MAX_GROUPS */
  int32_t num_rows;       /* padded row count */
} m3s_rows;

/*
 * m3s_store - [ATOM-2744] Write path: per 16 elements scale = e4m3(amax / 6),
 * codes rounded half to even and saturating at 6 (NVFP4); [ATOM-2744]
 * Follow-up: MXFP4 caches: one E8M0 scale per 32 elements (MXFP4, OCP MX v1.0
 * scale rule 2^(floor(log2 amax) - 2)). Rows with slot_mapping[t] < 0 are pad
 * rows and are left unwritten ([ATOM-2744] Tests).
 *
 *   k, v, idx_k   bf16 [num_tokens, row_stride] (the first 128 elements of each
 *                 row are used); any of the three may be NULL to skip it.
 *   row_stride    elements between consecutive rows (>= 128).
 *   slot_mapping  int32 [num_tokens]; slot = page * 128 + offset.
 * A slot >= num_pages * 128 sets M3S_DEV_BAD_SLOT and is skipped.
 * One launch covers all three tensors. NaN / Inf inputs are outside the format.
 */
m3s_status m3s_store(const m3s_cache* cache, const uint16_t* k, const uint16_t* v,
                     const uint16_t* idx_k, int64_t row_stride, const int32_t* slot_mapping,
                     int32_t num_tokens, uint32_t* dev_status, hipStream_t stream);

/*
 * m3s_decode_rows - [ATOM-2746] Summary, Attention: one launch builds each
 * decode row's (request, causal length) on the device. Row r in
 * [cu_q[b], cu_q[b+1]) gets row_req = b and
 *     row_len = seq_lens[b] - q_len_b + 1 + (r - cu_q[b]),  q_len_b = cu_q[b+1] - cu_q[b]
 * (seq_lens include the step's own rows). Rows r >= cu_q[num_reqs] are pad
 * rows: (-1, 0). req_blk[b] = sum over b' < b of ceil(seq_lens[b'] / 128).
 *
 *   cu_q       int32 [num_reqs + 1], seq_lens int32 [num_reqs]
 *   row_req, row_len  int32 [num_rows] (outputs), req_blk int32 [num_reqs + 1] (output)
 * A request with q_len outside [1, 16] or seq_len < q_len sets M3S_DEV_BAD_ROWS
 * and its rows become pad rows (its block count is 0). For m3s_index_topk and
 * m3s_sparse_attend, pass m3s_rows { grp_row = cu_q, grp_req = NULL,
 * grp_blk = req_blk, row_req, row_len, num_groups = num_reqs, num_rows }.
 */
m3s_status m3s_decode_rows(const int32_t* cu_q, const int32_t* seq_lens, int32_t num_reqs,
                           int32_t num_rows, int32_t* row_req, int32_t* row_len,
                           int32_t* req_blk, uint32_t* dev_status, hipStream_t stream);

/*
 * m3s_store_and_rows - m3s_store and m3s_decode_rows in one launch (the two
 * are independent: the store writes the planes, the row map its own arrays).
 * Arguments, validation, results and status bits are those of the two calls;
 * a call that would fail either of them launches nothing. For a caller that
 * runs both each step, it saves one launch ([ATOM-2744] Design, Write path:
 * the pages measure the store as launch-bound).
 */
m3s_status m3s_store_and_rows(const m3s_cache* cache, const uint16_t* k, const uint16_t* v,
                              const uint16_t* idx_k, int64_t row_stride, const int32_t* slot_mapping,
                              int32_t num_tokens, const int32_t* cu_q, const int32_t* seq_lens,
                              int32_t num_reqs, int32_t num_rows, int32_t* row_req, int32_t* row_len,
                              int32_t* req_blk, uint32_t* dev_status, hipStream_t stream);

/*
 * m3s_qknorm_rope_store - the fused producer store ([ATOM-2744] Follow-up:
 * MXFP4 caches: the quantization moves into the fused qk-norm / RoPE / cache
 * kernel, with no staging buffer and no store launch; [VLLM-64198] Claims: that
 * kernel writes the K, V and index-K pages and the main query as e4m3). The
 * pages do not define the norm or the rotary embedding; per token this call
 * computes, in fp32, for each 128-dim row x of the G query heads, the key, the
 * index query and the index key (weight rows 0, 1, 2, 3 of norm_weights):
 *     y = x / sqrt(mean(x^2) + eps) * w
 *     for d < h = rotary_dim / 2:  (y_d, y_{d+h}) <- (y_d c - y_{d+h} s, y_{d+h} c + y_d s)
 *         c = cos_sin[pos][d], s = cos_sin[pos][h + d], pos = positions[t]
 * and rounds each result to bf16 (to nearest even). The value row is neither
 * normed nor rotated. Outputs:
 *   q_out       bf16 [num_tokens, G, 128] (contiguous): the query rows;
 *   q_out_e4m3  uint8 [num_tokens, G, 128] or NULL: E4M3FN bytes of q_out
 *               (nearest, ties to even, saturating at 448, no scale);
 *   idx_q_out   bf16 [num_tokens, 128] (contiguous): the index-query rows;
 *   the cache   the key, value and index-key rows quantized at slot_mapping[t]
 *               exactly as m3s_store quantizes these bf16 rows (pad tokens,
 *               slot < 0, write no cache bytes but do write their queries).
 * Inputs:
 *   q           bf16 [num_tokens, q_stride], head h at elements [128 h, 128 h + 128);
 *               q_stride >= 128 * num_heads, a multiple of 8
 *   num_heads   G in [1, 16]
 *   k, v, idx_q, idx_k  bf16 [num_tokens, row_stride] (first 128 used), row_stride >= 128,
 *               a multiple of 8
 *   norm_weights bf16 [4, 128]
 *   eps         finite, >= 0
 *   positions   int32 [num_tokens] (may be NULL when rotary_dim is 0)
 *   cos_sin     float32 [max_pos, rotary_dim]: cos in columns [0, h), sin in [h, 2h)
 *   rotary_dim  a multiple of 16 in [0, 128]
 * Pointers to bf16, float and e4m3 data must be 16-byte aligned (q_out_e4m3:
 * 8-byte). Errors: host validation returns M3S_ERR_INVALID_ARG /
 * M3S_ERR_UNSUPPORTED without launching; a position outside [0, max_pos) sets
 * M3S_DEV_BAD_POSITION and leaves that token's outputs unwritten; a slot >=
 * num_pages * 128 sets M3S_DEV_BAD_SLOT and writes no cache bytes for it.
 */
m3s_status m3s_qknorm_rope_store(const m3s_cache* cache, const uint16_t* q, int64_t q_stride,
                                 int32_t num_heads, const uint16_t* k, const uint16_t* v,
                                 const uint16_t* idx_q, const uint16_t* idx_k, int64_t row_stride,
                                 const uint16_t* norm_weights, float eps, const int32_t* positions,
                                 const float* cos_sin, int32_t max_pos, int32_t rotary_dim,
                                 const int32_t* slot_mapping, int32_t num_tokens, uint16_t* q_out,
                                 uint8_t* q_out_e4m3, uint16_t* idx_q_out, uint32_t* dev_status,
                                 hipStream_t stream);

/*
 * m3s_prefill_rows - [ATOM-2744] Design, row maps (prefill_rows): every query
 * token of a request's prefill chunk is a row; row r of request b sees
 *   row_len = seq_lens[b] - (cu_q[b+1] - cu_q[b]) + 1 + (r - cu_q[b])
 * tokens (the decode_rows map with no bound on a request's row count). It
 * also cuts each request's rows into work groups of 64 for the index scan:
 *   grp_row int32 [max_groups + 1], grp_req int32 [max_groups],
 *   grp_blk int32 [max_groups + 1] (outputs; groups past the last real one
 *   are empty); pass them with num_groups = max_groups in m3s_rows.
 *   max_groups   in [1, M3S_MAX_GROUPS]; sum_b ceil(q_len_b / 64) groups are
 *                needed, at most ceil(cu_q[B] / 64) + num_reqs
 * A request with seq_len < q_len sets M3S_DEV_BAD_ROWS and its rows become pad
 * rows. A cu_q that does not start at 0, decreases or passes num_rows, or more
 * groups than max_groups, sets M3S_DEV_BAD_ROWS and makes every row a pad row.
 */
m3s_status m3s_prefill_rows(const int32_t* cu_q, const int32_t* seq_lens, int32_t num_reqs,
                            int32_t num_rows, int32_t max_groups, int32_t* row_req, int32_t* row_len,
                            int32_t* grp_row, int32_t* grp_req, int32_t* grp_blk, uint32_t* dev_status,
                            hipStream_t stream);

/*
 * m3s_store_and_prefill_rows - m3s_store and m3s_prefill_rows in one launch (the
 * two are independent: the store writes the planes, the row map its own arrays),
 * for a prefill chunk's step. Arguments, validation, results and status bits are
 * those of the two calls; a call that would fail either of them launches nothing.
 * It saves one launch of a step whose store and row map are each mostly launch and
 * first-load latency ([ATOM-2744] Design, Write path: the store is launch-bound).
 */
m3s_status m3s_store_and_prefill_rows(const m3s_cache* cache, const uint16_t* k, const uint16_t* v,
                                      const uint16_t* idx_k, int64_t row_stride, const int32_t* slot_mapping,
                                      int32_t num_tokens, const int32_t* cu_q, const int32_t* seq_lens,
                                      int32_t num_reqs, int32_t num_rows, int32_t max_groups, int32_t* row_req,
                                      int32_t* row_len, int32_t* grp_row, int32_t* grp_req, int32_t* grp_blk,
                                      uint32_t* dev_status, hipStream_t stream);

/*
 * m3s_index_topk - [ATOM-2744] Design, Index and Decode score grid, and Fused
 * verify top-k: score every causal 128-token block of every row against the
 * FP4 index cache (reached through the block table) and keep the top-k.
 *   score(row, j) = max over tokens t of block j with t < row_len of
 *                   sum_d q_idx[row][d] * dequant(idx)[t][d]
 * ids are the k best blocks by (score desc, id asc; id desc with
 * M3S_TOPK_TIE_HIGH_ID), emitted ASCENDING, padded with -1 when the row has
 * fewer than k causal blocks. The selection equals the one exact arithmetic
 * makes: the scan computes fp32 scores with a rigorous error bound and
 * rescores, in exact float64, every block whose rank the bound leaves open.
 * Forced blocks ([VLLM-64198] Design: init / local sentinels on a row's causal
 * blocks; [ATOM-2744] review notes on init_blocks + local_blocks > topk): the
 * row's first init_blocks blocks rank above its newest local_blocks blocks,
 * which rank above every scored block; a block in both sets counts as initial;
 * ties among forced blocks go to the higher id, so when the forced blocks
 * exceed k the newest ones (the row's own block among them) are kept.
 *
 *   q_idx        bf16 [num_rows, q_idx_stride] (first 128 used)
 *   block_table  int32 [num_reqs, bt_stride]; block j of request b lives on
 *                page block_table[b * bt_stride + j]
 *   max_blocks   upper bound of ceil(row_len / 128) over rows (<= bt_stride)
 *   topk         in [1, 64]
 *   flags        0 or M3S_TOPK_TIE_HIGH_ID
 *   init_blocks, local_blocks  forced block counts, each in [0, M3S_MAX_BLOCKS]
 *   topk_ids     int32 [num_rows, topk] (output); pad rows get -1
 *   workspace    device scratch of m3s_workspace_bytes(M3S_OP_INDEX_TOPK, ...)
 */
m3s_status m3s_index_topk(const m3s_cache* cache, const uint16_t* q_idx, int64_t q_idx_stride,
                          const int32_t* block_table, int32_t bt_stride, int32_t max_blocks,
                          const m3s_rows* rows, int32_t topk, int32_t flags, int32_t init_blocks,
                          int32_t local_blocks, int32_t* topk_ids, void* workspace,
                          size_t workspace_bytes, uint32_t* dev_status, hipStream_t stream);

/*
 * m3s_sparse_attend - [ATOM-2746] Summary, Attention: block-sparse attention
 * addressed by the top-k block ids and the request block table. For each
 * row and query head h < num_heads (all heads share the one KV head):
 *   out[row][h] = sum_t p_t * dequant(V)[t],  p = softmax_t(sm_scale * q[row][h] . dequant(K)[t])
 * over the tokens t < row_len of the row's selected blocks. ids < 0 are
 * skipped; an id outside [0, ceil(row_len/128)) or a page outside
 * [0, num_pages) sets a status bit and is skipped. A row with no valid token
 * (pad rows included) outputs zeros. ids must be distinct.
 *
 *   q            bf16, element (row, h, d) at q[row * q_row_stride + h * q_head_stride + d]
 *   num_heads    G in [1, 16]
 *   topk_ids     int32 [num_rows, topk]
 *   out          fp32 [num_rows, num_heads, 128], contiguous
 *   workspace    device scratch of m3s_workspace_bytes(M3S_OP_SPARSE_ATTEND, ...)
 *                (split partials; none needed when topk <= 4). Calls that share
 *                a workspace must not overlap in time.
 * Computation: K and V are decoded exactly (code * scale): NVFP4 to fp16, with
 * the query scaled by a power of two into fp16 range, QK^T and PV on fp16 MFMA;
 * MXFP4 to bf16 (the only 16-bit type whose range holds every E8M0 scale a
 * store writes), the bf16 query as is, QK^T on bf16 MFMA and PV with P split
 * into two bf16 terms (16 significant bits); fp32 accumulation and softmax. Each workgroup takes 4 of a row's blocks
 * (a split); a combine pass merges the splits' partials (split-K online
 * softmax).
 */
m3s_status m3s_sparse_attend(const m3s_cache* cache, const uint16_t* q, int64_t q_row_stride,
                             int64_t q_head_stride, int32_t num_heads,
                             const int32_t* block_table, int32_t bt_stride, int32_t max_blocks,
                             const m3s_rows* rows, const int32_t* topk_ids, int32_t topk,
                             float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                             uint32_t* dev_status, hipStream_t stream);

/*
 * m3s_index_topk_attend - m3s_index_topk followed by m3s_sparse_attend on its
 * ids, with the select and the attention's split pass in one kernel
 * ([ATOM-2744] review notes: the fused top-k carries the splits and their
 * merge). Each (row, split) workgroup selects the row's blocks itself and then
 * attends its share of them with the ids and pages still on chip: one kernel
 * boundary and the attention's dependent id and page loads fewer than the two
 * calls. Arguments, validation, outputs (topk_ids and out) and status bits are
 * those of the two calls, bit for bit; the select runs once per split, so a
 * row's status bits may be set more than once.
 *   workspace    device scratch of m3s_workspace_bytes(M3S_OP_INDEX_TOPK_ATTEND, ...)
 *                (the index call's part, the attention's, then the selected ids'
 *                pages as num_rows x topk int32, each 256-byte aligned; the pages
 *                are written when many rows make the call run the select and the
 *                attention as separate kernels, and let the attention skip its
 *                block-table lookup)
 */
m3s_status m3s_index_topk_attend(const m3s_cache* cache, const uint16_t* q_idx, int64_t q_idx_stride,
                                 const uint16_t* q, int64_t q_row_stride, int64_t q_head_stride,
                                 int32_t num_heads, const int32_t* block_table, int32_t bt_stride,
                                 int32_t max_blocks, const m3s_rows* rows, int32_t topk, int32_t flags,
                                 int32_t init_blocks, int32_t local_blocks, float sm_scale,
                                 int32_t* topk_ids, float* out, void* workspace, size_t workspace_bytes,
                                 uint32_t* dev_status, hipStream_t stream);

/*
 * m3s_index_topk_attend_noalloc - for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): m3s_index_topk_attend with the workspace taken from a scratch buffer
 * the library owns instead of an argument. The scratch is one static device array
 * of M3S_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends; the call
 * allocates and frees nothing. Arguments, outputs and status bits are those of
 * m3s_index_topk_attend.
 *   - A call whose m3s_workspace_bytes(M3S_OP_INDEX_TOPK_ATTEND, ...) exceeds
 *     M3S_NOALLOC_SCRATCH_BYTES returns M3S_ERR_WORKSPACE and launches nothing
 *     (32 MiB: the 8 x 8-row 150K and skewed 450K batches need about 3-4 MiB,
 *     the 48 x 8-row lognormal batch about 23 MiB).
 *   - Every call on one GPU uses that GPU's one scratch buffer: calls that overlap
 *     in time on one GPU (two streams, two threads) race on it and must not be
 *     issued; calls in one stream order are fine. The buffer keeps the last call's
 *     contents; the kernels write every byte they read.
 *   - The first call on a device looks the buffer's device address up
 *     (hipGetSymbolAddress); make that first call outside graph capture.
 */
#define M3S_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
m3s_status m3s_index_topk_attend_noalloc(const m3s_cache* cache, const uint16_t* q_idx, int64_t q_idx_stride,
                                         const uint16_t* q, int64_t q_row_stride, int64_t q_head_stride,
                                         int32_t num_heads, const int32_t* block_table, int32_t bt_stride,
                                         int32_t max_blocks, const m3s_rows* rows, int32_t topk, int32_t flags,
                                         int32_t init_blocks, int32_t local_blocks, float sm_scale, int32_t* topk_ids,
                                         float* out, uint32_t* dev_status, hipStream_t stream);

/*
 * m3s_decode_step - one decode step of the whole path: m3s_store_and_rows (with
 * num_tokens = num_rows: token r is row r) followed by m3s_index_topk_attend on
 *   rows = { grp_row = cu_q, grp_req = NULL, grp_blk = req_blk, row_req, row_len,
 *            num_groups = num_reqs, num_rows },
 * with the store, the row map and the index scan in ONE launch ([ATOM-2744]
 * Design, Write path: the store is launch-bound on its own). In that launch one
 * workgroup builds the row map, and each request's blocks that hold one of its new
 * tokens are stored and scored by the same workgroup, after its stores; every other
 * causal block is scored by the scan workgroups, which never read a page the step
 * writes. Arguments, validation, outputs (planes, row_req, row_len, req_blk,
 * topk_ids, out) and status bits are those of the two calls, bit for bit, when the
 * step follows the decode convention:
 *   - slot_mapping[r] for row r of a request b that m3s_decode_rows accepts is
 *     block_table[b][p / 128] * 128 + p % 128 with p = seq_lens[b] - q_len_b + (r - cu_q[b]);
 *     a row that breaks it sets M3S_DEV_STEP_SLOT (results then undefined);
 *   - pad rows and rows of rejected requests have slot -1, and no page the step
 *     writes is also an older block of another request (shared prefix pages are
 *     read only); these two are not checked.
 * (Requests whose cu_q ranges overlap, which M3S_DEV_BAD_ROWS flags, leave the row
 * map undefined in either form.)
 *   workspace    as for m3s_index_topk_attend (m3s_workspace_bytes(M3S_OP_INDEX_TOPK_ATTEND, ...)).
 */
m3s_status m3s_decode_step(const m3s_cache* cache, const uint16_t* k, const uint16_t* v,
                           const uint16_t* idx_k, int64_t row_stride, const int32_t* slot_mapping,
                           const int32_t* cu_q, const int32_t* seq_lens, int32_t num_reqs,
                           int32_t num_rows, int32_t* row_req, int32_t* row_len, int32_t* req_blk,
                           const uint16_t* q_idx, int64_t q_idx_stride, const uint16_t* q,
                           int64_t q_row_stride, int64_t q_head_stride, int32_t num_heads,
                           const int32_t* block_table, int32_t bt_stride, int32_t max_blocks,
                           int32_t topk, int32_t flags, int32_t init_blocks, int32_t local_blocks,
                           float sm_scale, int32_t* topk_ids, float* out, void* workspace,
                           size_t workspace_bytes, uint32_t* dev_status, hipStream_t stream);

/* Workspace sizing (host only, pure). */
enum { M3S_OP_INDEX_TOPK = 1, M3S_OP_SPARSE_ATTEND = 2, M3S_OP_INDEX_TOPK_ATTEND = 3 };
size_t m3s_workspace_bytes(int32_t op, int32_t num_rows, int32_t num_reqs, int32_t max_blocks,
                           int32_t topk, int32_t num_heads);

/* Copies *dev_status to host memory `*out` (host pointer) and synchronizes `stream`. */
m3s_status m3s_read_device_status(const uint32_t* dev_status, uint32_t* out, hipStream_t stream);

/* Static description of a status code (never NULL). */
const char* m3s_status_string(m3s_status status);

/* M3S_VERSION of the built library. */
int32_t m3s_version(void);

/*
 * m3s_probe_page_reads - measurement only, not part of the decode path: reads
 * num_units whole NVFP4 pages (payload [P][128][64] and scales [P][128][8], page
 * pages[u] for unit u) with the index scan's load pattern and nothing else, so its
 * time gives the memory system's ceiling for that pattern. One 16-wave workgroup per
 * sink entry (pass the CU count); each writes one folded word to sink[num_sink].
 * mode 0: 2-byte scale loads per 16-token tile, as the NVFP4 scan loads them;
 * mode 1: one 16-byte load per lane over the page's 1 KB scale block;
 * mode 2: a plain stream of the same number of bytes for comparison: the first
 *   num_units pages of both planes front to back, 16-byte loads striding over the
 *   grid (pages is not read; num_units must not exceed the planes' pages).
 * Returns M3S_ERR_INVALID_ARG for null pointers, num_units < 0, num_sink < 1 or
 * another mode. Page ids are not checked: every pages[u] must lie in the planes.
 */
m3s_status m3s_probe_page_reads(const uint8_t* payload, const uint8_t* scales, const int32_t* pages,
                                int32_t num_units, int32_t mode, uint32_t* sink, int32_t num_sink,
                                hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* M3S_H */
