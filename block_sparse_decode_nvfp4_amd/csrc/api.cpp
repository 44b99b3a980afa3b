// C-ABI entry points: synchronous host-side validation, then asynchronous
// launches on the caller's stream. Nothing here allocates, frees or waits
// (except m3s_read_device_status, which is documented to synchronize).
#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include <atomic>

#include "m3s.h"
#include "launch.hpp"

static_assert(M3S_NOALLOC_SCRATCH_BYTES == m3s::kNoallocScratchBytes, "scratch size mismatch");

using namespace m3s;

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

m3s_status check_cache(const m3s_cache* c) {
  if (!c) return M3S_ERR_INVALID_ARG;
  if (c->format != M3S_FMT_NVFP4 && c->format != M3S_FMT_MXFP4) return M3S_ERR_UNSUPPORTED;
  if (c->page_size != M3S_PAGE || c->head_dim != M3S_HEAD_DIM || c->num_kv_heads != 1)
    return M3S_ERR_UNSUPPORTED;
  if (c->num_pages < 0) return M3S_ERR_INVALID_ARG;
  return M3S_OK;
}

m3s_status check_rows(const m3s_rows* r) {
  if (!r) return M3S_ERR_INVALID_ARG;
  if (r->num_groups < 0 || r->num_rows < 0) return M3S_ERR_INVALID_ARG;
  if (r->num_groups > M3S_MAX_GROUPS || r->num_rows > M3S_MAX_ROWS) return M3S_ERR_UNSUPPORTED;
  if (!r->grp_row || !r->grp_blk) return M3S_ERR_INVALID_ARG;
  if (r->num_rows > 0 && (!r->row_req || !r->row_len)) return M3S_ERR_INVALID_ARG;
  return M3S_OK;
}

m3s_status check_table(const int32_t* bt, int32_t bt_stride, int32_t max_blocks) {
  if (!bt) return M3S_ERR_INVALID_ARG;
  if (max_blocks < 1 || bt_stride < max_blocks) return M3S_ERR_INVALID_ARG;
  if (max_blocks > M3S_MAX_BLOCKS) return M3S_ERR_UNSUPPORTED;
  return M3S_OK;
}

int scan_grid() {
  // one 16-wave scan workgroup per CU of the current device
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::atomic<int>* slot = (dev >= 0 && dev < 64) ? &cached[dev] : nullptr;
  if (slot) {
    const int c = slot->load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (slot) slot->store(cus, std::memory_order_relaxed);
  return cus;
}

m3s_status from_hip(hipError_t e) { return e == hipSuccess ? M3S_OK : M3S_ERR_HIP; }

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Fused call's workspace: the index call's part, the attention's, then the
// selected ids' pages, each 256-byte aligned. Offset of the last part.
size_t fused_ws_pages_offset(int32_t num_rows, int32_t max_blocks, int32_t topk) {
  return align256(index_ws_bytes(num_rows, max_blocks)) + align256(attend_ws_bytes(num_rows, attend_nsplit(topk)));
}

}  // namespace

extern "C" {

int32_t m3s_version(void) { return M3S_VERSION; }

const char* m3s_status_string(m3s_status s) {
  switch (s) {
    case M3S_OK: return "ok";
    case M3S_ERR_INVALID_ARG: return "invalid argument (null pointer, negative count, bad stride or alignment)";
    case M3S_ERR_UNSUPPORTED: return "unsupported shape (page/head_dim != 128, G, top-k, or size limits)";
    case M3S_ERR_WORKSPACE:
      return "workspace null or smaller than m3s_workspace_bytes (for the no-allocation call: "
             "more than the library's scratch)";
    case M3S_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

size_t m3s_workspace_bytes(int32_t op, int32_t num_rows, int32_t num_reqs, int32_t max_blocks, int32_t topk,
                           int32_t num_heads) {
  (void)num_reqs;
  (void)num_heads;
  if (num_rows < 0 || max_blocks < 0 || topk < 1 || topk > M3S_MAX_TOPK) return 0;
  if (op == M3S_OP_INDEX_TOPK) return index_ws_bytes(num_rows, max_blocks);
  if (op == M3S_OP_SPARSE_ATTEND) return attend_ws_bytes(num_rows, attend_nsplit(topk));
  if (op == M3S_OP_INDEX_TOPK_ATTEND)
    return fused_ws_pages_offset(num_rows, max_blocks, topk) + align256((size_t)num_rows * topk * sizeof(int32_t));
  return 0;
}

namespace {

m3s_status store_args(StoreArgs& a, const m3s_cache* cache, const uint16_t* k, const uint16_t* v,
                      const uint16_t* idx_k, int64_t row_stride, const int32_t* slot_mapping, int32_t num_tokens,
                      uint32_t* dev_status) {
  m3s_status st = check_cache(cache);
  if (st != M3S_OK) return st;
  if (num_tokens < 0) return M3S_ERR_INVALID_ARG;
  if (num_tokens > 0) {
    if (!slot_mapping) return M3S_ERR_INVALID_ARG;
    if (row_stride < M3S_HEAD_DIM || (row_stride & 7)) return M3S_ERR_INVALID_ARG;
    const uint16_t* src[3] = {k, v, idx_k};
    uint8_t* dat[3] = {cache->k_data, cache->v_data, cache->idx_data};
    uint8_t* scl[3] = {cache->k_scale, cache->v_scale, cache->idx_scale};
    for (int t = 0; t < 3; ++t) {
      if (!src[t]) continue;
      if (!aligned16(src[t]) || !dat[t] || !scl[t]) return M3S_ERR_INVALID_ARG;
    }
  }
  a.format = cache->format;
  a.k = k;
  a.v = v;
  a.idx = idx_k;
  a.row_stride = row_stride;
  a.slots = slot_mapping;
  a.num_tokens = num_tokens;
  a.num_pages = cache->num_pages;
  a.k_data = cache->k_data;
  a.k_scale = cache->k_scale;
  a.v_data = cache->v_data;
  a.v_scale = cache->v_scale;
  a.idx_data = cache->idx_data;
  a.idx_scale = cache->idx_scale;
  a.status = dev_status;
  return M3S_OK;
}

m3s_status rows_args(RowsArgs& a, const int32_t* cu_q, const int32_t* seq_lens, int32_t num_reqs,
                     int32_t num_rows, int32_t* row_req, int32_t* row_len, int32_t* req_blk, uint32_t* dev_status) {
  if (num_reqs < 0 || num_rows < 0) return M3S_ERR_INVALID_ARG;
  if (num_reqs > M3S_MAX_REQS || num_rows > M3S_MAX_ROWS) return M3S_ERR_UNSUPPORTED;
  if (!cu_q || !req_blk) return M3S_ERR_INVALID_ARG;
  if (num_reqs > 0 && !seq_lens) return M3S_ERR_INVALID_ARG;
  if (num_rows > 0 && (!row_req || !row_len)) return M3S_ERR_INVALID_ARG;
  a.cu_q = cu_q;
  a.seq_lens = seq_lens;
  a.num_reqs = num_reqs;
  a.num_rows = num_rows;
  a.row_req = row_req;
  a.row_len = row_len;
  a.req_blk = req_blk;
  a.grp_row = nullptr;
  a.grp_req = nullptr;
  a.max_groups = 0;
  a.status = dev_status;
  return M3S_OK;
}

m3s_status prefill_rows_args(RowsArgs& a, const int32_t* cu_q, const int32_t* seq_lens, int32_t num_reqs,
                             int32_t num_rows, int32_t max_groups, int32_t* row_req, int32_t* row_len,
                             int32_t* grp_row, int32_t* grp_req, int32_t* grp_blk, uint32_t* dev_status) {
  if (num_reqs < 0 || num_rows < 0) return M3S_ERR_INVALID_ARG;
  if (num_reqs > M3S_MAX_REQS || num_rows > M3S_MAX_ROWS) return M3S_ERR_UNSUPPORTED;
  if (max_groups < 1 || max_groups > M3S_MAX_GROUPS) return M3S_ERR_UNSUPPORTED;
  if (!cu_q || !grp_row || !grp_req || !grp_blk) return M3S_ERR_INVALID_ARG;
  if (num_reqs > 0 && !seq_lens) return M3S_ERR_INVALID_ARG;
  if (num_rows > 0 && (!row_req || !row_len)) return M3S_ERR_INVALID_ARG;
  a.cu_q = cu_q;
  a.seq_lens = seq_lens;
  a.num_reqs = num_reqs;
  a.num_rows = num_rows;
  a.row_req = row_req;
  a.row_len = row_len;
  a.req_blk = grp_blk;
  a.grp_row = grp_row;
  a.grp_req = grp_req;
  a.max_groups = max_groups;
  a.status = dev_status;
  return M3S_OK;
}

}  // namespace

m3s_status m3s_store(const m3s_cache* cache, const uint16_t* k, const uint16_t* v, const uint16_t* idx_k,
                     int64_t row_stride, const int32_t* slot_mapping, int32_t num_tokens, uint32_t* dev_status,
                     hipStream_t stream) {
  StoreArgs a;
  const m3s_status st = store_args(a, cache, k, v, idx_k, row_stride, slot_mapping, num_tokens, dev_status);
  if (st != M3S_OK || num_tokens == 0) return st;
  return from_hip(launch_store(a, stream));
}

m3s_status m3s_decode_rows(const int32_t* cu_q, const int32_t* seq_lens, int32_t num_reqs, int32_t num_rows,
                           int32_t* row_req, int32_t* row_len, int32_t* req_blk, uint32_t* dev_status,
                           hipStream_t stream) {
  RowsArgs a;
  const m3s_status st = rows_args(a, cu_q, seq_lens, num_reqs, num_rows, row_req, row_len, req_blk, dev_status);
  if (st != M3S_OK) return st;
  return from_hip(launch_decode_rows(a, stream));
}

m3s_status m3s_store_and_rows(const m3s_cache* cache, const uint16_t* k, const uint16_t* v, const uint16_t* idx_k,
                              int64_t row_stride, const int32_t* slot_mapping, int32_t num_tokens,
                              const int32_t* cu_q, const int32_t* seq_lens, int32_t num_reqs, int32_t num_rows,
                              int32_t* row_req, int32_t* row_len, int32_t* req_blk, uint32_t* dev_status,
                              hipStream_t stream) {
  StoreArgs s;
  m3s_status st = store_args(s, cache, k, v, idx_k, row_stride, slot_mapping, num_tokens, dev_status);
  if (st != M3S_OK) return st;
  RowsArgs r;
  st = rows_args(r, cu_q, seq_lens, num_reqs, num_rows, row_req, row_len, req_blk, dev_status);
  if (st != M3S_OK) return st;
  return from_hip(launch_store_rows(s, r, stream));
}

m3s_status m3s_qknorm_rope_store(const m3s_cache* cache, const uint16_t* q, int64_t q_stride,
                                 int32_t num_heads, const uint16_t* k, const uint16_t* v,
                                 const uint16_t* idx_q, const uint16_t* idx_k, int64_t row_stride,
                                 const uint16_t* norm_weights, float eps, const int32_t* positions,
                                 const float* cos_sin, int32_t max_pos, int32_t rotary_dim,
                                 const int32_t* slot_mapping, int32_t num_tokens, uint16_t* q_out,
                                 uint8_t* q_out_e4m3, uint16_t* idx_q_out, uint32_t* dev_status,
                                 hipStream_t stream) {
  m3s_status st = check_cache(cache);
  if (st != M3S_OK) return st;
  if (num_tokens < 0) return M3S_ERR_INVALID_ARG;
  if (num_heads < 1 || num_heads > M3S_MAX_HEADS) return M3S_ERR_UNSUPPORTED;
  if (rotary_dim < 0 || rotary_dim > M3S_HEAD_DIM || (rotary_dim & 15)) return M3S_ERR_UNSUPPORTED;
  if (!(eps >= 0.0f) || !isfinite(eps)) return M3S_ERR_INVALID_ARG;
  if (num_tokens > 0) {
    const void* in16[] = {q, k, v, idx_q, idx_k, norm_weights, q_out, idx_q_out};
    for (const void* p : in16)
      if (!p || !aligned16(p)) return M3S_ERR_INVALID_ARG;
    if (!slot_mapping) return M3S_ERR_INVALID_ARG;
    if (q_out_e4m3 && ((uintptr_t)q_out_e4m3 & 7u)) return M3S_ERR_INVALID_ARG;
    if (q_stride < (int64_t)M3S_HEAD_DIM * num_heads || (q_stride & 7)) return M3S_ERR_INVALID_ARG;
    if (row_stride < M3S_HEAD_DIM || (row_stride & 7)) return M3S_ERR_INVALID_ARG;
    if (rotary_dim > 0 && (!positions || !cos_sin || !aligned16(cos_sin) || max_pos < 1)) return M3S_ERR_INVALID_ARG;
    if (!cache->k_data || !cache->k_scale || !cache->v_data || !cache->v_scale || !cache->idx_data ||
        !cache->idx_scale)
      return M3S_ERR_INVALID_ARG;
  }
  if (num_tokens == 0) return M3S_OK;
  ProducerArgs a;
  a.format = cache->format;
  a.q = q;
  a.q_stride = q_stride;
  a.num_heads = num_heads;
  a.k = k;
  a.v = v;
  a.idx_q = idx_q;
  a.idx_k = idx_k;
  a.row_stride = row_stride;
  a.norm_w = norm_weights;
  a.eps = eps;
  a.positions = positions;
  a.cos_sin = cos_sin;
  a.max_pos = rotary_dim > 0 ? max_pos : 0;
  a.rotary_dim = rotary_dim;
  a.slots = slot_mapping;
  a.num_tokens = num_tokens;
  a.num_pages = cache->num_pages;
  a.k_data = cache->k_data;
  a.k_scale = cache->k_scale;
  a.v_data = cache->v_data;
  a.v_scale = cache->v_scale;
  a.idx_data = cache->idx_data;
  a.idx_scale = cache->idx_scale;
  a.q_out = q_out;
  a.q_out_e4m3 = q_out_e4m3;
  a.idx_q_out = idx_q_out;
  a.status = dev_status;
  return from_hip(launch_producer(a, stream));
}

m3s_status m3s_prefill_rows(const int32_t* cu_q, const int32_t* seq_lens, int32_t num_reqs, int32_t num_rows,
                            int32_t max_groups, int32_t* row_req, int32_t* row_len, int32_t* grp_row,
                            int32_t* grp_req, int32_t* grp_blk, uint32_t* dev_status, hipStream_t stream) {
  RowsArgs a;
  const m3s_status st = prefill_rows_args(a, cu_q, seq_lens, num_reqs, num_rows, max_groups, row_req, row_len,
                                          grp_row, grp_req, grp_blk, dev_status);
  if (st != M3S_OK) return st;
  return from_hip(launch_prefill_rows(a, stream));
}

m3s_status m3s_store_and_prefill_rows(const m3s_cache* cache, const uint16_t* k, const uint16_t* v,
                                      const uint16_t* idx_k, int64_t row_stride, const int32_t* slot_mapping,
                                      int32_t num_tokens, const int32_t* cu_q, const int32_t* seq_lens,
                                      int32_t num_reqs, int32_t num_rows, int32_t max_groups, int32_t* row_req,
                                      int32_t* row_len, int32_t* grp_row, int32_t* grp_req, int32_t* grp_blk,
                                      uint32_t* dev_status, hipStream_t stream) {
  StoreArgs s;
  m3s_status st = store_args(s, cache, k, v, idx_k, row_stride, slot_mapping, num_tokens, dev_status);
  if (st != M3S_OK) return st;
  RowsArgs r;
  st = prefill_rows_args(r, cu_q, seq_lens, num_reqs, num_rows, max_groups, row_req, row_len, grp_row, grp_req,
                         grp_blk, dev_status);
  if (st != M3S_OK) return st;
  return from_hip(launch_store_prefill_rows(s, r, stream));
}

}  // extern "C"

namespace {

// Validation and argument set-up of the index call; workspace as given.
m3s_status index_args(IndexArgs& a, const m3s_cache* cache, const uint16_t* q_idx, int64_t q_idx_stride,
                      const int32_t* block_table, int32_t bt_stride, int32_t max_blocks, const m3s_rows* rows,
                      int32_t topk, int32_t flags, int32_t init_blocks, int32_t local_blocks, int32_t* topk_ids,
                      void* workspace, size_t workspace_bytes, uint32_t* dev_status) {
  m3s_status st = check_cache(cache);
  if (st != M3S_OK) return st;
  if (!cache->idx_data || !cache->idx_scale) return M3S_ERR_INVALID_ARG;
  st = check_rows(rows);
  if (st != M3S_OK) return st;
  st = check_table(block_table, bt_stride, max_blocks);
  if (st != M3S_OK) return st;
  if (topk < 1 || topk > M3S_MAX_TOPK) return M3S_ERR_UNSUPPORTED;
  if (flags & ~(int32_t)M3S_TOPK_TIE_HIGH_ID) return M3S_ERR_INVALID_ARG;
  if (init_blocks < 0 || local_blocks < 0 || init_blocks > M3S_MAX_BLOCKS || local_blocks > M3S_MAX_BLOCKS)
    return M3S_ERR_INVALID_ARG;
  if (rows->num_rows > 0) {
    if (!q_idx || !aligned16(q_idx) || q_idx_stride < M3S_HEAD_DIM || (q_idx_stride & 7)) return M3S_ERR_INVALID_ARG;
    if (!topk_ids) return M3S_ERR_INVALID_ARG;
  }
  const size_t need = index_ws_bytes(rows->num_rows, max_blocks);
  if (workspace_bytes < need || (need > 0 && !workspace) || !aligned16(workspace)) return M3S_ERR_WORKSPACE;
  a.format = cache->format;
  a.idx_data = cache->idx_data;
  a.idx_scale = cache->idx_scale;
  a.num_pages = cache->num_pages;
  a.q_idx = q_idx;
  a.q_stride = q_idx_stride;
  a.block_table = block_table;
  a.bt_stride = bt_stride;
  a.max_blocks = max_blocks;
  a.cu_q = rows->grp_row;
  a.grp_req = rows->grp_req;
  a.row_req = rows->row_req;
  a.row_len = rows->row_len;
  a.req_blk = rows->grp_blk;
  a.seq_lens = nullptr;
  a.num_reqs = rows->num_groups;
  a.num_rows = rows->num_rows;
  a.topk = topk;
  a.tie_high = (flags & M3S_TOPK_TIE_HIGH_ID) ? 1 : 0;
  a.init_blocks = init_blocks;
  a.local_blocks = local_blocks;
  a.topk_ids = topk_ids;
  a.sel_pages = nullptr;
  a.ws_score = static_cast<float*>(workspace);
  a.ws_bound = reinterpret_cast<float*>(static_cast<char*>(workspace) + need / 2);
  a.status = dev_status;
  a.scan_grid = rows->num_rows > 0 ? scan_grid() : 0;
  a.group_tiles = rows->grp_req ? 4 : 1;
  return M3S_OK;
}

// Validation and argument set-up of the attention; workspace as given.
m3s_status attend_args(AttendArgs& a, const m3s_cache* cache, const uint16_t* q, int64_t q_row_stride,
                       int64_t q_head_stride, int32_t num_heads, const int32_t* block_table, int32_t bt_stride,
                       int32_t max_blocks, const m3s_rows* rows, const int32_t* topk_ids, int32_t topk,
                       float sm_scale, float* out, void* workspace, size_t workspace_bytes, uint32_t* dev_status) {
  m3s_status st = check_cache(cache);
  if (st != M3S_OK) return st;
  if (!cache->k_data || !cache->k_scale || !cache->v_data || !cache->v_scale) return M3S_ERR_INVALID_ARG;
  st = check_rows(rows);
  if (st != M3S_OK) return st;
  st = check_table(block_table, bt_stride, max_blocks);
  if (st != M3S_OK) return st;
  if (num_heads < 1 || num_heads > M3S_MAX_HEADS) return M3S_ERR_UNSUPPORTED;
  if (topk < 1 || topk > M3S_MAX_TOPK) return M3S_ERR_UNSUPPORTED;
  if (!isfinite(sm_scale)) return M3S_ERR_INVALID_ARG;
  if (rows->num_rows > 0) {
    if (!q || !aligned16(q) || (q_row_stride & 7) || (q_head_stride & 7) || q_row_stride < 0 || q_head_stride < 0)
      return M3S_ERR_INVALID_ARG;
    if (num_heads > 1 && q_head_stride < M3S_HEAD_DIM) return M3S_ERR_INVALID_ARG;
    if (!topk_ids || !out) return M3S_ERR_INVALID_ARG;
  }
  const int32_t nsplit = attend_nsplit(topk);
  const size_t need = attend_ws_bytes(rows->num_rows, nsplit);
  if (workspace_bytes < need || (need > 0 && !workspace) || !aligned16(workspace)) return M3S_ERR_WORKSPACE;
  a.format = cache->format;
  a.k_data = cache->k_data;
  a.k_scale = cache->k_scale;
  a.v_data = cache->v_data;
  a.v_scale = cache->v_scale;
  a.num_pages = cache->num_pages;
  a.q = q;
  a.q_row_stride = q_row_stride;
  a.q_head_stride = q_head_stride;
  a.num_heads = num_heads;
  a.block_table = block_table;
  a.bt_stride = bt_stride;
  a.max_blocks = max_blocks;
  a.row_req = rows->row_req;
  a.row_len = rows->row_len;
  a.num_rows = rows->num_rows;
  a.topk_ids = topk_ids;
  a.sel_pages = nullptr;
  a.topk = topk;
  a.nsplit = nsplit;
  // A row's splits on one XCD lets the combine read the partials from that XCD's
  // L2; measured faster while every split workgroup is resident at once (64 rows:
  // 14.9 -> 14.1 us), slightly slower with several rounds of workgroups (384 rows).
  a.xcd_rows = rows->num_rows > 0 && (int64_t)rows->num_rows * nsplit <= 2 * (int64_t)scan_grid() ? 1 : 0;
  // With more than two rounds of split workgroups, each wave attends four blocks
  // in turn (online softmax across them), or two when k <= 12: a quarter (half) of
  // the splits, so fewer partials written and combined, and a top-k of 16 is one
  // split per row with no combine at all. The workspace stays sized for the
  // one-block split count.
  a.reps = 1;
  if (nsplit > 1 && rows->num_rows > 0 && (int64_t)rows->num_rows * nsplit > 4 * (int64_t)scan_grid()) {
    a.reps = nsplit >= 4 ? 4 : 2;
    a.nsplit = (nsplit + a.reps - 1) / a.reps;
  }
  a.sm_scale = sm_scale;
  a.out = out;
  const size_t po = align256((size_t)rows->num_rows * nsplit * 16 * M3S_HEAD_DIM * sizeof(float));
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = need ? reinterpret_cast<float*>(static_cast<char*>(workspace) + po) : nullptr;
  a.status = dev_status;
  return M3S_OK;
}

}  // namespace

extern "C" {

m3s_status m3s_index_topk(const m3s_cache* cache, const uint16_t* q_idx, int64_t q_idx_stride,
                          const int32_t* block_table, int32_t bt_stride, int32_t max_blocks, const m3s_rows* rows,
                          int32_t topk, int32_t flags, int32_t init_blocks, int32_t local_blocks,
                          int32_t* topk_ids, void* workspace, size_t workspace_bytes,
                          uint32_t* dev_status, hipStream_t stream) {
  IndexArgs a;
  const m3s_status st = index_args(a, cache, q_idx, q_idx_stride, block_table, bt_stride, max_blocks, rows, topk,
                                   flags, init_blocks, local_blocks, topk_ids, workspace, workspace_bytes, dev_status);
  if (st != M3S_OK || rows->num_rows == 0) return st;
  return from_hip(launch_index_topk(a, stream));
}

m3s_status m3s_sparse_attend(const m3s_cache* cache, const uint16_t* q, int64_t q_row_stride, int64_t q_head_stride,
                             int32_t num_heads, const int32_t* block_table, int32_t bt_stride, int32_t max_blocks,
                             const m3s_rows* rows, const int32_t* topk_ids, int32_t topk, float sm_scale, float* out,
                             void* workspace, size_t workspace_bytes, uint32_t* dev_status, hipStream_t stream) {
  AttendArgs a;
  const m3s_status st = attend_args(a, cache, q, q_row_stride, q_head_stride, num_heads, block_table, bt_stride,
                                    max_blocks, rows, topk_ids, topk, sm_scale, out, workspace, workspace_bytes,
                                    dev_status);
  if (st != M3S_OK || rows->num_rows == 0) return st;
  return from_hip(launch_sparse_attend(a, stream));
}

}  // extern "C"

namespace {

// m3s_index_topk_attend on a given workspace (the caller's, or the library's scratch).
m3s_status index_topk_attend_impl(const m3s_cache* cache, const uint16_t* q_idx, int64_t q_idx_stride,
                                  const uint16_t* q, int64_t q_row_stride, int64_t q_head_stride, int32_t num_heads,
                                  const int32_t* block_table, int32_t bt_stride, int32_t max_blocks,
                                  const m3s_rows* rows, int32_t topk, int32_t flags, int32_t init_blocks,
                                  int32_t local_blocks, float sm_scale, int32_t* topk_ids, float* out,
                                  void* workspace, size_t workspace_bytes, uint32_t* dev_status, hipStream_t stream) {
  if (!rows) return M3S_ERR_INVALID_ARG;
  if (max_blocks < 0 || rows->num_rows < 0) return M3S_ERR_INVALID_ARG;
  const size_t ni = align256(index_ws_bytes(rows->num_rows, max_blocks));
  if (workspace_bytes < ni) return M3S_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  IndexArgs ia;
  m3s_status st = index_args(ia, cache, q_idx, q_idx_stride, block_table, bt_stride, max_blocks, rows, topk, flags,
                             init_blocks, local_blocks, topk_ids, ws, ni, dev_status);
  if (st != M3S_OK) return st;
  AttendArgs aa;
  st = attend_args(aa, cache, q, q_row_stride, q_head_stride, num_heads, block_table, bt_stride, max_blocks, rows,
                   topk_ids, topk, sm_scale, out, ws ? ws + ni : nullptr, workspace_bytes - ni, dev_status);
  if (st != M3S_OK || rows->num_rows == 0) return st;
  // The last part holds the page of each selected id, written by the select
  // beside the ids when the call runs the select and the attention as
  // separate kernels (many rows); the attention then skips its block-table
  // lookup.
  const size_t np = fused_ws_pages_offset(rows->num_rows, max_blocks, topk);
  if (workspace_bytes < np + align256((size_t)rows->num_rows * topk * sizeof(int32_t))) return M3S_ERR_WORKSPACE;
  ia.sel_pages = reinterpret_cast<int32_t*>(ws + np);
  aa.sel_pages = ia.sel_pages;
  return from_hip(launch_index_topk_attend(ia, aa, stream));
}

}  // namespace

extern "C" {

m3s_status m3s_index_topk_attend(const m3s_cache* cache, const uint16_t* q_idx, int64_t q_idx_stride,
                                 const uint16_t* q, int64_t q_row_stride, int64_t q_head_stride, int32_t num_heads,
                                 const int32_t* block_table, int32_t bt_stride, int32_t max_blocks,
                                 const m3s_rows* rows, int32_t topk, int32_t flags, int32_t init_blocks,
                                 int32_t local_blocks, float sm_scale, int32_t* topk_ids, float* out,
                                 void* workspace, size_t workspace_bytes, uint32_t* dev_status, hipStream_t stream) {
  return index_topk_attend_impl(cache, q_idx, q_idx_stride, q, q_row_stride, q_head_stride, num_heads, block_table,
                                bt_stride, max_blocks, rows, topk, flags, init_blocks, local_blocks, sm_scale,
                                topk_ids, out, workspace, workspace_bytes, dev_status, stream);
}

m3s_status m3s_index_topk_attend_noalloc(const m3s_cache* cache, const uint16_t* q_idx, int64_t q_idx_stride,
                                         const uint16_t* q, int64_t q_row_stride, int64_t q_head_stride,
                                         int32_t num_heads, const int32_t* block_table, int32_t bt_stride,
                                         int32_t max_blocks, const m3s_rows* rows, int32_t topk, int32_t flags,
                                         int32_t init_blocks, int32_t local_blocks, float sm_scale, int32_t* topk_ids,
                                         float* out, uint32_t* dev_status, hipStream_t stream) {
  if (!rows || max_blocks < 0 || rows->num_rows < 0) return M3S_ERR_INVALID_ARG;
  // sizes past the scratch are refused before anything touches the GPU
  const size_t need = m3s_workspace_bytes(M3S_OP_INDEX_TOPK_ATTEND, rows->num_rows, rows->num_groups, max_blocks,
                                          topk, num_heads);
  if (need > M3S_NOALLOC_SCRATCH_BYTES) return M3S_ERR_WORKSPACE;
  void* ws = nullptr;
  if (noalloc_scratch(&ws) != hipSuccess) return M3S_ERR_HIP;
  return index_topk_attend_impl(cache, q_idx, q_idx_stride, q, q_row_stride, q_head_stride, num_heads, block_table,
                                bt_stride, max_blocks, rows, topk, flags, init_blocks, local_blocks, sm_scale,
                                topk_ids, out, ws, M3S_NOALLOC_SCRATCH_BYTES, dev_status, stream);
}

m3s_status m3s_decode_step(const m3s_cache* cache, const uint16_t* k, const uint16_t* v, const uint16_t* idx_k,
                           int64_t row_stride, const int32_t* slot_mapping, const int32_t* cu_q,
                           const int32_t* seq_lens, int32_t num_reqs, int32_t num_rows, int32_t* row_req,
                           int32_t* row_len, int32_t* req_blk, const uint16_t* q_idx, int64_t q_idx_stride,
                           const uint16_t* q, int64_t q_row_stride, int64_t q_head_stride, int32_t num_heads,
                           const int32_t* block_table, int32_t bt_stride, int32_t max_blocks, int32_t topk,
                           int32_t flags, int32_t init_blocks, int32_t local_blocks, float sm_scale,
                           int32_t* topk_ids, float* out, void* workspace, size_t workspace_bytes,
                           uint32_t* dev_status, hipStream_t stream) {
  StoreArgs s;
  m3s_status st = store_args(s, cache, k, v, idx_k, row_stride, slot_mapping, num_rows, dev_status);
  if (st != M3S_OK) return st;
  RowsArgs r;
  st = rows_args(r, cu_q, seq_lens, num_reqs, num_rows, row_req, row_len, req_blk, dev_status);
  if (st != M3S_OK) return st;
  m3s_rows rows;
  rows.grp_row = cu_q;
  rows.grp_req = nullptr;
  rows.grp_blk = req_blk;
  rows.row_req = row_req;
  rows.row_len = row_len;
  rows.num_groups = num_reqs;
  rows.num_rows = num_rows;
  if (max_blocks < 0) return M3S_ERR_INVALID_ARG;
  const size_t ni = align256(index_ws_bytes(num_rows, max_blocks));
  if (workspace_bytes < ni) return M3S_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  IndexArgs ia;
  st = index_args(ia, cache, q_idx, q_idx_stride, block_table, bt_stride, max_blocks, &rows, topk, flags,
                  init_blocks, local_blocks, topk_ids, ws, ni, dev_status);
  if (st != M3S_OK) return st;
  AttendArgs aa;
  st = attend_args(aa, cache, q, q_row_stride, q_head_stride, num_heads, block_table, bt_stride, max_blocks, &rows,
                   topk_ids, topk, sm_scale, out, ws ? ws + ni : nullptr, workspace_bytes - ni, dev_status);
  if (st != M3S_OK) return st;
  const size_t np = fused_ws_pages_offset(num_rows, max_blocks, topk);
  if (num_rows > 0 && workspace_bytes < np + align256((size_t)num_rows * topk * sizeof(int32_t)))
    return M3S_ERR_WORKSPACE;
  ia.sel_pages = num_rows > 0 ? reinterpret_cast<int32_t*>(ws + np) : nullptr;
  aa.sel_pages = ia.sel_pages;
  ia.seq_lens = seq_lens;
  if (ia.scan_grid == 0) ia.scan_grid = scan_grid();
  return from_hip(launch_decode_step(ia, aa, s, r, stream));
}

m3s_status m3s_read_device_status(const uint32_t* dev_status, uint32_t* out, hipStream_t stream) {
  if (!dev_status || !out) return M3S_ERR_INVALID_ARG;
  hipError_t e = hipMemcpyAsync(out, dev_status, sizeof(uint32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  return from_hip(e);
}

}  // extern "C"
