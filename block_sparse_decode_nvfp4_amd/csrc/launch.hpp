// Internal interface between the C-ABI host layer (api.cpp) and the kernel
// translation units. Argument structs are passed by value as kernel arguments.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace m3s {

// Device status bits (mirror of the M3S_DEV_* values in m3s.h).
enum : uint32_t {
  kDevBadSlot = 1u << 0,
  kDevBadRows = 1u << 1,
  kDevBadLength = 1u << 2,
  kDevBadPage = 1u << 3,
  kDevBadBlockId = 1u << 4,
  kDevInexact = 1u << 5,
  kDevBandOverflow = 1u << 6,
  kDevBadPosition = 1u << 7,
  kDevRange = 1u << 8,
  kDevStepSlot = 1u << 9,
};

constexpr int kMaxBlocks = 8192;   // causal blocks per request
constexpr int kMaxQLen = 16;
constexpr int kBandCap = 1024;     // exact-rescore capacity per row

struct StoreArgs {
  int format;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* idx;
  int64_t row_stride;
  const int32_t* slots;
  int32_t num_tokens;
  int32_t num_pages;
  uint8_t* k_data;
  uint8_t* k_scale;
  uint8_t* v_data;
  uint8_t* v_scale;
  uint8_t* idx_data;
  uint8_t* idx_scale;
  uint32_t* status;
};

struct ProducerArgs {
  int format;
  const uint16_t* q;       // [T, q_stride], head h at h * 128
  int64_t q_stride;
  int32_t num_heads;
  const uint16_t* k;       // k, v, idx_q, idx_k: [T, row_stride]
  const uint16_t* v;
  const uint16_t* idx_q;
  const uint16_t* idx_k;
  int64_t row_stride;
  const uint16_t* norm_w;  // [4, 128]: query, key, index query, index key
  float eps;
  const int32_t* positions;
  const float* cos_sin;    // [max_pos, rotary_dim]
  int32_t max_pos;
  int32_t rotary_dim;
  const int32_t* slots;
  int32_t num_tokens;
  int32_t num_pages;
  uint8_t* k_data;
  uint8_t* k_scale;
  uint8_t* v_data;
  uint8_t* v_scale;
  uint8_t* idx_data;
  uint8_t* idx_scale;
  uint16_t* q_out;         // [T, G, 128]
  uint8_t* q_out_e4m3;     // [T, G, 128] or null
  uint16_t* idx_q_out;     // [T, 128]
  uint32_t* status;
};

struct RowsArgs {
  const int32_t* cu_q;
  const int32_t* seq_lens;
  int32_t num_reqs;
  int32_t num_rows;
  int32_t* row_req;
  int32_t* row_len;
  int32_t* req_blk;   // decode_rows: block prefix per request; prefill_rows: per group
  int32_t* grp_row;   // prefill_rows only: [max_groups + 1]
  int32_t* grp_req;   // prefill_rows only: [max_groups]
  int32_t max_groups; // prefill_rows only
  uint32_t* status;
};

struct IndexArgs {
  int format;
  const uint8_t* idx_data;
  const uint8_t* idx_scale;
  int32_t num_pages;
  const uint16_t* q_idx;
  int64_t q_stride;
  const int32_t* block_table;
  int32_t bt_stride;
  int32_t max_blocks;
  const int32_t* cu_q;     // first row of each scan work group [num_reqs + 1]
  const int32_t* grp_req;  // request of each work group, or null: group g is request g
  const int32_t* row_req;
  const int32_t* row_len;
  const int32_t* req_blk;
  const int32_t* seq_lens;  // decode step kernel only (else null): row lengths in closed form from
                            // seq_lens and cu_q; the scan's units are each request's blocks with no
                            // new token, the tail workgroups score the rest
  int32_t num_reqs;
  int32_t num_rows;
  int32_t topk;
  int32_t tie_high;
  int32_t init_blocks;   // forced initial blocks per row
  int32_t local_blocks;  // forced newest blocks per row
  int32_t* topk_ids;
  int32_t* sel_pages;  // [num_rows, topk]: page of each selected id beside topk_ids, or null
  float* ws_score;   // [num_rows, max_blocks]
  float* ws_bound;   // [num_rows, max_blocks]
  uint32_t* status;
  int32_t scan_grid; // workgroups of the scan kernel
  int32_t group_tiles; // 16-row query tiles per work group: 1 (decode, groups of <= 16 rows) or 4 (<= 64)
};

struct AttendArgs {
  int format;
  const uint8_t* k_data;
  const uint8_t* k_scale;
  const uint8_t* v_data;
  const uint8_t* v_scale;
  int32_t num_pages;
  const uint16_t* q;
  int64_t q_row_stride;
  int64_t q_head_stride;
  int32_t num_heads;
  const int32_t* block_table;
  int32_t bt_stride;
  int32_t max_blocks;
  const int32_t* row_req;
  const int32_t* row_len;
  int32_t num_rows;
  const int32_t* topk_ids;
  const int32_t* sel_pages;  // [num_rows, topk]: page of each id, written by the select; null: block table
  int32_t topk;
  int32_t nsplit;
  int32_t xcd_rows;  // nonzero: the split kernel deals a row's splits to one XCD
  int32_t reps;      // blocks each split-kernel wave attends in turn (1, 2 or 4)
  float sm_scale;
  float* out;
  float* part_o;   // [num_rows, nsplit, 16, 128]
  float* part_ml;  // [num_rows, nsplit, 16, 2]
  uint32_t* status;
};

hipError_t launch_store(const StoreArgs& a, hipStream_t stream);
hipError_t launch_decode_rows(const RowsArgs& a, hipStream_t stream);
hipError_t launch_prefill_rows(const RowsArgs& a, hipStream_t stream);
hipError_t launch_store_rows(const StoreArgs& s, const RowsArgs& r, hipStream_t stream);
hipError_t launch_store_prefill_rows(const StoreArgs& s, const RowsArgs& r, hipStream_t stream);
hipError_t launch_producer(const ProducerArgs& a, hipStream_t stream);
hipError_t launch_index_topk(const IndexArgs& a, hipStream_t stream);
hipError_t launch_sparse_attend(const AttendArgs& a, hipStream_t stream);
hipError_t launch_index_topk_attend(const IndexArgs& ia, const AttendArgs& aa, hipStream_t stream);
hipError_t launch_attend_combine(const AttendArgs& a, hipStream_t stream);
hipError_t launch_decode_step(const IndexArgs& ia, const AttendArgs& aa, const StoreArgs& s, const RowsArgs& r,
                              hipStream_t stream);

// The no-allocation entry point's scratch: a static device array of this size per GPU
// (scratch.hip); noalloc_scratch gives its device address on the current device.
constexpr size_t kNoallocScratchBytes = size_t(32) << 20;
hipError_t noalloc_scratch(void** ptr);

// Workspace layout helpers shared by sizing and launching.
size_t index_ws_bytes(int32_t num_rows, int32_t max_blocks);
size_t attend_ws_bytes(int32_t num_rows, int32_t nsplit);
int32_t attend_nsplit(int32_t topk);

}  // namespace m3s
