// m3s_decode_rows: one launch maps every decode / verify row to its request
// and causal length on the device ([ATOM-2746] Summary, Attention: built on
// the device in one launch so it stays valid under graph capture), and emits
// the exclusive prefix sum of each request's causal block count, which the
// index scan uses to flatten (request, block) work into one list.
//
// Row r in [cu_q[b], cu_q[b+1]): row_req = b,
//   row_len = seq_len[b] - q_len_b + 1 + (r - cu_q[b]).
// Pad rows (r >= cu_q[B], or rows of a rejected request): (-1, 0).
#include "fp4.hpp"
#include "launch.hpp"
#include "m3s.h"
#include "rows_body.hpp"

namespace m3s {

constexpr int kRowsThreads = 1024;

__global__ __launch_bounds__(kRowsThreads) void decode_rows_kernel(RowsArgs a) {
  __shared__ int s_scan[kRowsThreads / 64];
  decode_rows_body<kRowsThreads>(a, s_scan);
}

// Prefill row map and the scan's 64-row work groups, in one workgroup
// (prefill_rows_body, rows_body.hpp).
__global__ __launch_bounds__(kRowsThreads) void prefill_rows_kernel(RowsArgs a) {
  extern __shared__ int s_pref[];
  prefill_rows_body<kRowsThreads>(a, s_pref);
}

hipError_t launch_prefill_rows(const RowsArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(prefill_rows_kernel, dim3(1), dim3(kRowsThreads), prefill_rows_lds_bytes(a.num_reqs), stream, a);
  return hipGetLastError();
}

hipError_t launch_decode_rows(const RowsArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(decode_rows_kernel, dim3(1), dim3(kRowsThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace m3s
