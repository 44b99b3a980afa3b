// The decode row map's body, shared by the m3s_decode_rows kernel and the
// store-and-rows kernel (one workgroup of T threads; s_scan holds T / 64 ints).
// Row r in [cu_q[b], cu_q[b+1]): row_req = b,
//   row_len = seq_len[b] - q_len_b + 1 + (r - cu_q[b]);
// pad rows (r >= cu_q[B], or rows of a rejected request): (-1, 0); and the
// exclusive prefix sum of each request's causal block count.
#pragma once
#include "fp4.hpp"
#include "launch.hpp"

namespace m3s {

template <int T>
__device__ __forceinline__ void decode_rows_body(const RowsArgs& a, int* s_scan) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int B = a.num_reqs;
  // every load of the launch is independent of the others: issued at once
  const int q_first = a.cu_q[0];
  const int q_end = a.cu_q[B];
  int carry = 0;  // blocks of the requests before this chunk (uniform)
  for (int base = 0; base < B; base += T) {
    const int b = base + tid;
    int nblk = 0;
    if (b < B) {
      const int q0 = a.cu_q[b], q1 = a.cu_q[b + 1];
      const int ql = q1 - q0;
      const int sl = a.seq_lens[b];
      const bool in_range = q0 >= 0 && q1 <= a.num_rows && ql >= 0;
      const bool ok = in_range && ql >= 1 && ql <= kMaxQLen && sl >= ql;
      if (!ok) set_status(a.status, kDevBadRows);
      if (ok) {
        nblk = (sl + kPage - 1) / kPage;
        for (int i = 0; i < ql; ++i) {
          a.row_req[q0 + i] = b;
          a.row_len[q0 + i] = sl - ql + 1 + i;
        }
      } else if (in_range) {
        for (int i = 0; i < ql; ++i) {
          a.row_req[q0 + i] = -1;
          a.row_len[q0 + i] = 0;
        }
      }
    }
    // exclusive scan of nblk over this chunk of requests
    int x = nblk;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_scan[wid] = x;
    __syncthreads();
    if (wid == 0) {
      int w = lane < T / 64 ? s_scan[lane] : 0;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(w, off, 64);
        if (lane >= off) w += y;
      }
      if (lane < T / 64) s_scan[lane] = w;  // inclusive wave totals
    }
    __syncthreads();
    const int wave_base = wid ? s_scan[wid - 1] : 0;
    if (b < B) a.req_blk[b] = carry + wave_base + x - nblk;
    carry += s_scan[T / 64 - 1];
    __syncthreads();  // s_scan is rewritten by the next chunk
  }
  if (tid == 0) {
    a.req_blk[B] = carry;
    if (q_first != 0 || q_end > a.num_rows || q_end < 0) set_status(a.status, kDevBadRows);
  }
  // pad rows after the last request, and before cu_q[0] if it is not 0
  const int lo = q_end < 0 ? 0 : (q_end > a.num_rows ? a.num_rows : q_end);
  for (int r = lo + tid; r < a.num_rows; r += T) {
    a.row_req[r] = -1;
    a.row_len[r] = 0;
  }
  const int hi0 = q_first < 0 ? 0 : (q_first > a.num_rows ? a.num_rows : q_first);
  for (int r = tid; r < hi0; r += T) {
    a.row_req[r] = -1;
    a.row_len[r] = 0;
  }
}

}  // namespace m3s
