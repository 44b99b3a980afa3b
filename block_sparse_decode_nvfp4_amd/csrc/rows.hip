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

// Exclusive scan of one value per thread over the workgroup; returns the
// thread's exclusive prefix, *total gets the sum. Uses s_scan (16 ints).
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_scan, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_scan[wid] = x;
  __syncthreads();
  if (wid == 0) {
    int w = lane < kRowsThreads / 64 ? s_scan[lane] : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(w, off, 64);
      if (lane >= off) w += y;
    }
    if (lane < kRowsThreads / 64) s_scan[lane] = w;  // inclusive wave totals
  }
  __syncthreads();
  const int excl = (wid ? s_scan[wid - 1] : 0) + x - v;
  *total = s_scan[kRowsThreads / 64 - 1];
  __syncthreads();  // s_scan is reused by the next scan
  return excl;
}

constexpr int kGroupRows = 64;  // rows per scan work group (four MFMA column tiles)

// Prefill row map and the scan's 64-row work groups, in one workgroup. The
// request offsets, lengths and group offsets are staged in LDS; every row and
// every group is then written by its own thread (a chunk of thousands of rows
// is no longer one thread's loop).
__global__ __launch_bounds__(kRowsThreads) void prefill_rows_kernel(RowsArgs a) {
  __shared__ int s_cu[M3S_MAX_REQS + 1];
  __shared__ int s_sl[M3S_MAX_REQS];
  __shared__ int s_goff[M3S_MAX_REQS + 1];
  __shared__ int s_scan[kRowsThreads / 64];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  const int B = a.num_reqs, R = a.num_rows, MG = a.max_groups;
  if (tid == 0) s_bad = 0;
  for (int b = tid; b <= B; b += kRowsThreads) s_cu[b] = a.cu_q[b];
  for (int b = tid; b < B; b += kRowsThreads) s_sl[b] = a.seq_lens[b];
  __syncthreads();
  // the whole batch: cu_q must start at 0, never decrease and end within num_rows
  for (int b = tid; b < B; b += kRowsThreads)
    if (s_cu[b + 1] < s_cu[b]) atomicOr(&s_bad, 1);
  if (tid == 0 && (s_cu[0] != 0 || s_cu[B] > R)) atomicOr(&s_bad, 1);
  __syncthreads();
  const bool bad = s_bad != 0;
  // groups per request, then their offsets
  int carry = 0;
  for (int base = 0; base < B; base += kRowsThreads) {
    const int b = base + tid;
    const int ng = (!bad && b < B) ? (s_cu[b + 1] - s_cu[b] + kGroupRows - 1) / kGroupRows : 0;
    int tot;
    const int ex = block_exclusive_scan(ng, s_scan, &tot);
    if (b < B) s_goff[b] = carry + ex;
    carry += tot;
  }
  if (tid == 0) s_goff[B] = carry;
  __syncthreads();
  const int G = bad ? 0 : s_goff[B];
  const bool fits = G <= MG;
  if (tid == 0 && (bad || !fits)) set_status(a.status, kDevBadRows);
  const bool live = !bad && fits;
  auto req_of = [&](const int* arr, int x) {  // largest b with arr[b] <= x
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (arr[mid] <= x) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  // rows
  for (int r = tid; r < R; r += kRowsThreads) {
    int rq = -1, rl = 0;
    if (live && B > 0 && r < s_cu[B]) {
      const int b = req_of(s_cu, r);
      const int ql = s_cu[b + 1] - s_cu[b];
      const int sl = s_sl[b];
      if (sl >= ql) {
        rq = b;
        rl = sl - ql + 1 + (r - s_cu[b]);
      }
    }
    a.row_req[r] = rq;
    a.row_len[r] = rl;
  }
  for (int b = tid; b < B; b += kRowsThreads)
    if (live && s_sl[b] < s_cu[b + 1] - s_cu[b]) set_status(a.status, kDevBadRows);
  // groups: first row, request, causal blocks of the group's last (longest) row
  const int row_end = live ? s_cu[B] : 0;
  carry = 0;
  for (int base = 0; base < MG; base += kRowsThreads) {
    const int g = base + tid;
    int nblk = 0;
    if (g < MG) {
      int first = row_end, rq = -1;
      if (live && g < G) {
        const int b = req_of(s_goff, g);
        const int i = g - s_goff[b];
        const int q0 = s_cu[b], q1 = s_cu[b + 1];
        const int ql = q1 - q0, sl = s_sl[b];
        first = q0 + kGroupRows * i;
        rq = b;
        if (sl >= ql) {
          const int last = min(first + kGroupRows, q1) - 1;
          nblk = (sl - ql + 1 + (last - q0) + kPage - 1) / kPage;
        }
      }
      a.grp_row[g] = first;
      a.grp_req[g] = rq;
    }
    int tot;
    const int ex = block_exclusive_scan(nblk, s_scan, &tot);
    if (g < MG) a.req_blk[g] = carry + ex;
    carry += tot;
  }
  if (tid == 0) {
    a.req_blk[MG] = carry;
    a.grp_row[MG] = row_end;
  }
}

hipError_t launch_prefill_rows(const RowsArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(prefill_rows_kernel, dim3(1), dim3(kRowsThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode_rows(const RowsArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(decode_rows_kernel, dim3(1), dim3(kRowsThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace m3s
