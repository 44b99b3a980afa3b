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

// Exclusive scan of one value per thread over the workgroup; returns the
// thread's exclusive prefix, *total gets the sum. Uses s_scan (T / 64 ints).
template <int T>
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
    int w = lane < T / 64 ? s_scan[lane] : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(w, off, 64);
      if (lane >= off) w += y;
    }
    if (lane < T / 64) s_scan[lane] = w;  // inclusive wave totals
  }
  __syncthreads();
  const int excl = (wid ? s_scan[wid - 1] : 0) + x - v;
  *total = s_scan[T / 64 - 1];
  __syncthreads();  // s_scan is reused by the next scan
  return excl;
}

constexpr int kGroupRows = 64;  // rows per scan work group (four MFMA column tiles)

// LDS of prefill_rows_body for B requests: request offsets, lengths, group offsets,
// the scan's wave totals and a flag.
__host__ __device__ constexpr size_t prefill_rows_lds_bytes(int B) { return (size_t)(3 * B + 2 + 16 + 1) * sizeof(int); }

// Prefill row map and the scan's 64-row work groups, in one workgroup of T threads
// (the m3s_prefill_rows kernel, and the last workgroup of the store-and-prefill-rows
// launch). The request offsets, lengths and group offsets are staged in LDS (lds:
// prefill_rows_lds_bytes(num_reqs) bytes); every row and every group is then written
// by its own thread (a chunk of thousands of rows is not one thread's loop).
template <int T>
__device__ __forceinline__ void prefill_rows_body(const RowsArgs& a, int* lds) {
  const int tid = threadIdx.x;
  const int B = a.num_reqs, R = a.num_rows, MG = a.max_groups;
  int* s_cu = lds;
  int* s_sl = s_cu + (B + 1);
  int* s_goff = s_sl + B;
  int* s_scan = s_goff + (B + 1);
  int& s_bad = s_scan[16];
  if (tid == 0) s_bad = 0;
  for (int b = tid; b <= B; b += T) s_cu[b] = a.cu_q[b];
  for (int b = tid; b < B; b += T) s_sl[b] = a.seq_lens[b];
  __syncthreads();
  // the whole batch: cu_q must start at 0, never decrease and end within num_rows
  for (int b = tid; b < B; b += T)
    if (s_cu[b + 1] < s_cu[b]) atomicOr(&s_bad, 1);
  if (tid == 0 && (s_cu[0] != 0 || s_cu[B] > R)) atomicOr(&s_bad, 1);
  __syncthreads();
  const bool bad = s_bad != 0;
  // groups per request, then their offsets
  int carry = 0;
  for (int base = 0; base < B; base += T) {
    const int b = base + tid;
    const int ng = (!bad && b < B) ? (s_cu[b + 1] - s_cu[b] + kGroupRows - 1) / kGroupRows : 0;
    int tot;
    const int ex = block_exclusive_scan<T>(ng, s_scan, &tot);
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
  for (int r = tid; r < R; r += T) {
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
  for (int b = tid; b < B; b += T)
    if (live && s_sl[b] < s_cu[b + 1] - s_cu[b]) set_status(a.status, kDevBadRows);
  // groups: first row, request, causal blocks of the group's last (longest) row
  const int row_end = live ? s_cu[B] : 0;
  carry = 0;
  for (int base = 0; base < MG; base += T) {
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
    const int ex = block_exclusive_scan<T>(nblk, s_scan, &tot);
    if (g < MG) a.req_blk[g] = carry + ex;
    carry += tot;
  }
  if (tid == 0) {
    a.req_blk[MG] = carry;
    a.grp_row[MG] = row_end;
  }
}

}  // namespace m3s
