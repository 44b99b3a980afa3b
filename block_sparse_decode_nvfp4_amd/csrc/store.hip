// m3s_store: quantize the step's new K / V / index-K rows to NVFP4 or MXFP4
// and scatter them into the paged planes, one launch for all three tensors.
// The quantization rule and its exact rounding are in quant.hpp. Pad rows
// (slot < 0) are left unwritten ([ATOM-2744] Tests).
//
// Layout of the work: 16 lanes per 128-element row, 8 elements (one 16 B
// load) per lane; a 256-thread workgroup covers 16 rows; row index
// rr = token * 3 + tensor so a token's three rows sit in one workgroup.
#include "fp4.hpp"
#include "launch.hpp"
#include "quant.hpp"
#include "rows_body.hpp"
#include "store_body.hpp"

namespace m3s {

template <int FMT>
__global__ __launch_bounds__(256) void store_kernel(StoreArgs a) {
  store_body<FMT>(a, blockIdx.x);
}

// Store and decode row map in one launch: workgroups [0, store_grid) store, the
// last one builds the row map (the two are independent; one launch instead of
// two, each of which is mostly launch and first-load latency).
template <int FMT>
__global__ __launch_bounds__(256) void store_rows_kernel(StoreArgs s, RowsArgs r, int store_grid) {
  __shared__ int s_scan[256 / 64];
  if ((int)blockIdx.x < store_grid) store_body<FMT>(s, blockIdx.x);
  else decode_rows_body<256>(r, s_scan);
}

// Store and prefill row map in one launch: workgroups [0, store_grid) store, the last
// one builds the prefill row map and the 64-row groups (its LDS, prefill_rows_lds_bytes
// of the batch, is the launch's dynamic LDS).
template <int FMT>
__global__ __launch_bounds__(256) void store_prefill_rows_kernel(StoreArgs s, RowsArgs r, int store_grid) {
  extern __shared__ int s_pref[];
  if ((int)blockIdx.x < store_grid) store_body<FMT>(s, blockIdx.x);
  else prefill_rows_body<256>(r, s_pref);
}

hipError_t launch_store(const StoreArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.num_tokens * 3;
  const int64_t grid = (rows + 15) / 16;
  if (grid == 0) return hipSuccess;
  if (a.format == 1)
    hipLaunchKernelGGL(store_kernel<1>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(store_kernel<2>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_store_rows(const StoreArgs& s, const RowsArgs& r, hipStream_t stream) {
  const int64_t grid = ((int64_t)s.num_tokens * 3 + 15) / 16;
  if (s.format == 1)
    hipLaunchKernelGGL(store_rows_kernel<1>, dim3((unsigned)grid + 1), dim3(256), 0, stream, s, r, (int)grid);
  else
    hipLaunchKernelGGL(store_rows_kernel<2>, dim3((unsigned)grid + 1), dim3(256), 0, stream, s, r, (int)grid);
  return hipGetLastError();
}

hipError_t launch_store_prefill_rows(const StoreArgs& s, const RowsArgs& r, hipStream_t stream) {
  const int64_t grid = ((int64_t)s.num_tokens * 3 + 15) / 16;
  const size_t lds = prefill_rows_lds_bytes(r.num_reqs);
  if (s.format == 1)
    hipLaunchKernelGGL(store_prefill_rows_kernel<1>, dim3((unsigned)grid + 1), dim3(256), lds, stream, s, r, (int)grid);
  else
    hipLaunchKernelGGL(store_prefill_rows_kernel<2>, dim3((unsigned)grid + 1), dim3(256), lds, stream, s, r, (int)grid);
  return hipGetLastError();
}

}  // namespace m3s
