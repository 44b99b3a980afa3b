// m3s_probe_page_reads: a bandwidth ceiling for the index scan's access pattern. It
// reads whole 128-token pages (8 KB of codes + the page's scale bytes) the way the
// scan's waves do, and does nothing with them but fold them into one word per
// workgroup, so its time is the memory system's for that pattern alone. Used by the
// bench to measure the ceilings the scan is compared with; not part of the path.
//
// One 16-wave workgroup per CU; the waves claim pages one at a time from an LDS
// counter (as the scan does), each keeping one page in flight. Lane (n, G) of a wave
// loads, for i = 0..7, 16 B of token 16 i + n at byte 16 G of its 64 B row. Scales:
//   mode 0: 2 B per lane per 16-token tile (token 16 i + n, bytes 2G..2G+1), as the
//           NVFP4 scan loads them;
//   mode 1: one 16 B load per lane covering the whole 1 KB scale block of the page.
// Mode 2 is a plain stream for comparison: the first num_units pages of both planes
// (the same bytes as num_units pages) read front to back with 16-byte loads, every
// thread striding over the grid; the page list is not read.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "m3s.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(1024) void probe_kernel(const uint8_t* pay, const uint8_t* scl, const int32_t* pages,
                                                      int32_t num_units, int32_t mode, uint32_t* sink) {
  __shared__ int s_ctr;
  __shared__ uint32_t s_acc[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, G = lane >> 4;
  const int64_t u0 = (int64_t)blockIdx.x * num_units / gridDim.x;
  const int64_t u1 = (int64_t)(blockIdx.x + 1) * num_units / gridDim.x;
  const int cnt = (int)(u1 - u0);
  if (tid == 0) s_ctr = 0;
  __syncthreads();
  uint32_t acc = 0;
  while (true) {
    int v = 0;
    if (lane == 0) v = atomicAdd(&s_ctr, 1);
    const int i0 = __builtin_amdgcn_readlane(v, 0);
    if (i0 >= cnt) break;
    const int64_t page = pages[u0 + i0];
    const uint8_t* p = pay + page * (128 * 64);
    const uint8_t* s = scl + page * (128 * 8);
    u32x4 kr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) kr[i] = *reinterpret_cast<const u32x4*>(p + (16 * i + n) * 64 + 16 * G);
    uint32_t x = 0;
    if (mode == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) x ^= *reinterpret_cast<const uint16_t*>(s + (16 * i + n) * 8 + 2 * G);
    } else {
      const u32x4 sv = *reinterpret_cast<const u32x4*>(s + 16 * lane);
      x = sv[0] ^ sv[1] ^ sv[2] ^ sv[3];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) x ^= kr[i][0] ^ kr[i][1] ^ kr[i][2] ^ kr[i][3];
    acc ^= x;
  }
  // fold: one word per wave, then per workgroup
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= __shfl_xor(acc, m, 64);
  if (lane == 0) s_acc[w] = acc;
  __syncthreads();
  if (tid == 0) {
    uint32_t t = 0;
    for (int i = 0; i < 16; ++i) t ^= s_acc[i];
    sink[blockIdx.x] = t;
  }
}

__global__ __launch_bounds__(1024) void stream_kernel(const u32x4* pay, const u32x4* scl, int64_t n_pay,
                                                       int64_t n_scl, uint32_t* sink) {
  __shared__ uint32_t s_acc[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + tid; i < n_pay; i += stride) {
    const u32x4 v = pay[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + tid; i < n_scl; i += stride) {
    const u32x4 v = scl[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= __shfl_xor(acc, m, 64);
  if (lane == 0) s_acc[w] = acc;
  __syncthreads();
  if (tid == 0) {
    uint32_t t = 0;
    for (int i = 0; i < 16; ++i) t ^= s_acc[i];
    sink[blockIdx.x] = t;
  }
}

}  // namespace

extern "C" m3s_status m3s_probe_page_reads(const uint8_t* payload, const uint8_t* scales, const int32_t* pages,
                                           int32_t num_units, int32_t mode, uint32_t* sink, int32_t num_sink,
                                           hipStream_t stream) {
  if (!payload || !scales || !pages || !sink || num_units < 0 || mode < 0 || mode > 2 || num_sink < 1)
    return M3S_ERR_INVALID_ARG;
  if (num_units == 0) return M3S_OK;
  if (mode == 2) {
    hipLaunchKernelGGL(stream_kernel, dim3((unsigned)num_sink), dim3(1024), 0, stream,
                       reinterpret_cast<const u32x4*>(payload), reinterpret_cast<const u32x4*>(scales),
                       (int64_t)num_units * (128 * 64 / 16), (int64_t)num_units * (128 * 8 / 16), sink);
    return hipGetLastError() == hipSuccess ? M3S_OK : M3S_ERR_HIP;
  }
  hipLaunchKernelGGL(probe_kernel, dim3((unsigned)num_sink), dim3(1024), 0, stream, payload, scales, pages,
                     num_units, mode, sink);
  return hipGetLastError() == hipSuccess ? M3S_OK : M3S_ERR_HIP;
}
