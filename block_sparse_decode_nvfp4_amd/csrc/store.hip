// m3s_store: quantize the step's new K / V / index-K rows to NVFP4 or MXFP4
// and scatter them into the paged planes, one launch for all three tensors.
//
// Rule ([ATOM-2744] Design / Write path): per 16 elements scale =
// e4m3(amax / 6), codes rounded half to even and saturating at 6. MXFP4
// ([ATOM-2744] Follow-up: MXFP4 caches): one E8M0 scale per 32 elements,
// taken as 2^(floor(log2 amax) - 2) (OCP MX v1.0). Pad rows (slot < 0) are
// left unwritten ([ATOM-2744] Tests).
//
// Every rounding decision is made exactly:
//   * amax is the integer max of the bf16 magnitude bits;
//   * the E4M3 scale is a candidate from amax / 6 corrected by exact compares
//     of amax against 6 * (midpoint of neighbouring E4M3 values); each such
//     product has at most 7 significant bits, so it is exact in fp32;
//   * a code is the number of e2m1 midpoints t * s (t = .25 .75 1.25 1.75
//     2.5 3.5 5) below |x|, where a tie goes to the even code; t * s has at
//     most 7 significant bits and is exact in fp32 (no reciprocal is used).
//
// Layout of the work: 16 lanes per 128-element row, 8 elements (one 16 B
// load) per lane; a 256-thread workgroup covers 16 rows; row index
// rr = token * 3 + tensor so a token's three rows sit in one workgroup.
#include "fp4.hpp"
#include "launch.hpp"
#include "rows_body.hpp"

namespace m3s {

// Nearest E4M3FN byte (ties to even, saturating at 448) of a / 6, a >= 0 finite.
__device__ __forceinline__ uint32_t e4m3_scale_of_amax(float a) {
  float y = a / 6.0f;
  uint32_t c;
  if (y >= 448.0f) {
    c = 0x7E;
  } else if (y < 0x1p-6f) {
    c = (uint32_t)__builtin_rintf(y * 512.0f);  // subnormal step 2^-9; 8 -> 0x08 = 2^-6
  } else {
    uint32_t u = __float_as_uint(y);
    u = u + 0x7FFFFu + ((u >> 20) & 1u);  // round the mantissa to 3 bits, ties to even
    c = (u >> 20) - (120u << 3);
    c = c > 0x7Eu ? 0x7Eu : c;
  }
  // y is within an ulp of a / 6, so the candidate is off by at most one step:
  // correct it against the exact midpoints (times 6).
  for (int it = 0; it < 2; ++it) {
    if (c > 0) {
      float mlo = 3.0f * (e4m3_to_f32(c - 1) + e4m3_to_f32(c));
      if (a < mlo || (a == mlo && (c & 1u))) { c -= 1; continue; }
    }
    if (c < 0x7E) {
      float mhi = 3.0f * (e4m3_to_f32(c) + e4m3_to_f32(c + 1));
      if (a > mhi || (a == mhi && (c & 1u))) { c += 1; continue; }
    }
    break;
  }
  return c;
}

// e2m1 magnitude index of |x| for scale s (s > 0): midpoints between codes
// i and i+1 are t_i * s; an exact tie goes to the even index.
__device__ __forceinline__ uint32_t e2m1_mag(float a, float s) {
  uint32_t m = 0;
  m += a > 0.25f * s;
  m += a >= 0.75f * s;
  m += a > 1.25f * s;
  m += a >= 1.75f * s;
  m += a > 2.5f * s;
  m += a >= 3.5f * s;
  m += a > 5.0f * s;
  return m;
}

// Sign bit of a code: x < 0 (so -0.0 gives a positive zero code, while a
// negative value that rounds to magnitude 0 keeps its sign bit).
__device__ __forceinline__ uint32_t neg(uint32_t bits) { return (bits >> 15) & ((bits & 0x7FFFu) != 0u); }

template <int FMT>
__device__ __forceinline__ void store_body(const StoreArgs& a, int64_t block) {
  const int lane16 = threadIdx.x & 15;
  const int64_t rr = block * 16 + (threadIdx.x >> 4);
  const int64_t tok = rr / 3;
  const int ten = (int)(rr - tok * 3);
  const uint16_t* src = ten == 0 ? a.k : (ten == 1 ? a.v : a.idx);
  uint8_t* dd = ten == 0 ? a.k_data : (ten == 1 ? a.v_data : a.idx_data);
  uint8_t* ds = ten == 0 ? a.k_scale : (ten == 1 ? a.v_scale : a.idx_scale);

  bool live = tok < a.num_tokens && src != nullptr;
  int32_t slot = live ? a.slots[tok] : -1;
  live = live && slot >= 0;
  if (live && (int64_t)slot >= (int64_t)a.num_pages * kPage) {
    if (lane16 == 0) set_status(a.status, 1u << 0);
    live = false;
  }
  u32x4 raw = {0u, 0u, 0u, 0u};
  if (live) raw = *reinterpret_cast<const u32x4*>(src + tok * a.row_stride + 8 * lane16);

  uint32_t bits[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bits[2 * i] = raw[i] & 0xFFFFu;
    bits[2 * i + 1] = raw[i] >> 16;
  }
  uint32_t amax = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = max(amax, bits[e] & 0x7FFFu);
  amax = max(amax, lane_xor<1>(amax));
  if (FMT == 2) amax = max(amax, lane_xor<2>(amax));

  uint32_t scale_byte;
  uint32_t packed = 0;
  if (FMT == 1) {
    const float af = bf16_bits_to_f32(amax);
    scale_byte = e4m3_scale_of_amax(af);
    const float s = e4m3_to_f32(scale_byte);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t mag = scale_byte ? e2m1_mag(bf16_bits_to_f32(bits[e] & 0x7FFFu), s) : 0u;
      packed |= ((neg(bits[e]) << 3) | mag) << (4 * e);
    }
  } else {
    int fl;  // floor(log2 amax) from the bf16 bits
    const uint32_t ex = amax >> 7, mant = amax & 0x7Fu;
    fl = ex ? (int)ex - 127 : (mant ? (31 - __builtin_clz(mant)) - 133 : 0);
    int byte = fl - 2 + 127;
    byte = byte < 0 ? 0 : (byte > 254 ? 254 : byte);
    scale_byte = amax ? (uint32_t)byte : 0u;
    const int shift = 127 - (int)scale_byte;  // x / 2^(byte-127)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float r = __builtin_ldexpf(bf16_bits_to_f32(bits[e] & 0x7FFFu), shift);
      uint32_t mag = amax ? e2m1_mag(r, 1.0f) : 0u;
      packed |= ((neg(bits[e]) << 3) | mag) << (4 * e);
    }
  }
  if (live) {
    *reinterpret_cast<uint32_t*>(dd + (int64_t)slot * kPayload + 4 * lane16) = packed;
    if (FMT == 1 && (lane16 & 1) == 0) ds[(int64_t)slot * 8 + (lane16 >> 1)] = (uint8_t)scale_byte;
    if (FMT == 2 && (lane16 & 3) == 0) ds[(int64_t)slot * 4 + (lane16 >> 2)] = (uint8_t)scale_byte;
  }
}

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

}  // namespace m3s
