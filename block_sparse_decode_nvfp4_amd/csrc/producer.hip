// m3s_qknorm_rope_store: the fused producer store. Per token it RMS-normalizes
// and rotates the query heads, the key, the index query and the index key,
// writes the main query (bf16, and optionally e4m3) and the index query, and
// quantizes K, V and index K straight into the paged FP4 planes: no bf16
// staging buffer and no separate store launch.
//
// Pages: [ATOM-2744] Follow-up: MXFP4 caches (the quantization moves into the
// fused qk-norm / RoPE / cache kernel); [VLLM-64198] Claims (that kernel writes
// the K, V and index-K pages and the main query as e4m3). The pages define
// neither the norm nor the rotary embedding; this kernel computes
//   y = x / sqrt(mean(x^2) + eps) * w           (per 128-dim head row, fp32)
//   (y_d, y_{d+h}) -> (y_d c - y_{d+h} s, y_{d+h} c + y_d s),  d < h = rd / 2,
// with c, s from the caller's angle table at the token's position; the value
// is neither normed nor rotated. Each result row is rounded to bf16 (to
// nearest even), the row the unfused path would stage, and K / V / index K
// are quantized from those bf16 rows exactly as m3s_store quantizes (so the
// fused store writes the bytes the unfused one would for the same bf16 rows).
// The e4m3 query is the E4M3FN byte nearest to the bf16 query (ties to even,
// saturating at 448), with no scale.
//
// Layout of the work: the token's G + 4 rows (G query heads, key, value, index
// query, index key) are rows rr = token * (G + 4) + kind; 16 lanes per row, 8
// elements (one 16-byte load) per lane, 16 rows per 256-thread workgroup. Every
// lane runs the same instructions (the value's norm factor and weight are 1
// and its rotation is off), so the cross-lane exchanges of the norm, the
// rotation and the quantization see their whole 16-lane group.
#include "fp4.hpp"
#include "launch.hpp"
#include "quant.hpp"

namespace m3s {

// bf16 bits nearest to a finite float (ties to the even significand).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// OCP E4M3FN byte nearest to a bf16 value: ties to even, magnitudes past 448
// saturate to 448 (0x7E), sign bit = (value < 0). The input is exact in fp32,
// so the bit rounding below is the exact rounding.
__device__ __forceinline__ uint32_t e4m3_of_bf16(uint32_t h) {
  const uint32_t mag = h & 0x7FFFu;
  const float v = bf16_bits_to_f32(mag);
  uint32_t c;
  if (v < 0x1p-6f) {
    c = (uint32_t)__builtin_rintf(v * 512.0f);  // subnormal step 2^-9; 8 -> 0x08 = 2^-6
  } else {
    uint32_t u = mag << 16;
    u = u + 0x7FFFFu + ((u >> 20) & 1u);  // round the mantissa to 3 bits, ties to even
    c = (u >> 20) - (120u << 3);
  }
  c = c > 0x7Eu ? 0x7Eu : c;
  return c | (((h >> 15) & (mag != 0u ? 1u : 0u)) << 7);
}

template <int FMT>
__global__ __launch_bounds__(256) void producer_kernel(ProducerArgs a) {
  const int lane = threadIdx.x & 63;
  const int lane16 = threadIdx.x & 15;
  const int G = a.num_heads;
  const int nr = G + 4;
  const int64_t rr = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int64_t tok = rr / nr;
  const int kind = (int)(rr - tok * nr);  // [0, G) query heads, G key, G+1 value, G+2 index query, G+3 index key
  const bool is_v = kind == G + 1;
  const int wsel = kind < G ? 0 : (kind == G ? 1 : (kind == G + 2 ? 2 : 3));  // weight row (unused for v)

  // ---- every load of the row is independent: issued together
  bool live = tok < a.num_tokens;
  const int64_t t = live ? tok : 0;
  const int32_t pos = a.rotary_dim > 0 && live ? a.positions[t] : 0;
  const int32_t slot = live ? a.slots[t] : -1;
  const uint16_t* src = kind < G ? a.q + t * a.q_stride + (int64_t)kind * kDim
                                 : (kind == G ? a.k : (is_v ? a.v : (kind == G + 2 ? a.idx_q : a.idx_k))) +
                                       t * a.row_stride;
  const u32x4 raw = *reinterpret_cast<const u32x4*>(src + 8 * lane16);
  const u32x4 wraw = *reinterpret_cast<const u32x4*>(a.norm_w + wsel * kDim + 8 * lane16);

  // ---- rotation: lanes of dims [0, rd) pair with the lane h / 8 away
  const int rd = a.rotary_dim;
  const int hl = rd >> 4;  // lanes per half of the rotated dims
  const bool rot_lane = !is_v && lane16 < 2 * hl;
  const bool first_half = lane16 < hl;
  const bool pos_ok = rd == 0 || (pos >= 0 && pos < a.max_pos);
  f32x4 cs[4] = {{1.f, 1.f, 1.f, 1.f}, {1.f, 1.f, 1.f, 1.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  if (rot_lane && pos_ok && live) {
    const int i0 = first_half ? 8 * lane16 : 8 * lane16 - (rd >> 1);  // pair index of the lane's first element
    const float* row = a.cos_sin + (int64_t)pos * rd;
    cs[0] = *reinterpret_cast<const f32x4*>(row + i0);
    cs[1] = *reinterpret_cast<const f32x4*>(row + i0 + 4);
    cs[2] = *reinterpret_cast<const f32x4*>(row + (rd >> 1) + i0);
    cs[3] = *reinterpret_cast<const f32x4*>(row + (rd >> 1) + i0 + 4);
  }
  if (live && !pos_ok) {
    if (lane16 == 0) set_status(a.status, kDevBadPosition);
    live = false;  // the token's rows write nothing
  }

  float x[8], w[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_bits_to_f32(raw[i] & 0xFFFFu);
    x[2 * i + 1] = bf16_bits_to_f32(raw[i] >> 16);
    w[2 * i] = is_v ? 1.0f : bf16_bits_to_f32(wraw[i] & 0xFFFFu);
    w[2 * i + 1] = is_v ? 1.0f : bf16_bits_to_f32(wraw[i] >> 16);
  }

  // ---- RMS norm over the row's 16 lanes (the value keeps factor 1)
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
  ss = lane_sum<1, 16>(ss);
  const float r = is_v ? 1.0f : 1.0f / __builtin_sqrtf(ss * (1.0f / kDim) + a.eps);
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = x[e] * r * w[e];

  // ---- rotate-half: partner lane holds the other element of each pair
  if (rd > 0) {
    const int partner = (lane & ~15) + (first_half ? lane16 + hl : lane16 - hl);
    const int src_lane = rot_lane ? partner : lane;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = __shfl(y[e], src_lane, 64);
      const float c = cs[e >> 2][e & 3], s = cs[2 + (e >> 2)][e & 3];
      if (rot_lane) y[e] = first_half ? y[e] * c - p * s : y[e] * c + p * s;
    }
  }

  // ---- bf16 rows, then the outputs of each kind
  uint32_t bits[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) bits[e] = f32_to_bf16_rne(y[e]);
  if (live && (kind < G || kind == G + 2)) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = bits[2 * i] | (bits[2 * i + 1] << 16);
    uint16_t* dst = kind < G ? a.q_out + (t * G + kind) * kDim : a.idx_q_out + t * kDim;
    *reinterpret_cast<u32x4*>(dst + 8 * lane16) = o;
    if (kind < G && a.q_out_e4m3) {
      u32x2 e8;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        e8[i] = e4m3_of_bf16(bits[4 * i]) | (e4m3_of_bf16(bits[4 * i + 1]) << 8) |
                (e4m3_of_bf16(bits[4 * i + 2]) << 16) | (e4m3_of_bf16(bits[4 * i + 3]) << 24);
      *reinterpret_cast<u32x2*>(a.q_out_e4m3 + (t * G + kind) * kDim + 8 * lane16) = e8;
    }
  }
  uint32_t packed, scale_byte;
  quantize_lane<FMT>(bits, packed, scale_byte);  // every row: the group exchange needs all lanes
  const bool cache_row = kind == G || is_v || kind == G + 3;
  bool write = live && cache_row && slot >= 0;
  if (write && (int64_t)slot >= (int64_t)a.num_pages * kPage) {
    if (lane16 == 0) set_status(a.status, kDevBadSlot);
    write = false;
  }
  if (write) {
    uint8_t* dd = kind == G ? a.k_data : (is_v ? a.v_data : a.idx_data);
    uint8_t* ds = kind == G ? a.k_scale : (is_v ? a.v_scale : a.idx_scale);
    write_lane<FMT>(dd, ds, slot, lane16, packed, scale_byte);
  }
}

hipError_t launch_producer(const ProducerArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.num_tokens * (a.num_heads + 4);
  const int64_t grid = (rows + 15) / 16;
  if (grid == 0) return hipSuccess;
  if (a.format == 1)
    hipLaunchKernelGGL(producer_kernel<1>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(producer_kernel<2>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace m3s
