// Exact NVFP4 / MXFP4 quantization of one 128-element bf16 row held by 16
// consecutive lanes (8 elements, one 16-byte load, per lane), shared by the
// store and the fused producer store.
//
// Rule ([ATOM-2744] Design / Write path): per 16 elements scale =
// e4m3(amax / 6), codes rounded half to even and saturating at 6. MXFP4
// ([ATOM-2744] Follow-up: MXFP4 caches): one E8M0 scale per 32 elements,
// taken as 2^(floor(log2 amax) - 2) (OCP MX v1.0).
//
// Every rounding decision is made exactly:
//   * amax is the integer max of the bf16 magnitude bits;
//   * the E4M3 scale is a candidate from amax / 6 corrected by exact compares
//     of amax against 6 * (midpoint of neighbouring E4M3 values); each such
//     product has at most 7 significant bits, so it is exact in fp32;
//   * a code is the number of e2m1 midpoints t * s (t = .25 .75 1.25 1.75
//     2.5 3.5 5) below |x|, where a tie goes to the even code; t * s has at
//     most 7 significant bits and is exact in fp32 (no reciprocal is used).
#pragma once

#include "fp4.hpp"

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

// Codes (packed, element e in bits [4e, 4e+4)) and the scale byte of the
// lane's 8 elements. Every lane of the row's 16-lane group must call it (the
// group's amax is exchanged across lanes).
template <int FMT>
__device__ __forceinline__ void quantize_lane(const uint32_t (&bits)[8], uint32_t& packed, uint32_t& scale_byte) {
  uint32_t amax = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = max(amax, bits[e] & 0x7FFFu);
  amax = max(amax, lane_xor<1>(amax));
  if (FMT == 2) amax = max(amax, lane_xor<2>(amax));
  packed = 0;
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
}

// Write the lane's codes and (from the lanes that own one) its scale byte at a slot.
template <int FMT>
__device__ __forceinline__ void write_lane(uint8_t* dd, uint8_t* ds, int64_t slot, int lane16, uint32_t packed,
                                           uint32_t scale_byte) {
  *reinterpret_cast<uint32_t*>(dd + slot * kPayload + 4 * lane16) = packed;
  if (FMT == 1 && (lane16 & 1) == 0) ds[slot * 8 + (lane16 >> 1)] = (uint8_t)scale_byte;
  if (FMT == 2 && (lane16 & 3) == 0) ds[slot * 4 + (lane16 >> 2)] = (uint8_t)scale_byte;
}

}  // namespace m3s
