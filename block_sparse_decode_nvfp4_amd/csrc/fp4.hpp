// Device helpers for the NVFP4 / MXFP4 decode path on gfx950 (MI355X).
//
// Formats ([ATOM-2744] Design / Write path and Follow-up: MXFP4 caches; see
// include/m3s.h for the source key): e2m1 codes (bit 3 sign, 2 exponent bits
// with bias 1, 1 mantissa bit), two per byte, element 2j in the low nibble;
// NVFP4 scales are OCP E4M3FN bytes (one per 16 elements), MXFP4 scales are
// E8M0 bytes (one per 32 elements).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m3s {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kPage = 128;
constexpr int kDim = 128;
constexpr int kPayload = 64;  // bytes of e2m1 codes per token

// Exact value of an OCP E4M3FN byte (the NaN byte is never produced by the store).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  uint32_t e = (b >> 3) & 0xFu, m = b & 7u;
  float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  return (b & 0x80u) ? -mag : mag;
}

// Exact value of an E8M0 byte: 2^(b - 127); byte 0 is the fp32 denormal 2^-127.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  return b ? __uint_as_float(b << 23) : __uint_as_float(0x00400000u);
}

// e2m1 -> fp16 decode.
//
// gfx950's scaled conversion (v_cvt_scalef32_pk_f16_fp4) applies only the
// exponent of its fp32 scale operand (checked on MI355X for all 16 codes x all
// 126 positive finite E4M3 scales: a non-power-of-two scale is truncated to
// its power of two). So an NVFP4 group is decoded with scale 1.0 and then
// multiplied by the E4M3 scale in fp16, which is exact: code * scale has at
// most 6 significant bits and lies in [2^-10, 2688]. An MXFP4 (E8M0) scale is
// a power of two and goes straight into the conversion.

// 8 codes of one dword (element e in bits [4e, 4e+4)) as fp16, unscaled.
__device__ __forceinline__ f16x8 fp4x8_to_f16_unscaled(uint32_t d) {
  f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0);
  f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1);
  f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2);
  f16x2 e = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3);
  f16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = e[0]; r[7] = e[1];
  return r;
}

// 8 codes times a power-of-two scale `p2` (an E8M0 byte as fp32: its exponent field is the
// byte), as bf16. bf16 has the fp32 exponent range, so code * 2^(b - 127) is exact for
// every scale byte a store writes (0 .. 252: at most 2 significant bits, magnitudes from
// 2^-128 to 1.5 * 2^127); 253 and 254 overflow to infinity. The conversion's handling of
// every code x every byte, subnormal results included, was checked on MI355X.
// The packed results are kept as raw dwords: extracting the bf16 elements of the
// builtin's bf16x2 result compiles to a permute that duplicates the low half.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16_pow2(uint32_t d, float p2) {
  const u32x4 r = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, p2, 0)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, p2, 1)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, p2, 2)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, p2, 3))};
  return __builtin_bit_cast(bf16x8, r);
}

// The two E4M3FN bytes in the low 16 bits of w as fp16 (byte 0 in element 0), in one
// hardware conversion: gfx950's fp8 conversion reads OCP E4M3FN, subnormals included, and
// every value it gives (2^-9 .. 448) converts to fp16 exactly, so the rounding mode of
// the narrowing does not matter.
__device__ __forceinline__ f16x2 e4m3x2_to_f16x2(uint32_t w) {
  const auto sf = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  return __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(sf[0], sf[1]));
}

// 8 codes of one dword times an E4M3 scale, as fp16 (exact).
__device__ __forceinline__ f16x8 fp4x8_to_f16_e4m3(uint32_t d, _Float16 s) {
  f16x8 r = fp4x8_to_f16_unscaled(d);
  f16x8 sv = {s, s, s, s, s, s, s, s};
  return r * sv;
}

// K / V decode of the attention. NVFP4 decodes to fp16 (code * E4M3 scale lies in
// [2^-10, 2688]: exact in fp16, whose 11-bit significand also keeps P to 2^-12); MXFP4
// decodes to bf16, the one 16-bit type whose range holds code * 2^(b - 127) for every
// E8M0 byte. op_t is the MFMA operand of 8 decoded elements.
template <int FMT>
struct Decode;
// scales(w, s0, s1): the scales of a lane's two 16-dim halves of its 32 dims, from the
// scale bytes it loaded (NVFP4: two E4M3 bytes, one per 16-element group; MXFP4: one E8M0
// byte for the whole 32-element group).
template <>
struct Decode<1> {  // NVFP4: scale byte is E4M3FN
  typedef _Float16 scale_t;
  typedef f16x8 op_t;
  static __device__ __forceinline__ void scales(uint32_t w, scale_t& s0, scale_t& s1) {
    const f16x2 s = e4m3x2_to_f16x2(w);
    s0 = s[0];
    s1 = s[1];
  }
  static __device__ __forceinline__ op_t run(uint32_t d, scale_t s) { return fp4x8_to_f16_e4m3(d, s); }
};
template <>
struct Decode<2> {  // MXFP4: scale byte is E8M0
  typedef float scale_t;
  typedef bf16x8 op_t;
  static __device__ __forceinline__ void scales(uint32_t w, scale_t& s0, scale_t& s1) {
    s0 = s1 = e8m0_to_f32(w);
  }
  static __device__ __forceinline__ op_t run(uint32_t d, scale_t s) { return fp4x8_to_bf16_pow2(d, s); }
};

// Scale of the 16-element (NVFP4) or 32-element (MXFP4) group as fp32.
template <int FMT>
__device__ __forceinline__ float scale_to_f32(uint32_t byte);
template <>
__device__ __forceinline__ float scale_to_f32<1>(uint32_t byte) { return e4m3_to_f32(byte); }
template <>
__device__ __forceinline__ float scale_to_f32<2>(uint32_t byte) { return e8m0_to_f32(byte); }

// 16x16x32 MFMA. Lane l holds A[l % 16][8 * (l / 16) + e] and B[8 * (l / 16) + e][l % 16]
// for e = 0..7; the result lane l holds D[4 * (l / 16) + v][l % 16] for v = 0..3.
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Cross-lane exchange with lane ^ M without the LDS crossbar: DPP quad_perm for
// M = 1, 2; two DPP mirrors for M = 4 (half_mirror then quad xor 3) and M = 8
// (row_mirror then half_mirror); gfx950's permlane16 / permlane32 swaps for
// M = 16, 32 (the swap returns the even and the odd row halves; the partner is
// the other half). Each pattern was checked lane by lane on MI355X.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, false);
}
template <int M>
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t x) {
  if constexpr (M == 1) return dpp_mov<0xB1>(x);
  else if constexpr (M == 2) return dpp_mov<0x4E>(x);
  else if constexpr (M == 4) return dpp_mov<0x1B>(dpp_mov<0x141>(x));
  else if constexpr (M == 8) return dpp_mov<0x141>(dpp_mov<0x140>(x));
  else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (threadIdx.x & 16) ? r[0] : r[1];
  } else {
    static_assert(M == 32, "lane_xor: M must be a power of two below 64");
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (threadIdx.x & 32) ? r[0] : r[1];
  }
}
template <int M>
__device__ __forceinline__ float lane_xor(float x) {
  return __uint_as_float(lane_xor_u32<M>(__float_as_uint(x)));
}
template <int M>
__device__ __forceinline__ int lane_xor(int x) {
  return (int)lane_xor_u32<M>((uint32_t)x);
}
template <int M>
__device__ __forceinline__ uint32_t lane_xor(uint32_t x) {
  return lane_xor_u32<M>(x);
}
template <int M>
__device__ __forceinline__ uint64_t lane_xor(uint64_t x) {
  return ((uint64_t)lane_xor_u32<M>((uint32_t)(x >> 32)) << 32) | lane_xor_u32<M>((uint32_t)x);
}
template <int M>
__device__ __forceinline__ double lane_xor(double x) {
  return __longlong_as_double((long long)lane_xor<M>((uint64_t)__double_as_longlong(x)));
}

// Butterfly reductions over the lanes whose index differs in bits LO..HI-1
// (e.g. <1, 16>: the 16 lanes of a row; <16, 64>: the four rows; <1, 64>: all).
// op must be commutative: at M = 16 and 32 the permlane swap hands every lane its own
// value and its partner's, in an order that depends on the lane, and op takes the two
// as they come (no select of the partner's half). A lane whose bit M is clear gets
// op(own, partner), as through lane_xor.
template <int LO, int HI, typename T, typename F>
__device__ __forceinline__ T lane_reduce(T x, F op) {
  if constexpr (LO < HI) {
    if constexpr ((LO == 16 || LO == 32) && sizeof(T) == 4) {
      const uint32_t u = __builtin_bit_cast(uint32_t, x);
      uint32_t a, b;
      if constexpr (LO == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        a = r[0];
        b = r[1];
      } else {
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        a = r[0];
        b = r[1];
      }
      x = op(__builtin_bit_cast(T, a), __builtin_bit_cast(T, b));
    } else {
      x = op(x, lane_xor<LO>(x));
    }
    return lane_reduce<LO * 2, HI>(x, op);
  } else {
    return x;
  }
}
template <int LO, int HI, typename T>
__device__ __forceinline__ T lane_max(T x) {
  return lane_reduce<LO, HI>(x, [](T a, T b) { return a > b ? a : b; });
}
template <int LO, int HI>
__device__ __forceinline__ float lane_fmax(float x) {
  return lane_reduce<LO, HI>(x, [](float a, float b) { return __builtin_fmaxf(a, b); });
}
template <int LO, int HI, typename T>
__device__ __forceinline__ T lane_sum(T x) {
  return lane_reduce<LO, HI>(x, [](T a, T b) { return a + b; });
}

__device__ __forceinline__ void set_status(uint32_t* status, uint32_t bit) {
  if (status) atomicOr(status, bit);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

}  // namespace m3s
