// m3s_index_topk: block scores of every causal 128-token block of every row
// against the FP4 index cache, then each row's top-k block ids.
//
// Pages: [ATOM-2744] Design (Index: the scorers read the FP4 plane through an
// e2m1 -> fp16 decode; Decode score grid: a (chunk, request) order, because
// workgroups go to the 8 XCDs round-robin by linear id and a request-fastest
// order pins each request to one XCD; Fused verify top-k: ids only, ascending),
// and the review notes on equal-score ties.
//
// Score of block j for a row: max over tokens t of block j, t < row_len, of
// q_idx . dequant(idx[t]).
//
// Two kernels:
//   scan   - the (request, block) units of all requests are one flat list,
//            block fastest inside a request; each workgroup takes a contiguous
//            slice of it, so a long request spreads over every XCD. A wave
//            scores one 128-token page against all <= 16 rows of its request
//            with fp16 MFMA (K tile as A, queries as B, fp32 accumulate) and
//            writes, per row, the block's fp32 score and a rigorous bound on
//            its error.
//   select - one workgroup per row: the k-th and (k+1)-th best fp32 scores by
//            (score, id), from a threshold on per-wave sorted maxima and one
//            sort of the keys above it; then certify: a block whose rank the
//            error bound leaves open is rescored in exact float64 and the open
//            slots are filled from those exact scores. The result is the
//            selection that exact arithmetic makes.
//
// Error bound of the scan (per row and block). The query row is scaled by a
// power of two 2^P (exact) and rounded to fp16 (error e_d, computed exactly);
// every product q'_d * k_d is exact in fp32 (<= 11 + 6 significant bits). For
// any order of fp32 additions with relative error <= 2^-23 each, the sum of
// 128 products is off by at most 127 * 2^-23 * sum |q'_d k_d| < 2^-16 * sum.
// With |k_d| <= 6 * smax_g (smax_g = the block's largest scale of group g):
//   |s' - exact'| <= sum_g 6 * smax_g * (2^-15 * Q'_g + E_g),
// Q'_g = sum over group g of |q'_d|, E_g = sum of e_d (2x margin on 2^-16).
#include <float.h>
#include <limits.h>

#include <type_traits>

#include "fp4.hpp"
#include "launch.hpp"
#include "attend_body.hpp"
#include "rows_body.hpp"
#include "store_body.hpp"

namespace m3s {

constexpr float kAccRel = 0x1p-15f;
constexpr int M3S_MAX_REQS_INTERNAL = 4096;

__device__ __forceinline__ uint32_t ord_f32(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);  // -0.0 -> +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord_f32(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// floor(log2 |x|) of a non-zero bf16 magnitude given as bits
__device__ __forceinline__ int bf16_floor_log2(uint32_t m) {
  const uint32_t ex = m >> 7, mant = m & 0x7Fu;
  return ex ? (int)ex - 127 : (31 - __builtin_clz(mant)) - 133;
}

// ---------------------------------------------------------------------------
// scan
// ---------------------------------------------------------------------------
// One 128-token page of the index cache, as the lanes of a wave hold it:
// lane (G, t) has token 16 i + t, dims [32 G, 32 G + 32) of tile i.
struct PageBuf {
  u32x4 kr[8];
  uint32_t ks[8];
};

template <int FMT>
__device__ __forceinline__ void load_page(PageBuf& p, const IndexArgs& a, int page, int n, int G) {
  constexpr int SB = FMT == 1 ? 8 : 4;
  const uint8_t* pay = a.idx_data + (int64_t)page * (kPage * kPayload);
  const uint8_t* scb = a.idx_scale + (int64_t)page * (kPage * SB);
#pragma unroll
  for (int i = 0; i < 8; ++i) p.kr[i] = *reinterpret_cast<const u32x4*>(pay + (16 * i + n) * kPayload + 16 * G);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (FMT == 1) p.ks[i] = *reinterpret_cast<const uint16_t*>(scb + (16 * i + n) * SB + 2 * G);
    else p.ks[i] = scb[(16 * i + n) * SB + G];
  }
}

// Per-request query state of a wave (rows r0 .. r0 + ql - 1 of request b).
// NVFP4: op = the row's 2^P-scaled fp16 query (B operand of the f16 MFMA).
// MXFP4: qb[t] / qsc[t] = term t of the query as e4m3 bytes with its E8M0 scale
// (B operand of the scaled fp4 MFMA).
struct QueryTile {
  f16x8 op[4];
  i32x8 qb[3];
  int qsc[3];
  float qs0, qs1, qe0, qe1, unscale;
  int b, r0, ql, len_n, min_len;
};

// MXFP4 query: the B operand of v_mfma_scale_f32_16x16x128_f8f6f4 in e4m3 holds, in
// lane (n, G), column (row) n with dims [16 G, 16 G + 16) in bytes 0-15 and
// [64 + 16 G, 64 + 16 G + 16) in bytes 16-31; the lane's scale is that of row n,
// dims [32 G, 32 G + 32) (layout measured on gfx950). Each 32-dim block of the
// bf16 row, with largest magnitude in [2^e, 2^(e+1)), is written as
//   q = 2^s1 t1 + 2^s2 t2 + 2^s3 t3 + r,  s1 = e - 3, s2 = s1 - 5, s3 = s2 - 5,
// each t an integer in [-16, 16] (exact in e4m3) taken by round-to-nearest of
// what the earlier terms leave, and r the exact remainder (|r| <= 2^(s3 - 1)).
// With integer-valued e4m3 operands the scaled MFMA accumulates like fp32 (its
// error on full-range e4m3 operands is far larger, which this split avoids).
// qs0 = sum over the lane's scale block of |2^s t| over the three terms and
// qe0 = sum of |r|: the scorer's error bound is 6 smax (2^-15 qs0 + qe0) per
// block, the 2^-15 covering any order of the <= 383 fp32 additions of the three
// chained MFMAs (383 * 2^-24 < 2^-15).
__device__ __forceinline__ void query_from_raw_mx(QueryTile& q, const u32x4 (&raw)[4], int n, int G) {
  // half 0 (raw[0..1]) lies in block G / 2, half 1 (raw[2..3]) in block 2 + G / 2;
  // lanes G and G ^ 1 hold the two halves of each block
  uint32_t mh[2] = {0u, 0u};
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int w = 0; w < 4; ++w) mh[s >> 1] = max(mh[s >> 1], max(raw[s][w] & 0x7FFFu, (raw[s][w] >> 16) & 0x7FFFu));
  int s1h[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t m = max(mh[h], lane_xor<16>(mh[h]));
    s1h[h] = m ? max(bf16_floor_log2(m) - 3, -127) : 0;
  }
  float qabs[2] = {0.f, 0.f}, qres[2] = {0.f, 0.f};
  int words[2][4][3];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int h = s >> 1;
    const int sc1 = s1h[h], sc2 = max(sc1 - 5, -127), sc3 = max(sc2 - 5, -127);
#pragma unroll
    for (int w = 0; w < 4; w += 2) {
      float t[3][4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t word = raw[s][w + (e >> 1)];
        float x = bf16_bits_to_f32((e & 1) ? (word >> 16) : (word & 0xFFFFu));
        const float t1 = __builtin_rintf(__builtin_ldexpf(x, -sc1));
        x -= __builtin_ldexpf(t1, sc1);
        const float t2 = __builtin_rintf(__builtin_ldexpf(x, -sc2));
        x -= __builtin_ldexpf(t2, sc2);
        const float t3 = __builtin_rintf(__builtin_ldexpf(x, -sc3));
        x -= __builtin_ldexpf(t3, sc3);
        t[0][e] = t1;
        t[1][e] = t2;
        t[2][e] = t3;
        qabs[h] += __builtin_ldexpf(fabsf(t1), sc1) + __builtin_ldexpf(fabsf(t2), sc2) + __builtin_ldexpf(fabsf(t3), sc3);
        qres[h] += fabsf(x);
      }
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        int v = __builtin_amdgcn_cvt_pk_fp8_f32(t[k][0], t[k][1], 0, false);
        v = __builtin_amdgcn_cvt_pk_fp8_f32(t[k][2], t[k][3], v, true);
        words[h][(s & 1) * 2 + (w >> 1)][k] = v;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 3; ++k) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      q.qb[k][d] = words[0][d][k];
      q.qb[k][4 + d] = words[1][d][k];
    }
  }
  // the lane supplies the scale (and takes the bound sums) of block G: block G < 2
  // is half 0 of lanes 2G, 2G + 1; block G >= 2 is half 1 of lanes 2G - 4, 2G - 3
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    qabs[h] += lane_xor<16>(qabs[h]);
    qres[h] += lane_xor<16>(qres[h]);
  }
  const int src = n + 16 * ((2 * G) & 3);
  const int e0 = __shfl(s1h[0], src, 64), e1 = __shfl(s1h[1], src, 64);
  const float a0 = __shfl(qabs[0], src, 64), a1 = __shfl(qabs[1], src, 64);
  const float r0 = __shfl(qres[0], src, 64), r1 = __shfl(qres[1], src, 64);
  const int sc1 = G < 2 ? e0 : e1;
  const int sc2 = max(sc1 - 5, -127), sc3 = max(sc2 - 5, -127);
  q.qsc[0] = sc1 + 127;
  q.qsc[1] = sc2 + 127;
  q.qsc[2] = sc3 + 127;
  q.qs0 = G < 2 ? a0 : a1;
  q.qe0 = G < 2 ? r0 : r1;
  q.qs1 = q.qe1 = 0.f;
  q.unscale = 1.0f;
}

// Lane (n, G)'s share of query row `row` (zeros when row < 0), as the B operand
// takes it: NVFP4 dims [32 G, 32 G + 32); MXFP4 dims [16 G, 16 G + 16) and
// [64 + 16 G, 64 + 16 G + 16).
template <int FMT>
__device__ __forceinline__ void query_raw(u32x4 (&raw)[4], const IndexArgs& a, int row, int G) {
#pragma unroll
  for (int s = 0; s < 4; ++s) raw[s] = u32x4{0u, 0u, 0u, 0u};
  if (row >= 0) {
    const uint16_t* qp = a.q_idx + (int64_t)row * a.q_stride;
    if (FMT == 1) {
#pragma unroll
      for (int s = 0; s < 4; ++s) raw[s] = *reinterpret_cast<const u32x4*>(qp + 32 * G + 8 * s);
    } else {
      raw[0] = *reinterpret_cast<const u32x4*>(qp + 16 * G);
      raw[1] = *reinterpret_cast<const u32x4*>(qp + 16 * G + 8);
      raw[2] = *reinterpret_cast<const u32x4*>(qp + 64 + 16 * G);
      raw[3] = *reinterpret_cast<const u32x4*>(qp + 64 + 16 * G + 8);
    }
  }
}

// query_raw from a copy of the row in LDS (qs: the row's 128 bf16 values).
template <int FMT>
__device__ __forceinline__ void query_raw_lds(u32x4 (&raw)[4], const uint16_t* qs, int G) {
  if (FMT == 1) {
#pragma unroll
    for (int s = 0; s < 4; ++s) raw[s] = *reinterpret_cast<const u32x4*>(qs + 32 * G + 8 * s);
  } else {
    raw[0] = *reinterpret_cast<const u32x4*>(qs + 16 * G);
    raw[1] = *reinterpret_cast<const u32x4*>(qs + 16 * G + 8);
    raw[2] = *reinterpret_cast<const u32x4*>(qs + 64 + 16 * G);
    raw[3] = *reinterpret_cast<const u32x4*>(qs + 64 + 16 * G + 8);
  }
}

// The B operand built from the lane's share of its row (query_raw), with the sums
// the error bound needs. Lanes n of one 16-lane column share a row.
template <int FMT>
__device__ __forceinline__ void query_from_raw(QueryTile& q, const u32x4 (&raw)[4], int n, int G) {
  if (FMT == 2) {
    query_from_raw_mx(q, raw, n, G);
    return;
  }
  uint32_t mx = 0;
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int w = 0; w < 4; ++w) mx = max(mx, max(raw[s][w] & 0x7FFFu, (raw[s][w] >> 16) & 0x7FFFu));
  mx = lane_max<16, 64>(mx);
  int P = mx ? 13 - bf16_floor_log2(mx) : 0;
  P = P > 64 ? 64 : (P < -64 ? -64 : P);
  q.unscale = __builtin_ldexpf(1.0f, -P);
  q.qs0 = q.qs1 = q.qe0 = q.qe1 = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t bits = (e & 1) ? (raw[s][e >> 1] >> 16) : (raw[s][e >> 1] & 0xFFFFu);
      const float x = __builtin_ldexpf(bf16_bits_to_f32(bits), P);
      const _Float16 h = (_Float16)x;
      const float err = fabsf(x - (float)h);
      q.op[s][e] = h;
      if (FMT == 1 && s >= 2) { q.qs1 += fabsf((float)h); q.qe1 += err; }
      else { q.qs0 += fabsf((float)h); q.qe0 += err; }
    }
  }
}

// The B operand of query row `row` (or zeros when row < 0) in lane (n, G).
template <int FMT>
__device__ __forceinline__ void build_query(QueryTile& q, const IndexArgs& a, int row, int n, int G) {
  u32x4 raw[4];
  query_raw<FMT>(raw, a, row, G);
  query_from_raw<FMT>(q, raw, n, G);
}

// The rows of query tile k of work group b, given g0 = cu_q[b] and g1 = cu_q[b + 1]:
// rows g0 + 16 k .. (at most 16, fewer at the group's end), and their causal lengths,
// from the row map, or in closed form for the decode step (its row map is written
// by the same launch): row r of request b sees step_base + r tokens, step_base =
// seq_len - q_len + 1 - cu_q[b].
__device__ __forceinline__ void query_rows(QueryTile& q, const IndexArgs& a, int b, int k, int g0, int g1,
                                           bool closed, int step_base, int n) {
  q.b = b;
  q.r0 = g0 + 16 * k;
  q.ql = min(max(g1 - q.r0, 0), 16);
  if (closed) {
    q.min_len = q.ql > 0 ? step_base + q.r0 : 0x7FFFFFFF;
    q.len_n = n < q.ql ? step_base + q.r0 + n : 0;
  } else {
    q.min_len = q.ql > 0 ? a.row_len[q.r0] : 0x7FFFFFFF;
    q.len_n = n < q.ql ? a.row_len[q.r0 + n] : 0;
  }
}

// Query tile k of work group b: the group's rows 16 k .. 16 k + 15 (fewer at its end).
template <int FMT>
__device__ __forceinline__ void load_query(QueryTile& q, const IndexArgs& a, int b, int k, int n, int G) {
  const int g0 = a.cu_q[b], g1 = a.cu_q[b + 1];
  const bool closed = a.seq_lens != nullptr;
  query_rows(q, a, b, k, g0, g1, closed, closed ? a.seq_lens[b] - (g1 - g0) + 1 - g0 : 0, n);
  build_query<FMT>(q, a, n < q.ql ? q.r0 + n : -1, n, G);
}

// NVFP4 K tile i of a page as the MFMA A operand (kd[c]: k-step c) and its two scales.
// The tile's words are pinned where the decode starts, so that a caller's order of
// decodes is kept (each decoded tile holds 16 registers).
__device__ __forceinline__ void decode_tile_nv(const PageBuf& p, int i, f16x8 (&kd)[4], f16x2& sc) {
  u32x4 kw = p.kr[i];
  uint32_t ksw = p.ks[i];
  asm volatile("" : "+v"(kw), "+v"(ksw));
  const auto sf = __builtin_amdgcn_cvt_pk_f32_fp8((int)ksw, false);
  sc = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(sf[0], sf[1]));
  const f16x8 s0 = {sc[0], sc[0], sc[0], sc[0], sc[0], sc[0], sc[0], sc[0]};
  const f16x8 s1 = {sc[1], sc[1], sc[1], sc[1], sc[1], sc[1], sc[1], sc[1]};
#pragma unroll
  for (int c = 0; c < 4; ++c) kd[c] = fp4x8_to_f16_unscaled(kw[c]) * (c < 2 ? s0 : s1);
}

// S^T tile i of a page against NT query tiles: acc[k][v] = (scaled) score of
// token 16 i + 4 G + v against the query in column n (lane (n, G)) of tile k.
// The K tile is decoded once for all NT tiles, and each column's result is the
// same as with that tile alone (columns of an MFMA do not interact). NVFP4 also
// returns the tile's scales.
template <int FMT, int NT>
__device__ __forceinline__ void tile_scores_n(const PageBuf& p, const QueryTile (&q)[NT], int i, f16x2& sc,
                                              f32x4 (&acc)[NT]) {
#pragma unroll
  for (int k = 0; k < NT; ++k) acc[k] = {0.f, 0.f, 0.f, 0.f};
  // pin the tile's words here: keeps the compiler from decoding every tile of the
  // page ahead of the MFMAs (each decoded tile holds 20+ registers)
  u32x4 kw = p.kr[i];
  uint32_t ksw = p.ks[i];
  asm volatile("" : "+v"(kw), "+v"(ksw));
  if (FMT == 1) {
    // both E4M3 scales of the lane's two groups in one conversion (OCP E4M3FN, exact)
    const auto sf = __builtin_amdgcn_cvt_pk_f32_fp8((int)ksw, false);
    sc = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(sf[0], sf[1]));
    const f16x8 s0 = {sc[0], sc[0], sc[0], sc[0], sc[0], sc[0], sc[0], sc[0]};
    const f16x8 s1 = {sc[1], sc[1], sc[1], sc[1], sc[1], sc[1], sc[1], sc[1]};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f16x8 kd = fp4x8_to_f16_unscaled(kw[c]) * (c < 2 ? s0 : s1);
#pragma unroll
      for (int k = 0; k < NT; ++k) acc[k] = mfma_f16(kd, q[k].op[c], acc[k]);
    }
  } else {
    // the lane's 32 codes and E8M0 byte are the fp4 A operand and its scale as loaded
    const i32x8 ka = {(int)kw[0], (int)kw[1], (int)kw[2], (int)kw[3], 0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
      for (int k = 0; k < NT; ++k)
        acc[k] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, q[k].qb[t], acc[k], 4, 0, 0, (int)ksw, 0,
                                                                  q[k].qsc[t]);
  }
}

// S^T tile i of a page: acc[v] = (scaled) score of token 16 i + 4 G + v against
// the query in column n (lane (n, G)); NVFP4 also returns the tile's scales.
template <int FMT>
__device__ __forceinline__ f32x4 tile_scores(const PageBuf& p, const QueryTile& q, int i, f16x2& sc) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (FMT == 1) {
    // both E4M3 scales of the lane's two groups in one conversion (OCP E4M3FN, exact)
    const auto sf = __builtin_amdgcn_cvt_pk_f32_fp8((int)p.ks[i], false);
    sc = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(sf[0], sf[1]));
    const f16x8 s0 = {sc[0], sc[0], sc[0], sc[0], sc[0], sc[0], sc[0], sc[0]};
    const f16x8 s1 = {sc[1], sc[1], sc[1], sc[1], sc[1], sc[1], sc[1], sc[1]};
    acc = mfma_f16(fp4x8_to_f16_unscaled(p.kr[i][0]) * s0, q.op[0], acc);
    acc = mfma_f16(fp4x8_to_f16_unscaled(p.kr[i][1]) * s0, q.op[1], acc);
    acc = mfma_f16(fp4x8_to_f16_unscaled(p.kr[i][2]) * s1, q.op[2], acc);
    acc = mfma_f16(fp4x8_to_f16_unscaled(p.kr[i][3]) * s1, q.op[3], acc);
  } else {
    // the lane's 32 codes and E8M0 byte are the fp4 A operand and its scale as loaded
    const i32x8 ka = {(int)p.kr[i][0], (int)p.kr[i][1], (int)p.kr[i][2], (int)p.kr[i][3], 0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < 3; ++t)
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, q.qb[t], acc, 4, 0, 0, (int)p.ks[i], 0, q.qsc[t]);
  }
  return acc;
}

// Largest of each half of a packed fp16 pair over the 16 lanes of a row (one packed max
// per exchange instead of two fp32 reductions).
__device__ __forceinline__ f16x2 row_max_f16x2(f16x2 v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  u = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(f16x2, u),
                                                              __builtin_bit_cast(f16x2, lane_xor_u32<1>(u))));
  u = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(f16x2, u),
                                                              __builtin_bit_cast(f16x2, lane_xor_u32<2>(u))));
  u = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(f16x2, u),
                                                              __builtin_bit_cast(f16x2, lane_xor_u32<4>(u))));
  u = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(f16x2, u),
                                                              __builtin_bit_cast(f16x2, lane_xor_u32<8>(u))));
  return __builtin_bit_cast(f16x2, u);
}

// Four per-lane values x[k] reduced over the wave's four rows (op commutative), so that
// row G ends with the result for k = G: a reduce-scatter of two swap steps (three swaps,
// three ops) instead of a butterfly per value. The permlane32 swap exchanges the upper
// half of its first operand with the lower half of its second, the permlane16 swap the
// odd rows of its first with the even rows of its second.
template <typename F>
__device__ __forceinline__ float rows_reduce_scatter4(float x0, float x1, float x2, float x3, F op) {
  const float x[4] = {x0, x1, x2, x3};
  auto swap32 = [](float a, float b, float& lo, float& hi) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
  };
  float a0, a1, b0, b1;
  swap32(x[0], x[2], a0, a1);  // lanes 0-31: x[0] of rows 0-1 and of rows 2-3; lanes 32-63: x[2]
  swap32(x[1], x[3], b0, b1);  // the same for x[1] / x[3]
  const float m02 = op(a0, a1), m13 = op(b0, b1);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(m02), __float_as_uint(m13), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Score one page against the request's rows; write the fp32 score and error bound.
template <int FMT>
__device__ __forceinline__ void score_page(const PageBuf& p, const QueryTile& q, const IndexArgs& a, int j, int n,
                                           int G) {
  const bool need_mask = (j + 1) * kPage > q.min_len;
  float run = -INFINITY;
  f16x2 smx = {(_Float16)0.f, (_Float16)0.f};  // largest scale of groups (2G, 2G+1) seen by this lane
  float smx_mx = 0.f;                          // MXFP4: largest E8M0 scale of group G
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f16x2 sc;
    f32x4 acc = tile_scores<FMT>(p, q, i, sc);
    if (FMT == 1) smx = __builtin_elementwise_max(smx, sc);
    else smx_mx = fmaxf(smx_mx, e8m0_to_f32(p.ks[i]));
    if (need_mask) {
      const int t0 = j * kPage + 16 * i + 4 * G;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (t0 + v >= q.len_n) acc[v] = -INFINITY;
    }
    run = __builtin_fmaxf(__builtin_fmaxf(run, acc[0]), acc[1]);
    run = __builtin_fmaxf(__builtin_fmaxf(run, acc[2]), acc[3]);
  }
  run = lane_fmax<16, 64>(run);
  float part;
  if (FMT == 1) {
    const f16x2 sm = row_max_f16x2(smx);
    const float m0 = (float)sm[0], m1 = (float)sm[1];
    part = 6.0f * (m0 * (kAccRel * q.qs0 + q.qe0) + m1 * (kAccRel * q.qs1 + q.qe1));
  } else {
    const float m0 = lane_fmax<1, 16>(smx_mx);
    part = 6.0f * m0 * (kAccRel * q.qs0 + q.qe0);
  }
  part = lane_sum<16, 64>(part);
  if (G == 0 && n < q.ql) {
    const int64_t o = (int64_t)(q.r0 + n) * a.max_blocks + j;
    a.ws_score[o] = run * q.unscale;
    a.ws_bound[o] = part * q.unscale * (1.0f + 0x1p-10f);
  }
}

// Score one page against the work group's rows (NT query tiles); write each
// row's fp32 score and error bound.
template <int FMT, int NT>
__device__ __forceinline__ void score_page_n(const PageBuf& p, const QueryTile (&q)[NT], const IndexArgs& a, int j,
                                             int n, int G) {
  bool need_mask[NT];
  float run[NT];
#pragma unroll
  for (int k = 0; k < NT; ++k) {
    need_mask[k] = (j + 1) * kPage > q[k].min_len;
    run[k] = -INFINITY;
  }
  f16x2 smx = {(_Float16)0.f, (_Float16)0.f};  // largest scale of groups (2G, 2G+1) seen by this lane
  float smx_mx = 0.f;                          // MXFP4: largest E8M0 scale of group G
  // NVFP4: tile i + 1 is decoded (VALU) while tile i's NT x 4 MFMAs run, one tile ahead
  f16x8 kd[4], kn[4];
  f16x2 sc_cur, sc_next;
  if constexpr (FMT == 1) decode_tile_nv(p, 0, kd, sc_cur);
  // the tiles, with or without the causal mask: a block needs it only where a row's
  // length ends inside it, and compiled into one loop the mask's compares and selects
  // ran on every tile (a quarter of the loop's arithmetic)
  bool any_mask = false;
#pragma unroll
  for (int k = 0; k < NT; ++k) any_mask |= need_mask[k];
  auto tiles = [&](auto masked) {
  constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f16x2 sc;
    f32x4 acc[NT];
    if constexpr (FMT == 1) {
      if (i < 7) decode_tile_nv(p, i + 1, kn, sc_next);
#pragma unroll
      for (int k = 0; k < NT; ++k) acc[k] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int k = 0; k < NT; ++k) acc[k] = mfma_f16(kd[c], q[k].op[c], acc[k]);
      sc = sc_cur;
    } else {
      tile_scores_n<FMT, NT>(p, q, i, sc, acc);
    }
    if (FMT == 1) smx = __builtin_elementwise_max(smx, sc);
    else smx_mx = fmaxf(smx_mx, e8m0_to_f32(p.ks[i]));
#pragma unroll
    for (int k = 0; k < NT; ++k) {
      if (MASKED && need_mask[k]) {
        const int t0 = j * kPage + 16 * i + 4 * G;
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (t0 + v >= q[k].len_n) acc[k][v] = -INFINITY;
      }
      run[k] = __builtin_fmaxf(__builtin_fmaxf(run[k], acc[k][0]), acc[k][1]);
      run[k] = __builtin_fmaxf(__builtin_fmaxf(run[k], acc[k][2]), acc[k][3]);
      asm volatile("" : "+v"(run[k]));  // the tile is finished before the one after next is decoded
    }
    if constexpr (FMT == 1) {
      if (i < 7) {
#pragma unroll
        for (int c = 0; c < 4; ++c) kd[c] = kn[c];
        sc_cur = sc_next;
      }
    }
  }
  };
  if (any_mask) tiles(std::true_type{});
  else tiles(std::false_type{});
  float m0, m1 = 0.f;
  if (FMT == 1) {
    const f16x2 sm = row_max_f16x2(smx);
    m0 = (float)sm[0];
    m1 = (float)sm[1];
  } else {
    m0 = lane_fmax<1, 16>(smx_mx);
  }
  if constexpr (NT == 4) {
    // row G of the wave finishes tile k = G: its maxima and bound terms reduce-scattered
    // over the rows, then one score and one bound store per lane
    float part[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      part[k] = FMT == 1 ? 6.0f * (m0 * (kAccRel * q[k].qs0 + q[k].qe0) + m1 * (kAccRel * q[k].qs1 + q[k].qe1))
                         : 6.0f * m0 * (kAccRel * q[k].qs0 + q[k].qe0);
    const float r = rows_reduce_scatter4(run[0], run[1], run[2], run[3],
                                         [](float x, float y) { return __builtin_fmaxf(x, y); });
    const float b = rows_reduce_scatter4(part[0], part[1], part[2], part[3], [](float x, float y) { return x + y; });
    // tile G's row fields; each candidate is pinned so that the choice stays a chain of
    // selects (folded into an index into the tile array it would put the tiles in scratch)
    float uns = q[0].unscale;
    int r0 = q[0].r0, ql = q[0].ql;
#pragma unroll
    for (int k = 1; k < 4; ++k) {
      float u = q[k].unscale;
      int rk = q[k].r0, qk = q[k].ql;
      asm volatile("" : "+v"(u), "+v"(rk), "+v"(qk));
      uns = G == k ? u : uns;
      r0 = G == k ? rk : r0;
      ql = G == k ? qk : ql;
    }
    if (n < ql) {
      const int64_t o = (int64_t)(r0 + n) * a.max_blocks + j;
      a.ws_score[o] = r * uns;
      a.ws_bound[o] = b * uns * (1.0f + 0x1p-10f);
    }
    return;
  }
#pragma unroll
  for (int k = 0; k < NT; ++k) {
    const float r = lane_fmax<16, 64>(run[k]);
    float part = FMT == 1 ? 6.0f * (m0 * (kAccRel * q[k].qs0 + q[k].qe0) + m1 * (kAccRel * q[k].qs1 + q[k].qe1))
                          : 6.0f * m0 * (kAccRel * q[k].qs0 + q[k].qe0);
    part = lane_sum<16, 64>(part);
    if (G == 0 && n < q[k].ql) {
      const int64_t o = (int64_t)(q[k].r0 + n) * a.max_blocks + j;
      a.ws_score[o] = r * q[k].unscale;
      a.ws_bound[o] = part * q[k].unscale * (1.0f + 0x1p-10f);
    }
  }
}

// Streaming scan. The (work group, block) units of all groups form one flat list
// (block fastest). Workgroup g (one per CU) takes the contiguous slice
// [g * N / W, (g + 1) * N / W), so consecutive slices of a long request land on
// different XCDs. The slice's block-table entries are staged in LDS, and its
// waves claim units one at a time from an LDS counter: a wave whose pages arrive
// late simply takes fewer units, so the waves of a workgroup finish together.
// Each wave keeps one page in flight: measured, 16 waves with one page each beat
// 8 waves with two or three (deeper per-wave prefetch only deepens the queue).
// Decode groups (one request, <= 16 rows) use NT = 1 query tile and 16 waves.
// Prefill groups (<= 64 rows) use 8 waves, for the registers of more query
// tiles: NVFP4 scores all 64 rows at once (NT = 4, so each decoded K tile feeds
// four MFMA column tiles); MXFP4, whose query tiles take three e4m3 terms each,
// scores them in H = 2 passes of NT = 2 tiles, a (group, block, half) unit each.
constexpr int kScanChunk = 1024;  // units staged in LDS at a time

// ---------------------------------------------------------------------------
// the decode step's scan (m3s_decode_step): store, row map and scan in one launch
// ---------------------------------------------------------------------------
// Inclusive prefix sum over the 64 lanes of a wave (six lane-xor exchanges, no LDS):
// after the exchange with lane ^ M, tot is the sum over the lane's aligned group of 2M
// lanes, and a lane in the upper half of that group adds the lower half's sum.
__device__ __forceinline__ int wave_incl_sum(int x) {
  const int lane = threadIdx.x & 63;
  int tot = x;
  int t;
  t = lane_xor<1>(tot);
  if (lane & 1) x += t;
  tot += t;
  t = lane_xor<2>(tot);
  if (lane & 2) x += t;
  tot += t;
  t = lane_xor<4>(tot);
  if (lane & 4) x += t;
  tot += t;
  t = lane_xor<8>(tot);
  if (lane & 8) x += t;
  tot += t;
  t = lane_xor<16>(tot);
  if (lane & 16) x += t;
  tot += t;
  t = lane_xor<32>(tot);
  if (lane & 32) x += t;
  return x;
}

// A request the decode row map accepts: its rows lie in [0, num_rows), q_len in [1, 16],
// seq_len >= q_len.
__device__ __forceinline__ bool step_request_ok(int q0, int q1, int sl, int num_rows) {
  const int ql = q1 - q0;
  return q0 >= 0 && q1 <= num_rows && ql >= 1 && ql <= kMaxQLen && sl >= ql;
}

// Wave 0: s_blk[b] = exclusive prefix over the requests of each accepted request's
// blocks with no new token, floor((seq_len - q_len) / 128) (0 for the others). The
// decode step's scan takes these blocks; the tail workgroups the rest.
// s_cq[b] = cu_q[b] (b <= B) and s_sb[b] = seq_len - q_len + 1 - cu_q[b], the rows'
// closed-form length base (query_rows), for the scan's query loads.
__device__ __forceinline__ void step_prefix_old(const IndexArgs& a, int* s_blk, int* s_cq, int* s_sb) {
  const int lane = threadIdx.x & 63;
  const int B = a.num_reqs;
  int carry = 0;
  if (lane == 0) s_cq[0] = a.cu_q[0];
  for (int base = 0; base < B; base += 64) {
    const int b = base + lane;
    int nb = 0;
    if (b < B) {
      const int q0 = a.cu_q[b], q1 = a.cu_q[b + 1], sl = a.seq_lens[b];
      if (step_request_ok(q0, q1, sl, a.num_rows)) nb = (sl - (q1 - q0)) / kPage;
      s_cq[b + 1] = q1;
      s_sb[b] = sl - (q1 - q0) + 1 - q0;
    }
    const int x = wave_incl_sum(nb);
    if (b < B) s_blk[b] = carry + x - nb;
    carry += __builtin_amdgcn_readlane(x, 63);
  }
  if (lane == 0) s_blk[B] = carry;
}

// STEP: the decode step's scan (NT = H = 1): its units are each accepted request's
// blocks with no new token (step_prefix_old), and the rows' causal lengths come from
// seq_lens (query_rows in closed form), since the row map is written by the same
// launch.
template <int FMT, int NT, int WAVES, int H, bool STEP>
__device__ __forceinline__ void scan_body(const IndexArgs& a, int wg, int nwg) {
  constexpr int kScanWaves = WAVES;
  __shared__ int s_blk[M3S_MAX_REQS_INTERNAL + 1];
  __shared__ int s_unit[kScanChunk];  // request * kMaxBlocks + block; -1: not scored
  __shared__ int s_page[kScanChunk];  // page; -1: unusable
  __shared__ int s_ctr;
  // prefill groups' requests, read with the block prefix (no dependent load before a
  // unit's block-table entry)
  __shared__ int s_greq[NT > 1 ? M3S_MAX_REQS_INTERNAL : 1];
  // decode step: cu_q and the rows' length base, read by the prefix anyway; a wave
  // that meets a new request issues its query loads from these, with no dependent
  // global load first (under the scan's load that round trip takes microseconds).
  // Elsewhere a wave reads cu_q itself: loading it in the prologue measured slower.
  __shared__ int s_cq[STEP ? M3S_MAX_REQS_INTERNAL + 1 : 1];
  __shared__ int s_sb[STEP ? M3S_MAX_REQS_INTERNAL : 1];
  // decode step: the index query rows of the slice's requests (when they fit), loaded
  // once by the workgroup beside the block-table entries, instead of by every wave
  // that meets a request (about a tenth of the workgroup's vector load instructions
  // otherwise, issued while its waves queue to issue their page loads; measured, the
  // MXFP4 step 3 us faster, NVFP4 0.3 us); rows padded against bank conflicts
  constexpr int kStageRows = 64, kStageRow = 136;
  __shared__ __attribute__((aligned(16))) uint16_t s_qst[STEP ? kStageRows : 1][kStageRow];
  static_assert(NT > 1 || H == 1, "one query tile per group: one pass");
  const int tid = threadIdx.x, lane = tid & 63;
  const int n = lane & 15, G = lane >> 4;
  const int B = a.num_reqs;
  if constexpr (STEP) {
    static_assert(NT == 1 && H == 1, "the decode step's scan");
    if (tid < 64) step_prefix_old(a, s_blk, s_cq, s_sb);
  } else {
    for (int i = tid; i <= B; i += kScanWaves * 64) {
      s_blk[i] = a.req_blk[i];
      if (NT > 1 && i < B) s_greq[i] = a.grp_req ? a.grp_req[i] : i;
    }
  }
  __syncthreads();
  const int64_t total = (int64_t)s_blk[B] * H;
  const int64_t w0 = (int64_t)wg * total / nwg;
  const int64_t w1 = (int64_t)(wg + 1) * total / nwg;

  auto req_of = [&](int64_t u) {  // largest b with s_blk[b] <= u
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_blk[mid] <= u) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  auto claim = [&]() {
    int v = 0;
    if (lane == 0) v = atomicAdd(&s_ctr, 1);
    return __builtin_amdgcn_readlane(v, 0);
  };

  // decode step: rows [q_lo, q_lo + q_n) are staged in s_qst, 16 B per thread, loaded
  // here and written to LDS after the block-table loads are issued (one round trip)
  int q_lo = 0, q_n = 0;
  u32x4 q_chunk = {0u, 0u, 0u, 0u};
  if constexpr (STEP) {
    static_assert(kStageRows * 16 <= kScanWaves * 64, "one staged chunk per thread");
    if (w1 > w0) {
      q_lo = s_cq[req_of(w0)];
      q_n = s_cq[req_of(w1 - 1) + 1] - q_lo;
      if (q_n <= 0 || q_n > kStageRows || q_lo < 0 || q_lo + q_n > a.num_rows) q_n = 0;
    }
    if (tid < q_n * 16)
      q_chunk = *reinterpret_cast<const u32x4*>(a.q_idx + (int64_t)(q_lo + (tid >> 4)) * a.q_stride + 8 * (tid & 15));
  }

  // the LDS unit table of chunk [c0, c0 + cnt): each unit's key and page
  auto build_table = [&](int64_t c0, int cnt) {
    for (int i = tid; i < cnt; i += kScanWaves * 64) {
      const int64_t u = (c0 + i) / H;  // the H passes of a block are adjacent units
      const int half = (int)((c0 + i) - u * H);
      const int bl = req_of(u);
      const int jl = (int)(u - s_blk[bl]);
      int key = -1, pg = -1;
      if (jl < a.max_blocks) {
        key = (bl * H + half) * kMaxBlocks + jl;
        // the page first: its load goes out before the checks below, which would hold it
        // back a round trip (a status atomic may not be passed by a later load)
        int breq = bl;  // the group's request
        if constexpr (NT > 1) breq = s_greq[bl];
        pg = breq >= 0 ? a.block_table[(int64_t)breq * a.bt_stride + jl] : -1;
        // rows past the query tiles' capacity are never scored: flag the group
        bool over = false;
        if (jl == 0 && half == 0) {
          if constexpr (STEP) over = s_cq[bl + 1] - s_cq[bl] > 16 * NT * H;
          else over = a.cu_q[bl + 1] - a.cu_q[bl] > 16 * NT * H;
        }
        if (over) set_status(a.status, kDevBadRows);
        if (pg < 0 || pg >= a.num_pages) {
          set_status(a.status, kDevBadPage);
          pg = -1;
        }
      } else {
        set_status(a.status, kDevBadLength);
      }
      s_unit[i] = key;
      s_page[i] = pg;
    }
  };
  // the first chunk's table is built before the loop, so the staged query chunk is
  // written (and dead) before the claim loop
  if (w1 > w0) build_table(w0, (int)min((int64_t)kScanChunk, w1 - w0));
  if constexpr (STEP) {
    if (tid < q_n * 16) *reinterpret_cast<u32x4*>(&s_qst[tid >> 4][8 * (tid & 15)]) = q_chunk;
  }

  for (int64_t c0 = w0; c0 < w1; c0 += kScanChunk) {  // uniform over the workgroup
    const int cnt = (int)min((int64_t)kScanChunk, w1 - c0);
    if (c0 != w0) build_table(c0, cnt);
    if (tid == 0) s_ctr = 0;
    __syncthreads();
    QueryTile qt[NT];
    int qb = -1;  // (work group, pass) whose query tiles qt holds
    // query tile k of (group, pass) bh
    auto load_tile = [&](int k, int bh) {
      const int b = bh / H;
      if constexpr (STEP) {
        query_rows(qt[k], a, b, k, s_cq[b], s_cq[b + 1], true, s_sb[b], n);
        const int row = n < qt[k].ql ? qt[k].r0 + n : -1;
        u32x4 raw[4];
        if (row >= q_lo && row < q_lo + q_n) query_raw_lds<FMT>(raw, s_qst[row - q_lo], G);
        else query_raw<FMT>(raw, a, row, G);
        query_from_raw<FMT>(qt[k], raw, n, G);
      } else {
        query_rows(qt[k], a, b, NT * (bh % H) + k, a.cu_q[b], a.cu_q[b + 1], false, 0, n);
        build_query<FMT>(qt[k], a, n < qt[k].ql ? qt[k].r0 + n : -1, n, G);
      }
    };
    auto process = [&](const PageBuf& buf, int key, int pg) {
      if (key < 0) return;
      const int bh = key / kMaxBlocks, j = key - bh * kMaxBlocks;
      if (bh != qb) {  // NT = 1: the query loads go out right behind the page's
        qb = bh;
#pragma unroll
        for (int k = 0; k < NT; ++k) load_tile(k, bh);
      }
      if (pg >= 0) {
        if constexpr (NT == 1) score_page<FMT>(buf, qt[0], a, j, n, G);
        else score_page_n<FMT, NT>(buf, qt, a, j, n, G);
      } else if (G == 0) {
#pragma unroll
        for (int k = 0; k < NT; ++k) {
          if (n < qt[k].ql) {
            const int64_t o = (int64_t)(qt[k].r0 + n) * a.max_blocks + j;
            a.ws_score[o] = -INFINITY;
            a.ws_bound[o] = 0.f;
          }
        }
      }
    };
    // one page in flight per wave; the other waves of the SIMD cover its latency
    // (measured: for the prefill variant a second page in flight per wave was
    // slower, its time goes to the scoring itself). In the NVFP4 decode step only 12 of
    // the 16 waves claim pages: with every wave in, the CU's vector-memory path is full
    // from the first round and the youngest waves' first pages come back last. Measured
    // (same-box A/B, steps per graph replay): 12 fastest of 8 to 16 at 8 x 8 rows at 150K
    // (44.8 against 46.3 us), the skewed batch (52.4 against 54.2) and 48 lognormal
    // requests (181.3 against 185.6). The MXFP4 step (more arithmetic per page) and the
    // separate scan measured no faster or slower with 12 and keep all 16.
    constexpr int kClaimWaves = STEP && FMT == 1 ? 12 : kScanWaves;
    while ((tid >> 6) < kClaimWaves) {
      const int c = claim();
      if (c >= cnt) break;
      // uniform over the wave (read from LDS at a uniform index): in scalar registers,
      // the page's base is the loads' scalar base, one lane offset each
      const int key = __builtin_amdgcn_readfirstlane(s_unit[c]);
      const int pg = __builtin_amdgcn_readfirstlane(s_page[c]);
      if constexpr (NT > 1) {
        // a new group's query tiles are built before its page is loaded, so the
        // page registers are not live across the build
        const int bh = key / kMaxBlocks;
        if (key >= 0 && bh != qb) {
          qb = bh;
#pragma unroll
          for (int k = 0; k < NT; ++k) {
            load_tile(k, bh);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      PageBuf pa;  // per unit: no page registers live across iterations
      if (pg >= 0) load_page<FMT>(pa, a, pg, n, G);
      process(pa, key, pg);
    }
    __syncthreads();  // the chunk's LDS tables are rewritten next
  }
}

template <int FMT, int NT, int WAVES, int H>
__global__ __launch_bounds__(WAVES * 64) void index_scan_kernel(IndexArgs a) {
  scan_body<FMT, NT, WAVES, H, false>(a, blockIdx.x, gridDim.x);
}

// Tail workgroup t of the decode step kernel: requests [b0, b1) (the launcher's split).
// It stores the step's new rows (every token in its share [t T / ntail, (t + 1) T / ntail)
// of the T tokens, and again the tokens of its own requests, so that those are in the
// planes before it reads them: writing the same bytes twice is harmless), waits for its
// stores, then scores each of its requests' blocks that hold a new token against the
// request's rows with the scan's arithmetic, one block per wave at a time (a request's
// q_len <= 16 new tokens touch at most two blocks). No other workgroup reads those pages
// in this launch. For the wave's first block and the first 64 requests' slot checks,
// every load that does not need the stores (the rows to store, the slots, the
// block-table entries, the query) is issued before the first wait.
template <int FMT>
__device__ __forceinline__ void tail_body(const IndexArgs& a, const StoreArgs& s, int t, int ntail) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, G = lane >> 4, l16 = tid & 15;
  const int B = a.num_reqs;
  const int b0 = (int)((int64_t)t * B / ntail), b1 = (int)((int64_t)(t + 1) * B / ntail);
  // the own requests' tokens lie in [lo, hi) (all rows of an accepted request are in
  // [0, num_rows), and num_tokens = num_rows); the wave's first tail unit (ub, uj)
  int lo = 0x7FFFFFFF, hi = 0, nu = 0, ub = -1, uj = 0;
  for (int b = b0; b < b1; ++b) {
    const int q0 = a.cu_q[b], q1 = a.cu_q[b + 1], sl = a.seq_lens[b];
    if (!step_request_ok(q0, q1, sl, a.num_rows)) continue;
    lo = min(lo, q0);
    hi = max(hi, q1);
    const int j_lo = (sl - (q1 - q0)) / kPage, j_hi = (sl + kPage - 1) / kPage;
    if (w >= nu && w < nu + (j_hi - j_lo)) {
      ub = b;
      uj = j_lo + (w - nu);
    }
    nu += j_hi - j_lo;
  }
  const int64_t T = s.num_tokens;
  const int64_t sh0 = (int64_t)t * T / ntail * 3, sh1 = (int64_t)(t + 1) * T / ntail * 3;
  const int64_t ow0 = (int64_t)lo * 3, ow1 = min((int64_t)hi, T) * 3;
  // first 192 rows of the share and of the own tokens: loads in flight together
  StoreLoad sh[3], ow[3];
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    const int64_t r1 = sh0 + 64 * p + (tid >> 4), r2 = ow0 + 64 * p + (tid >> 4);
    store_issue(s, r1 < sh1 ? r1 : -1, l16, sh[p]);
    store_issue(s, r2 < ow1 ? r2 : -1, l16, ow[p]);
  }
  // decode convention, lanes (k, i): token i of request b goes to position
  // seq_len - q_len + i of that request's block table (64 requests per pass)
  auto check = [&](int b, int& slot, int& want) {
    const int i = tid & 15;
    const int q0 = a.cu_q[b], q1 = a.cu_q[b + 1], sl = a.seq_lens[b];
    const int ql = q1 - q0;
    if (step_request_ok(q0, q1, sl, a.num_rows) && i < ql && q0 + i < T) {
      const int pos = sl - ql + i, j = pos / kPage;
      const int pg = j < a.max_blocks ? a.block_table[(int64_t)b * a.bt_stride + j] : -1;
      slot = s.slots[q0 + i];
      if (pg >= 0 && pg < a.num_pages) want = pg * kPage + pos % kPage;
    }
  };
  int chk_slot = -1, chk_want = -1;
  if (b0 + (tid >> 4) < b1) check(b0 + (tid >> 4), chk_slot, chk_want);
  // the wave's first unit: its page entry and its query tile
  int pg = -1;
  QueryTile qt;
  if (ub >= 0 && uj < a.max_blocks) {
    pg = a.block_table[(int64_t)ub * a.bt_stride + uj];
    load_query<FMT>(qt, a, ub, 0, n, G);
  }
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    store_commit<FMT>(s, l16, sh[p]);
    store_commit<FMT>(s, l16, ow[p]);
  }
  // rows past the first 192 of either range (more than 64 tokens per tail workgroup)
  for (int64_t rr = sh0 + 192 + (tid >> 4); rr < sh1; rr += 64) store_row<FMT>(s, rr, l16);
  for (int64_t rr = ow0 + 192 + (tid >> 4); rr < ow1; rr += 64) store_row<FMT>(s, rr, l16);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have landed (vmcnt counts stores)
  __syncthreads();                // ... and every wave's, before any page read
  if (chk_want >= 0 && chk_slot != chk_want) set_status(a.status, kDevStepSlot);
  for (int b = b0 + 64 + (tid >> 4); b < b1; b += 64) {  // further requests' slot checks
    int sl2 = -1, want2 = -1;
    check(b, sl2, want2);
    if (want2 >= 0 && sl2 != want2) set_status(a.status, kDevStepSlot);
  }
  // the wave's units: u = w, w + 16, ... of the workgroup's tail blocks in request order
  auto score_unit = [&](int b, int j, int pgv, QueryTile& q) {
    if (j >= a.max_blocks) {
      if (lane == 0) set_status(a.status, kDevBadLength);
      return;
    }
    if (pgv < 0 || pgv >= a.num_pages) {
      if (lane == 0) set_status(a.status, kDevBadPage);
      if (G == 0 && n < q.ql) {
        const int64_t o = (int64_t)(q.r0 + n) * a.max_blocks + j;
        a.ws_score[o] = -INFINITY;
        a.ws_bound[o] = 0.f;
      }
      return;
    }
    PageBuf pa;
    load_page<FMT>(pa, a, pgv, n, G);
    score_page<FMT>(pa, q, a, j, n, G);
  };
  if (ub < 0) return;
  score_unit(ub, uj, pg, qt);
  if (nu <= 16) return;
  int u = 0;
  for (int b = b0; b < b1; ++b) {
    const int q0 = a.cu_q[b], q1 = a.cu_q[b + 1], sl = a.seq_lens[b];
    if (!step_request_ok(q0, q1, sl, a.num_rows)) continue;
    const int j_lo = (sl - (q1 - q0)) / kPage, j_hi = (sl + kPage - 1) / kPage;
    for (int j = j_lo; j < j_hi; ++j, ++u) {
      if (u < 16 || u % 16 != w) continue;
      QueryTile q2;
      int pg2 = -1;
      if (j < a.max_blocks) {
        pg2 = a.block_table[(int64_t)b * a.bt_stride + j];
        load_query<FMT>(q2, a, b, 0, n, G);
      }
      score_unit(b, j, pg2, q2);
    }
  }
}

// The decode step's first kernel: workgroup 0 builds the row map (m3s_decode_rows),
// workgroups 1 .. ntail store the step's new rows and score the blocks that hold them
// (tail_body), and the rest scan every other causal block (scan_body with STEP). The
// three are independent within the launch, so the store and the row map cost no
// launch of their own.
template <int FMT>
__global__ __launch_bounds__(1024) void step_scan_kernel(IndexArgs a, StoreArgs s, RowsArgs r, int ntail) {
  if (blockIdx.x == 0) {
    __shared__ int s_scan[16];
    decode_rows_body<1024>(r, s_scan);
  } else if ((int)blockIdx.x <= ntail) {
    tail_body<FMT>(a, s, blockIdx.x - 1, ntail);
  } else {
    scan_body<FMT, 1, 16, 1, true>(a, blockIdx.x - 1 - ntail, gridDim.x - 1 - ntail);
  }
}

// ---------------------------------------------------------------------------
// select
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t comp_key(uint32_t key, int j, int tie_high) {
  return ((uint64_t)key << 32) | (uint32_t)(tie_high ? (uint32_t)j : ~(uint32_t)j);
}

__device__ __forceinline__ uint64_t shfl_u64(uint64_t x, int src) {
  const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)x, src, 64);
  const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(x >> 32), src, 64);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) { return lane_max<1, 64>(x); }

// Bitonic network over one u64 per lane, descending across the wave.
template <int SIZE, int STRIDE>
__device__ __forceinline__ uint64_t bitonic_steps(uint64_t x) {
  if constexpr (STRIDE == 0) {
    return x;
  } else {
    const int lane = threadIdx.x & 63;
    const uint64_t o = lane_xor<STRIDE>(x);
    const bool lower = (lane & STRIDE) == 0;       // first element of the pair
    const bool desc = (lane & SIZE) == 0;          // direction of this bitonic block (all at SIZE 64)
    x = (lower == desc) ? (o > x ? o : x) : (o < x ? o : x);
    return bitonic_steps<SIZE, STRIDE / 2>(x);
  }
}
// Sizes 2 .. MAX: each group of MAX lanes ends sorted, the first group
// (lanes 0 .. MAX - 1) descending.
template <int SIZE, int MAX = 64>
__device__ __forceinline__ uint64_t bitonic_sizes(uint64_t x) {
  if constexpr (SIZE > MAX) {
    return x;
  } else {
    return bitonic_sizes<SIZE * 2, MAX>(bitonic_steps<SIZE, SIZE / 2>(x));
  }
}
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t x) { return bitonic_sizes<2>(x); }
// Descending sort of the first n lanes' keys (the other lanes hold 0): a
// network over only the lanes that can hold keys.
__device__ __forceinline__ uint64_t sort_desc_first(uint64_t x, int n) {
  if (n <= 16) return bitonic_sizes<2, 16>(x);
  if (n <= 32) return bitonic_sizes<2, 32>(x);
  return bitonic_sizes<2>(x);
}

// Select: one 256-thread workgroup per row.
//   0. the row's scores (thread t holds blocks j = t + 256 i), its largest
//      error bound and its query are loaded at once; the page ids of its
//      blocks follow as soon as the row's request is known (a rescore needs
//      them, and loading them here takes that load off its critical path);
//   1. threshold: each wave bitonic-sorts its 64 thread maxima (ordered score
//      bits); wave w contributes c_w of the k+1 keys (ceil((k+1)/4) each, moved
//      to earlier waves when a short row leaves a later wave fewer live threads),
//      so the smallest of the four c_w-th largest maxima lies at or below the
//      (k+1)-th best key; the keys at or above it (usually < 64) are sorted by
//      one wave as (score, tie-rule id), giving the k-th and (k+1)-th keys
//      exactly; an iterative extraction covers larger sets and k = 64;
//   2. certification against the row's error bound, in one pass: blocks above
//      hi are in, below lo out, the band between is listed with its pages; when
//      it does not exactly fill the open slots each band block is rescored in
//      exact float64 by one wave, over only the tokens its bound leaves open;
//   3. the k selected ids are gathered in LDS and one wave sorts them ascending.
// Score registers per thread: PER = 5, 8, 14, 16 or 32 (rows of up to 256 PER blocks),
// picked at launch from max_blocks; the smallest that fits keeps the kernel's
// code small (it runs once per row on cold instruction caches).

struct SelectShared {
  uint64_t cand[64];
  int band[kBandCap];
  int bpage[kBandCap];
  float bdel[kBandCap];
  double dots[kBandCap];
  alignas(16) double q[kDim];
  uint32_t thr[4];
  float red[4];
  int ired[4];
  int cnt[4];  // candidates, in, band, selected
  uint64_t keys[2];
  int sel[64];
  int selp[64];  // page of each gathered id (when the caller wants pages)
};

// bitonic network over one u32 per lane, descending across the wave
template <int SIZE, int STRIDE>
__device__ __forceinline__ uint32_t bitonic32_steps(uint32_t x) {
  if constexpr (STRIDE == 0) {
    return x;
  } else {
    const int lane = threadIdx.x & 63;
    const uint32_t o = lane_xor<STRIDE>(x);
    const bool keep_max = ((lane & STRIDE) == 0) == ((lane & SIZE) == 0);
    x = keep_max ? max(o, x) : min(o, x);
    return bitonic32_steps<SIZE, STRIDE / 2>(x);
  }
}
template <int SIZE, int MAX = 64>
__device__ __forceinline__ uint32_t bitonic32_sizes(uint32_t x) {
  if constexpr (SIZE > MAX) return x;
  else return bitonic32_sizes<SIZE * 2, MAX>(bitonic32_steps<SIZE, SIZE / 2>(x));
}

// The select of row r as a device function, for a workgroup of NW waves (4 or
// 8). The first four waves hold the row's blocks (thread t < 256: blocks
// t + 256 i) and run every phase; further waves take part only in the exact
// rescore (one band block per wave) and in the barriers. It writes the row's
// ids to topk_ids when write_ids. When ids_out is given, wave 0 also leaves
// the sorted ids and their pages in ids_out / pages_out and the row's request
// and length in row_out (LDS, visible after the caller's next barrier).
template <int FMT, int PER, int NW, bool PAGES>
__device__ __forceinline__ void select_row(const IndexArgs& a, int r, SelectShared& sh, bool write_ids,
                                           int* ids_out, int* pages_out, int* row_out) {
  constexpr int SB = FMT == 1 ? 8 : 4;
  constexpr int kSelPer = PER;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int bt0 = tid < 256 ? tid : (1 << 30);  // first block of the thread; none past the fourth wave
  const int k = a.topk;
  const int th = a.tie_high;
  const int MB = a.max_blocks;
  int32_t* out = a.topk_ids + (int64_t)r * k;

  // 0. loads, all issued together
  const float* sc = a.ws_score + (int64_t)r * MB;
  const float* bd = a.ws_bound + (int64_t)r * MB;
  const int b = a.row_req[r];
  const int len = a.row_len[r];
  float sv[kSelPer], bv[kSelPer];
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const int j = bt0 + 256 * i;
    if (j >= MB) break;
    sv[i] = sc[j];
    bv[i] = bd[j];
  }
  uint32_t qbits = 0;
  if (tid < kDim) qbits = a.q_idx[(int64_t)r * a.q_stride + tid];
  const int nb = (len + kPage - 1) / kPage;
  if (PAGES && tid == 0) {
    row_out[0] = b;
    row_out[1] = len;
  }
  if (b < 0 || len <= 0 || nb > MB || nb <= k) {
    if (b >= 0 && (len <= 0 || nb > MB) && tid == 0) set_status(a.status, kDevBadLength);
    const bool all = b >= 0 && len > 0 && nb <= MB;
    const int id = (all && tid < nb) ? tid : -1;
    if (write_ids && tid < k) out[tid] = id;
    if (PAGES && tid < k) {
      ids_out[tid] = id;
      pages_out[tid] = id >= 0 ? a.block_table[(int64_t)b * a.bt_stride + id] : -1;
    }
    return;
  }
  int pv[kSelPer];
  const int32_t* btr = a.block_table + (int64_t)b * a.bt_stride;
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const int j = bt0 + 256 * i;
    if (j >= nb) break;
    pv[i] = btr[j];
  }
  // forced class of block j: 2 initial, 1 local, 0 scored (initial wins on overlap)
  const int I = a.init_blocks, L = a.local_blocks;
  auto cls_of = [&](int j) { return j < I ? 2 : (j >= nb - L ? 1 : 0); };
  // blocks past the row's causal range were never scored: they never compete
  // and their workspace entries are not read; forced blocks' scores play no part
  float dm = 0.f;
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const int j = bt0 + 256 * i;
    if (j >= MB) break;
    if (j >= nb) sv[i] = -INFINITY;
    else if (cls_of(j) == 0) dm = fmaxf(dm, bv[i]);
  }
  // ordered keys, formed once: forced blocks above every float (initial
  // 0xFFFFFFFF, local 0xFFFFFFFE; finite and infinite scores order below
  // 0xFF800001), ties among them to the higher id
  uint32_t ok[kSelPer];
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const int j = bt0 + 256 * i;
    if (j >= nb) break;
    const int c = cls_of(j);
    ok[i] = c == 2 ? 0xFFFFFFFFu : (c == 1 ? 0xFFFFFFFEu : ord_f32(sv[i]));
  }
  auto forced = [&](int i) { return ok[i] >= 0xFFFFFFFEu; };
  auto okey = [&](int i) { return ok[i]; };
  auto ckey = [&](int i) { return comp_key(ok[i], bt0 + 256 * i, forced(i) ? 1 : th); };

  // 1. threshold from the per-wave sorted thread maxima
  uint32_t tmax = 0;
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const int j = bt0 + 256 * i;
    if (j >= nb) break;
    tmax = max(tmax, okey(i));
  }
  int lqv = INT_MAX;
  if (tid < kDim) {
    sh.q[tid] = (double)bf16_bits_to_f32(qbits);
    const uint32_t m = qbits & 0x7FFFu;
    if (m) {
      const uint32_t ex = m >> 7, mant = m & 0x7Fu;
      const uint32_t M = ex ? (mant | 0x80u) : mant;
      lqv = (ex ? (int)ex - 134 : -133) + __builtin_ctz(M);
    }
  }
  dm = lane_fmax<1, 64>(dm);
  lqv = lane_reduce<1, 64>(lqv, [](int x, int y) { return x < y ? x : y; });
  const bool small_k = k < 64;
  int cw = 0;
  {
    const int c = (k + 4) / 4;
    int tot = 0;
    for (int q4 = 0; q4 < 4; ++q4) tot += min(min(max(nb - 64 * q4, 0), 64), c);
    int def = k + 1 - tot;
    for (int q4 = 0; q4 < 4; ++q4) {
      const int n = min(max(nb - 64 * q4, 0), 64);
      int cq = min(n, c);
      const int add = min(def, n - cq);
      cq += add;
      def -= add;
      if (q4 == w) cw = cq;
    }
  }
  uint32_t theta_w = 0xFFFFFFFFu;
  if (small_k) {
    const uint32_t srt = bitonic32_sizes<2>(tmax);
    if (cw > 0) theta_w = __shfl(srt, cw - 1, 64);
  }
  if (lane == 0 && w < 4) {
    sh.red[w] = dm;
    sh.ired[w] = lqv;
    sh.thr[w] = theta_w;
  }
  if (tid < 4) sh.cnt[tid] = 0;
  __syncthreads();
  const float dmax = fmaxf(fmaxf(sh.red[0], sh.red[1]), fmaxf(sh.red[2], sh.red[3]));
  int lq = min(min(sh.ired[0], sh.ired[1]), min(sh.ired[2], sh.ired[3]));
  lq = lq == INT_MAX ? 0 : lq;
  if (small_k) {
    const uint32_t theta = min(min(sh.thr[0], sh.thr[1]), min(sh.thr[2], sh.thr[3]));
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) {
      const int j = bt0 + 256 * i;
      if (j >= nb) break;
      if (okey(i) >= theta) {
        const int slot = atomicAdd(&sh.cnt[0], 1);
        if (slot < 64) sh.cand[slot] = ckey(i);
      }
    }
  }
  __syncthreads();
  const int ncand = sh.cnt[0];
  if (small_k && ncand <= 64) {
    if (w == 0) {
      const uint64_t srt = sort_desc_first(lane < ncand ? sh.cand[lane] : 0, ncand);
      const uint64_t Kk = shfl_u64(srt, k - 1), K1 = shfl_u64(srt, k);
      if (lane == 0) {
        sh.keys[0] = Kk;
        sh.keys[1] = K1;
      }
    }
  } else {  // iterative extraction of the k+1 best keys
    uint64_t prev = ~(uint64_t)0;
    for (int t = 0; t <= k; ++t) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < kSelPer; ++i) {
        const int j = bt0 + 256 * i;
        if (j >= nb) break;
        const uint64_t c = ckey(i);
        if (c < prev && c > best) best = c;
      }
      best = wave_max_u64(best);
      if (lane == 0) sh.cand[w] = best;
      __syncthreads();
      best = sh.cand[0];
      for (int q4 = 1; q4 < 4; ++q4) best = sh.cand[q4] > best ? sh.cand[q4] : best;
      if (tid == 0) {
        if (t == k - 1) sh.keys[0] = best;
        sh.keys[1] = best;
      }
      prev = best;
      __syncthreads();
    }
  }
  __syncthreads();
  const uint64_t Kk = sh.keys[0], K1 = sh.keys[1];

  // 2. certification
  int mode = 0;  // 0: by key (exact scores); 1: score >= lo; 2: score > hi, band rescored
  double lo = 0.0, hi = 0.0;
  // when the k-th key is forced, every selected block is forced: keys decide exactly
  if (dmax > 0.f && (uint32_t)(Kk >> 32) < 0xFFFFFFFEu) {
    lo = (double)unord_f32((uint32_t)(Kk >> 32)) - 2.0 * (double)dmax;
    hi = (double)unord_f32((uint32_t)(K1 >> 32)) + 2.0 * (double)dmax;
    // the certain blocks are gathered here (fewer than k: the k-th key is not
    // forced, and only the top k keys can clear hi), the band is listed
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) {
      const int j = bt0 + 256 * i;
      if (j >= nb) break;
      const double s_ = (double)sv[i];
      if (forced(i) || s_ > hi) {
        const int slot = atomicAdd(&sh.cnt[3], 1);
        if (slot < 64) {
          sh.sel[slot] = j;
          if (PAGES) sh.selp[slot] = pv[i];
        }
      } else if (s_ >= lo) {
        const int slot = atomicAdd(&sh.cnt[2], 1);
        if (slot < kBandCap) {
          sh.band[slot] = j;
          sh.bpage[slot] = pv[i];
          sh.bdel[slot] = bv[i];
        }
      }
    }
    __syncthreads();
    const int nin = sh.cnt[3];
    const int need = k - nin;
    const int nband = sh.cnt[2];
    if (nband == need) {
      mode = 1;  // the band fills the open slots: appended after the certain blocks
      for (int i = tid; i < nband; i += 64 * NW) {
        if (nin + i < 64) {
          sh.sel[nin + i] = sh.band[i];
          if (PAGES) sh.selp[nin + i] = sh.bpage[i];
        }
      }
    } else if (nband > kBandCap) {
      if (tid == 0) set_status(a.status, kDevBandOverflow);
      mode = 0;  // selected by key below, from an empty list
      __syncthreads();  // every thread has read the counts
      if (tid == 0) sh.cnt[3] = 0;
      __syncthreads();
    } else {
      mode = 2;
      // exact rescore, one band block per wave. The wave first re-scores the
      // block's tokens with the scan's own arithmetic (same query operand, same
      // MFMA), so the bound the scan stored for this row and block bounds every
      // token's error d: only tokens within 2 d of the block's approximate
      // maximum can hold the exact maximum. Each of those is then summed exactly
      // in float64 by the whole wave (lane l: dims 2l, 2l+1), its data taken from
      // the wave's page registers.
      bool inexact = false;
      const int n = lane & 15, G = lane >> 4;
      QueryTile qt;
      build_query<FMT>(qt, a, n == 0 ? r : -1, n, G);  // column 0: this row
      const double2 qq = *reinterpret_cast<const double2*>(&sh.q[2 * lane]);
      for (int m = w; m < nband; m += NW) {
        const int j = sh.band[m];
        const int page = sh.bpage[m];
        double best = -INFINITY;
        if (page >= 0 && page < a.num_pages) {
          PageBuf pb;
          load_page<FMT>(pb, a, page, n, G);
          const int t_lim = len - j * kPage;  // causal tokens of the block
          f32x4 ts[8];
          float mx = -INFINITY;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            f16x2 unused;
            ts[i] = tile_scores<FMT>(pb, qt, i, unused) * qt.unscale;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              if (n != 0 || 16 * i + 4 * G + v >= t_lim) ts[i][v] = -INFINITY;
              mx = fmaxf(mx, ts[i][v]);
            }
          }
          mx = lane_fmax<1, 64>(mx);
          const double thr = (double)mx - 2.0 * (double)sh.bdel[m];
          // candidate tokens: bit 4 i + v of lane (0, G) is token 16 i + 4 G + v
          uint32_t cm = 0;
#pragma unroll
          for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) cm |= ((double)ts[i][v] >= thr ? 1u : 0u) << (4 * i + v);
          uint64_t holders = __ballot(cm != 0);
          while (holders) {
            const int src = __builtin_ctzll(holders);
            holders &= holders - 1;
            uint32_t bits = __shfl(cm, src, 64);
            while (bits) {
              const int bit = __builtin_ctz(bits);
              bits &= bits - 1;
              const int ti = bit >> 2, v = bit & 3;
              const int nt = 4 * (src >> 4) + v;  // token 16 ti + nt of the block
              const int s2 = nt + 16 * G;         // lane holding dims [32 G, 32 G + 32) of it
              // the tile's words and scales, picked by a select chain (ti is uniform)
              u32x4 kw = pb.kr[0];
              uint32_t ksw = pb.ks[0];
#pragma unroll
              for (int i = 1; i < 8; ++i) {
                if (ti == i) {
                  kw = pb.kr[i];
                  ksw = pb.ks[i];
                }
              }
              const uint32_t w0 = __shfl(kw[0], s2, 64), w1 = __shfl(kw[1], s2, 64);
              const uint32_t w2 = __shfl(kw[2], s2, 64), w3 = __shfl(kw[3], s2, 64);
              const uint32_t sk = __shfl(ksw, s2, 64);
              const int ww = (lane & 15) >> 2;
              const uint32_t word = ww == 0 ? w0 : (ww == 1 ? w1 : (ww == 2 ? w2 : w3));
              const uint32_t byte = (word >> (8 * (lane & 3))) & 0xFFu;
              const auto cd = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(byte, 1.0f, 0);
              double sd;
              int lsb;
              if (FMT == 1) {
                const uint32_t sb = (sk >> (8 * ((lane & 15) >> 3))) & 0xFFu;
                const uint32_t e = (sb >> 3) & 15u, mm = sb & 7u;
                const uint32_t M = e ? (mm | 8u) : mm;
                const int ex = e ? (int)e - 10 : -9;
                sd = __builtin_ldexp((double)M, ex);
                lsb = M ? ex + __builtin_ctz(M) - 1 : INT_MAX;  // codes are multiples of 1/2
              } else {
                sd = __builtin_ldexp(1.0, (int)(sk & 0xFFu) - 127);
                lsb = (int)(sk & 0xFFu) - 128;
              }
              const double k0 = (double)cd[0] * sd, k1 = (double)cd[1] * sd;
              double dot = __builtin_fma(qq.x, k0, qq.y * k1);
              double mag = __builtin_fma(fabs(qq.x), fabs(k0), fabs(qq.y * k1));
              dot = lane_reduce<1, 64>(dot, [](double x, double y) { return x + y; });
              mag = lane_reduce<1, 64>(mag, [](double x, double y) { return x + y; });
              const int lk = lane_reduce<1, 64>(lsb, [](int x, int y) { return x < y ? x : y; });
              if (mag > 0.0 && lk != INT_MAX && !(mag * (1.0 + 0x1p-40) < __builtin_ldexp(1.0, 53 + lq + lk)))
                inexact = true;
              best = fmax(best, dot + 0.0);
            }
          }
        }
        if (lane == 0) sh.dots[m] = best;
      }
      if (inexact) set_status(a.status, kDevInexact);
      __syncthreads();
      for (int i = tid; i < nband; i += 64 * NW) {
        const double ei = sh.dots[i] + 0.0;
        const int ji = sh.band[i];
        const uint32_t ki = th ? (uint32_t)ji : ~(uint32_t)ji;
        int rank = 0;
        for (int m = 0; m < nband; ++m) {
          const double em = sh.dots[m] + 0.0;
          const int jm = sh.band[m];
          const uint32_t km = th ? (uint32_t)jm : ~(uint32_t)jm;
          rank += (em > ei) || (em == ei && km > ki);
        }
        if (rank < need) {
          const int slot = atomicAdd(&sh.cnt[3], 1);
          if (slot < 64) {
            sh.sel[slot] = ji;
            if (PAGES) sh.selp[slot] = sh.bpage[i];
          }
        }
      }
    }
  }
  // 3. the selected ids (gathered above when certified, else by key here),
  // sorted ascending by one wave
  if (mode == 0) {
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) {
      const int j = bt0 + 256 * i;
      if (j >= nb) break;
      if (ckey(i) >= Kk) {
        const int slot = atomicAdd(&sh.cnt[3], 1);
        if (slot < 64) {
          sh.sel[slot] = j;
          if (PAGES) sh.selp[slot] = pv[i];
        }
      }
    }
  }
  __syncthreads();
  if (w != 0) return;
  const int nsel = min(sh.cnt[3], 64);
  if constexpr (PAGES) {
    // (~id, page) pairs sorted descending: ascending ids with their pages
    const uint64_t y = lane < nsel ? ((uint64_t)~(uint32_t)sh.sel[lane] << 32) | (uint32_t)sh.selp[lane] : 0u;
    const uint64_t srt = sort_desc_first(y, nsel);
    const int id = lane < nsel ? (int)~(uint32_t)(srt >> 32) : -1;
    if (lane < k) {
      if (write_ids) out[lane] = id;
      ids_out[lane] = id;
      pages_out[lane] = lane < nsel ? (int)(uint32_t)srt : -1;
    }
  } else {
    const uint32_t y = lane < nsel ? ~(uint32_t)sh.sel[lane] : 0u;  // descending ~id = ascending id
    const uint32_t srt = nsel <= 16 ? bitonic32_sizes<2, 16>(y) : bitonic32_sizes<2>(y);
    if (write_ids && lane < k) out[lane] = lane < nsel ? (int)~srt : -1;
  }
}

// OCC: minimum waves per SIMD. A select workgroup is one latency chain; with
// more rows than two workgroups per CU, occupancy decides how many chains
// overlap, and the NVFP4 select of up to 16 blocks per thread fits three waves
// per SIMD (168 VGPRs, no spills) instead of two. With fewer rows OCC = 1 keeps
// the unconstrained allocation, measured slightly faster at 64 rows.
template <int FMT, int PER, int OCC>
__global__ __launch_bounds__(256, OCC) void index_select_kernel(IndexArgs a) {
  __shared__ SelectShared sh;
  select_row<FMT, PER, 4, false>(a, blockIdx.x, sh, true, nullptr, nullptr, nullptr);
}

// The same select, also writing each selected id's page to sel_pages, for an
// attention pass launched after it (its K / V addresses then need no
// block-table lookup).
template <int FMT, int PER, int OCC>
__global__ __launch_bounds__(256, OCC) void index_select_pages_kernel(IndexArgs a) {
  __shared__ SelectShared sh;
  __shared__ int s_row[2];
  const int r = blockIdx.x;
  select_row<FMT, PER, 4, true>(a, r, sh, false, a.topk_ids + (int64_t)r * a.topk,
                                a.sel_pages + (int64_t)r * a.topk, s_row);
}

// Top-k and attention split in one workgroup of 8 waves per (row, split): the
// row's select runs in every split's workgroup (the first split also writes the
// ids), and the split then attends its blocks with the ids, their pages and
// the row's request and length already on chip. This removes a kernel boundary
// and the attention's two dependent loads (ids, then pages) before its K / V
// loads. The select's LDS is reused by the attention once the ids are out.
union SelectAttendShared {
  SelectShared s;
  AttendShared t;
};

template <int FMT, int PER>
__global__ __launch_bounds__(kWaves * 64) void select_attend_kernel(IndexArgs ia, AttendArgs aa) {
  __shared__ SelectAttendShared u;
  __shared__ int s_ids[64], s_pages[64], s_row[2];
  const int r = blockIdx.x / aa.nsplit;
  const int sp = blockIdx.x - r * aa.nsplit;
  select_row<FMT, PER, kWaves, true>(ia, r, u.s, sp == 0, s_ids, s_pages, s_row);
  __syncthreads();
  attend_split_body<FMT, 1, true>(aa, r, sp, u.t, s_ids, s_pages, s_row[0], s_row[1]);
}

size_t index_ws_bytes(int32_t num_rows, int32_t max_blocks) {
  const size_t one = ((size_t)num_rows * (size_t)max_blocks * sizeof(float) + 255) & ~(size_t)255;
  return 2 * one;
}

static hipError_t launch_scan(const IndexArgs& a, hipStream_t stream) {
  if (a.num_reqs > 0) {
    const bool wide = a.group_tiles > 1;  // prefill work groups of up to 64 rows
    const int waves = wide ? 8 : 16;
    const int passes = wide && a.format == 2 ? 2 : 1;
    const int64_t units_upper = (int64_t)a.num_reqs * a.max_blocks * passes;
    int64_t grid = (units_upper + waves - 1) / waves;
    if (grid > a.scan_grid) grid = a.scan_grid;
    if (grid < 1) grid = 1;
    const dim3 g((unsigned)grid), blk((unsigned)(waves * 64));
    if (a.format == 1) {
      if (wide) hipLaunchKernelGGL((index_scan_kernel<1, 4, 8, 1>), g, blk, 0, stream, a);
      else hipLaunchKernelGGL((index_scan_kernel<1, 1, 16, 1>), g, blk, 0, stream, a);
    } else {
      if (wide) hipLaunchKernelGGL((index_scan_kernel<2, 2, 8, 2>), g, blk, 0, stream, a);
      else hipLaunchKernelGGL((index_scan_kernel<2, 1, 16, 1>), g, blk, 0, stream, a);
    }
    return hipGetLastError();
  }
  return hipSuccess;
}

template <int FMT, int PER, int OCC>
static void launch_select_as(const IndexArgs& a, hipStream_t stream) {
  const dim3 g((unsigned)a.num_rows), blk(256);
  if (a.sel_pages) hipLaunchKernelGGL((index_select_pages_kernel<FMT, PER, OCC>), g, blk, 0, stream, a);
  else hipLaunchKernelGGL((index_select_kernel<FMT, PER, OCC>), g, blk, 0, stream, a);
}

template <int FMT>
static void launch_select_fmt(const IndexArgs& a, hipStream_t stream) {
  if (a.max_blocks <= 256 * 16) {
    if constexpr (FMT == 1) {
      if (a.num_rows > 2 * (int64_t)a.scan_grid) {
        if (a.max_blocks <= 256 * 5) launch_select_as<FMT, 5, 3>(a, stream);
        else if (a.max_blocks <= 256 * 8) launch_select_as<FMT, 8, 3>(a, stream);
        else if (a.max_blocks <= 256 * 14) launch_select_as<FMT, 14, 3>(a, stream);
        else launch_select_as<FMT, 16, 3>(a, stream);
        return;
      }
    }
    if (a.max_blocks <= 256 * 5) launch_select_as<FMT, 5, 1>(a, stream);
    else if (a.max_blocks <= 256 * 8) launch_select_as<FMT, 8, 1>(a, stream);
    else if (a.max_blocks <= 256 * 14) launch_select_as<FMT, 14, 1>(a, stream);
    else launch_select_as<FMT, 16, 1>(a, stream);
  } else {
    launch_select_as<FMT, 32, 1>(a, stream);
  }
}

static hipError_t launch_select(const IndexArgs& a, hipStream_t stream) {
  if (a.format == 1) launch_select_fmt<1>(a, stream);
  else launch_select_fmt<2>(a, stream);
  return hipGetLastError();
}

hipError_t launch_index_topk(const IndexArgs& a, hipStream_t stream) {
  if (a.num_rows == 0) return hipSuccess;
  hipError_t e = launch_scan(a, stream);
  if (e != hipSuccess) return e;
  return launch_select(a, stream);
}

// The select and the attention of a fused call, after its scan.
static hipError_t launch_select_attend_after_scan(const IndexArgs& ia, const AttendArgs& aa, hipStream_t stream) {
  hipError_t e;
  const int64_t wgs = (int64_t)ia.num_rows * aa.nsplit;
  if (wgs > 2 * (int64_t)ia.scan_grid || aa.reps != 1) {
    // Many rows (prefill): every split's workgroup would repeat its row's select,
    // which only pays while the launch is latency-bound (measured at a 4096-row
    // chunk: twice the time of the separate kernels). Same results either way.
    e = launch_select(ia, stream);
    if (e != hipSuccess) return e;
    return launch_sparse_attend(aa, stream);
  }
  const dim3 g((unsigned)wgs), blk(kWaves * 64);
  if (ia.max_blocks <= 256 * 5) {
    if (ia.format == 1) hipLaunchKernelGGL((select_attend_kernel<1, 5>), g, blk, 0, stream, ia, aa);
    else hipLaunchKernelGGL((select_attend_kernel<2, 5>), g, blk, 0, stream, ia, aa);
  } else if (ia.max_blocks <= 256 * 8) {
    if (ia.format == 1) hipLaunchKernelGGL((select_attend_kernel<1, 8>), g, blk, 0, stream, ia, aa);
    else hipLaunchKernelGGL((select_attend_kernel<2, 8>), g, blk, 0, stream, ia, aa);
  } else if (ia.max_blocks <= 256 * 14) {
    if (ia.format == 1) hipLaunchKernelGGL((select_attend_kernel<1, 14>), g, blk, 0, stream, ia, aa);
    else hipLaunchKernelGGL((select_attend_kernel<2, 14>), g, blk, 0, stream, ia, aa);
  } else if (ia.max_blocks <= 256 * 16) {
    if (ia.format == 1) hipLaunchKernelGGL((select_attend_kernel<1, 16>), g, blk, 0, stream, ia, aa);
    else hipLaunchKernelGGL((select_attend_kernel<2, 16>), g, blk, 0, stream, ia, aa);
  } else {
    if (ia.format == 1) hipLaunchKernelGGL((select_attend_kernel<1, 32>), g, blk, 0, stream, ia, aa);
    else hipLaunchKernelGGL((select_attend_kernel<2, 32>), g, blk, 0, stream, ia, aa);
  }
  e = hipGetLastError();
  if (e != hipSuccess || aa.nsplit == 1) return e;
  return launch_attend_combine(aa, stream);
}

hipError_t launch_index_topk_attend(const IndexArgs& ia, const AttendArgs& aa, hipStream_t stream) {
  if (ia.num_rows == 0) return hipSuccess;
  hipError_t e = launch_scan(ia, stream);
  if (e != hipSuccess) return e;
  return launch_select_attend_after_scan(ia, aa, stream);
}

hipError_t launch_decode_step(const IndexArgs& ia, const AttendArgs& aa, const StoreArgs& s, const RowsArgs& r,
                              hipStream_t stream) {
  // tail workgroups: four requests each up to 32 requests (measured at 8 requests of
  // 150K: one tail workgroup of eight outlasts the scan, the step went from 46.3 to
  // 50.8 us), eight beyond, at most an eighth of the CUs (more requests per tail
  // workgroup beyond that); the scan keeps the other CUs, fewer when there are fewer
  // than 16 blocks per workgroup
  const int B = ia.num_reqs;
  const int per = B <= 32 ? 4 : 8;
  const int max_tail = ia.scan_grid / 8 > 1 ? ia.scan_grid / 8 : 1;
  int ntail = B > 0 ? (B + per - 1) / per : (s.num_tokens > 0 ? 1 : 0);
  if (ntail > max_tail) ntail = max_tail;
  int64_t nscan = (int64_t)ia.scan_grid - 1 - ntail;
  const int64_t units_upper = (int64_t)B * ia.max_blocks;
  if (nscan * 16 > units_upper) nscan = (units_upper + 15) / 16;
  if (nscan < 1) nscan = 1;
  const dim3 g((unsigned)(1 + ntail + nscan)), blk(1024);
  if (ia.format == 1) hipLaunchKernelGGL(step_scan_kernel<1>, g, blk, 0, stream, ia, s, r, ntail);
  else hipLaunchKernelGGL(step_scan_kernel<2>, g, blk, 0, stream, ia, s, r, ntail);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ia.num_rows == 0) return e;
  return launch_select_attend_after_scan(ia, aa, stream);
}

}  // namespace m3s
