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
//   select - one workgroup per row: radix-select the top-k of the fp32 scores
//            by (score, id), then certify: a block whose rank the error bound
//            leaves open is rescored in exact float64 and the open slots are
//            filled from those exact scores. The result is the selection that
//            exact arithmetic makes.
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

#include "fp4.hpp"
#include "launch.hpp"

namespace m3s {

constexpr float kAccRel = 0x1p-15f;

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
template <int FMT>
__global__ __launch_bounds__(256) void index_scan_kernel(IndexArgs a) {
  constexpr int SB = FMT == 1 ? 8 : 4;  // scale bytes per token
  typedef Decode<FMT> Dec;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int n = lane & 15;   // A operand: token of the tile; B operand / result: query row
  const int G = lane >> 4;   // lane group: dims [32G, 32G + 32)
  __shared__ int s_b0;

  const int64_t total = a.req_blk[a.num_reqs];
  const int64_t u_begin = total * blockIdx.x / gridDim.x;
  const int64_t u_end = total * (blockIdx.x + 1) / gridDim.x;
  if (u_begin >= u_end) return;  // uniform over the workgroup

  if (threadIdx.x == 0) s_b0 = 0;
  __syncthreads();
  for (int b = threadIdx.x; b < a.num_reqs; b += 256)
    if (a.req_blk[b] <= u_begin && u_begin < a.req_blk[b + 1]) s_b0 = b;
  __syncthreads();
  int b = s_b0;

  int cur_b = -1;
  f16x8 qop[4];
  float qs0 = 0.f, qs1 = 0.f, qe0 = 0.f, qe1 = 0.f, unscale = 1.f;
  int len_n = 0, r0 = 0, ql = 0, min_len = 0;

  for (int64_t u = u_begin + wid; u < u_end; u += 4) {
    while (b + 1 < a.num_reqs && u >= a.req_blk[b + 1]) ++b;
    const int j = (int)(u - a.req_blk[b]);
    if (j >= a.max_blocks) {  // the request is longer than the table: never read past it
      if (lane == 0) set_status(a.status, kDevBadLength);
      continue;
    }

    if (b != cur_b) {  // query tile of request b (rows r0 .. r0 + ql - 1)
      cur_b = b;
      r0 = a.cu_q[b];
      ql = a.cu_q[b + 1] - r0;
      min_len = a.row_len[r0];
      len_n = n < ql ? a.row_len[r0 + n] : 0;
      u32x4 raw[4] = {};
      if (n < ql) {
        const uint16_t* qp = a.q_idx + (int64_t)(r0 + n) * a.q_stride + 32 * G;
#pragma unroll
        for (int s = 0; s < 4; ++s) raw[s] = *reinterpret_cast<const u32x4*>(qp + 8 * s);
      }
      uint32_t mx = 0;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int w = 0; w < 4; ++w) mx = max(mx, max(raw[s][w] & 0x7FFFu, (raw[s][w] >> 16) & 0x7FFFu));
      mx = max(mx, (uint32_t)__shfl_xor((int)mx, 16, 64));
      mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32, 64));
      int P = mx ? 13 - bf16_floor_log2(mx) : 0;
      P = P > 64 ? 64 : (P < -64 ? -64 : P);
      unscale = __builtin_ldexpf(1.0f, -P);
      qs0 = qs1 = qe0 = qe1 = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t bits = (e & 1) ? (raw[s][e >> 1] >> 16) : (raw[s][e >> 1] & 0xFFFFu);
          const float x = __builtin_ldexpf(bf16_bits_to_f32(bits), P);
          const _Float16 h = (_Float16)x;
          const float err = fabsf(x - (float)h);
          qop[s][e] = h;
          if (FMT == 1 && s >= 2) { qs1 += fabsf((float)h); qe1 += err; }
          else { qs0 += fabsf((float)h); qe0 += err; }
        }
      }
    }

    const int page = a.block_table[(int64_t)b * a.bt_stride + j];
    float* dst_s = a.ws_score + (int64_t)(r0 + n) * a.max_blocks + j;
    float* dst_b = a.ws_bound + (int64_t)(r0 + n) * a.max_blocks + j;
    if (page < 0 || page >= a.num_pages) {
      if (lane == 0) set_status(a.status, kDevBadPage);
      if (G == 0 && n < ql) { *dst_s = -INFINITY; *dst_b = 0.f; }
      continue;
    }
    const uint8_t* pay = a.idx_data + (int64_t)page * (kPage * kPayload);
    const uint8_t* scb = a.idx_scale + (int64_t)page * (kPage * SB);
    u32x4 kr[8];
    uint32_t ksb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) kr[i] = *reinterpret_cast<const u32x4*>(pay + (16 * i + n) * kPayload + 16 * G);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (FMT == 1) ksb[i] = *reinterpret_cast<const uint16_t*>(scb + (16 * i + n) * SB + 2 * G);
      else ksb[i] = scb[(16 * i + n) * SB + G];
    }

    const bool need_mask = (j + 1) * kPage > min_len;
    float run = -INFINITY;
    uint32_t sm0 = 0, sm1 = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      typename Dec::scale_t s0, s1;
      if (FMT == 1) {
        const uint32_t b0 = ksb[i] & 0xFFu, b1 = ksb[i] >> 8;
        sm0 = max(sm0, b0);
        sm1 = max(sm1, b1);
        s0 = Dec::scale(b0);
        s1 = Dec::scale(b1);
      } else {
        sm0 = max(sm0, ksb[i]);
        s0 = s1 = Dec::scale(ksb[i]);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = mfma_f16(Dec::run(kr[i][s], s < 2 ? s0 : s1), qop[s], acc);
      if (need_mask) {
        const int t0 = j * kPage + 16 * i + 4 * G;
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (t0 + v >= len_n) acc[v] = -INFINITY;
      }
      run = fmaxf(run, fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3])));
    }
    run = fmaxf(run, __shfl_xor(run, 16, 64));
    run = fmaxf(run, __shfl_xor(run, 32, 64));
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
      sm0 = max(sm0, (uint32_t)__shfl_xor((int)sm0, m, 64));
      sm1 = max(sm1, (uint32_t)__shfl_xor((int)sm1, m, 64));
    }
    float part;
    if (FMT == 1)
      part = 6.0f * (e4m3_to_f32(sm0) * (kAccRel * qs0 + qe0) + e4m3_to_f32(sm1) * (kAccRel * qs1 + qe1));
    else
      part = 6.0f * e8m0_to_f32(sm0) * (kAccRel * qs0 + qe0);
    part += __shfl_xor(part, 16, 64);
    part += __shfl_xor(part, 32, 64);
    if (G == 0 && n < ql) {
      *dst_s = run * unscale;
      *dst_b = part * unscale * (1.0f + 0x1p-10f);
    }
  }
}

// ---------------------------------------------------------------------------
// select
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t comp_key(uint32_t key, int j, int tie_high) {
  return ((uint64_t)key << 32) | (uint32_t)(tie_high ? (uint32_t)j : ~(uint32_t)j);
}

struct SelectShared {
  uint32_t key[kMaxBlocks];
  uint8_t flag[kMaxBlocks];
  uint32_t hist[256];
  int band[kBandCap];
  double exact[kBandCap];
  double q[kDim];
  uint64_t red64[4];
  double redd[4];
  float redf[4];
  int redi[8];
  int misc[4];
  int scan[4];
};

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)x, m, 64);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(x >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

// k-th largest (1-based) composite key among j < n (keys are distinct).
__device__ uint64_t select_kth(SelectShared& sh, int n, int kth, int tie_high) {
  const int tid = threadIdx.x;
  uint64_t prefix = 0, mask = 0;
  int kk = kth;
  for (int d = 56; d >= 0; d -= 8) {
    sh.hist[tid] = 0;
    __syncthreads();
    for (int j = tid; j < n; j += 256) {
      const uint64_t c = comp_key(sh.key[j], j, tie_high);
      if ((c & mask) == prefix) atomicAdd(&sh.hist[(c >> d) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      const int L = tid;
      const int c0 = sh.hist[255 - 4 * L], c1 = sh.hist[254 - 4 * L];
      const int c2 = sh.hist[253 - 4 * L], c3 = sh.hist[252 - 4 * L];
      const int sum = c0 + c1 + c2 + c3;
      int incl = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (L >= off) incl += y;
      }
      const int above = incl - sum;
      if (above < kk && kk <= incl) {
        int acc = above, digit, cnt;
        if (kk <= acc + c0) { digit = 255 - 4 * L; cnt = c0; }
        else if (kk <= acc + c0 + c1) { acc += c0; digit = 254 - 4 * L; cnt = c1; }
        else if (kk <= acc + c0 + c1 + c2) { acc += c0 + c1; digit = 253 - 4 * L; cnt = c2; }
        else { acc += c0 + c1 + c2; digit = 252 - 4 * L; cnt = c3; }
        sh.misc[0] = digit;
        sh.misc[1] = kk - acc;
        sh.misc[2] = cnt;
      }
    }
    __syncthreads();
    const int digit = sh.misc[0], cnt = sh.misc[2];
    kk = sh.misc[1];
    prefix |= (uint64_t)digit << d;
    mask |= (uint64_t)0xFF << d;
    __syncthreads();
    if (cnt == 1) {
      for (int j = tid; j < n; j += 256) {
        const uint64_t c = comp_key(sh.key[j], j, tie_high);
        if ((c & mask) == prefix) sh.red64[0] = c;
      }
      __syncthreads();
      const uint64_t res = sh.red64[0];
      __syncthreads();
      return res;
    }
  }
  return prefix;
}

// Exact float64 score of block j of a row (-inf for an unusable page).
template <int FMT>
__device__ double exact_block_score(const IndexArgs& a, SelectShared& sh, int b, int j, int len, int lq) {
  constexpr int SB = FMT == 1 ? 8 : 4;
  const int tid = threadIdx.x, t = tid >> 1, h = tid & 1;
  const int page = a.block_table[(int64_t)b * a.bt_stride + j];
  const bool page_ok = page >= 0 && page < a.num_pages;
  const bool valid = page_ok && (j * kPage + t < len);
  double acc = 0.0, mag = 0.0;
  int lk = INT_MAX;
  if (page_ok) {
    const uint8_t* p = a.idx_data + (int64_t)page * (kPage * kPayload) + t * kPayload + 32 * h;
    const u32x4 w0 = *reinterpret_cast<const u32x4*>(p);
    const u32x4 w1 = *reinterpret_cast<const u32x4*>(p + 16);
    const uint8_t* sp = a.idx_scale + (int64_t)page * (kPage * SB) + t * SB + (SB / 2) * h;
    double sv[4];
    const int ng = FMT == 1 ? 4 : 2;
    for (int g = 0; g < ng; ++g) {
      const uint32_t byte = sp[g];
      double s;
      int lsb;
      if (FMT == 1) {
        const uint32_t e = (byte >> 3) & 15u, m = byte & 7u;
        const uint32_t M = e ? (m | 8u) : m;
        const int ex = e ? (int)e - 10 : -9;
        s = __builtin_ldexp((double)M, ex);
        lsb = M ? ex + __builtin_ctz(M) : INT_MAX;
      } else {
        s = __builtin_ldexp(1.0, (int)byte - 127);
        lsb = (int)byte - 127;
      }
      sv[g] = s;
      if (lsb != INT_MAX) lk = min(lk, lsb - 1);  // codes are multiples of 1/2
    }
    const double tab[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    for (int dd = 0; dd < 64; ++dd) {
      const uint32_t word = dd < 32 ? w0[dd >> 3] : w1[(dd - 32) >> 3];
      const uint32_t code = (word >> (4 * (dd & 7))) & 15u;
      const double kv = (code & 8u ? -tab[code & 7u] : tab[code & 7u]) * sv[FMT == 1 ? (dd >> 4) : (dd >> 5)];
      const double qv = sh.q[64 * h + dd];
      acc = __builtin_fma(qv, kv, acc);
      mag += fabs(qv) * fabs(kv);
    }
  }
  acc += __shfl_xor(acc, 1, 64);
  mag += __shfl_xor(mag, 1, 64);
  lk = min(lk, __shfl_xor(lk, 1, 64));
  if (valid && mag > 0.0 && lk != INT_MAX) {
    const double lim = __builtin_ldexp(1.0, 53 + lq + lk);
    if (!(mag * (1.0 + 0x1p-40) < lim)) set_status(a.status, kDevInexact);
  }
  double v = valid ? acc + 0.0 : -INFINITY;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmax(v, __shfl_xor(v, m, 64));
  __syncthreads();
  if ((tid & 63) == 0) sh.redd[tid >> 6] = v;
  __syncthreads();
  const double r = fmax(fmax(sh.redd[0], sh.redd[1]), fmax(sh.redd[2], sh.redd[3]));
  __syncthreads();
  return r;
}

template <int FMT>
__global__ __launch_bounds__(256) void index_select_kernel(IndexArgs a) {
  __shared__ SelectShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int r = blockIdx.x;
  const int k = a.topk;
  int32_t* out = a.topk_ids + (int64_t)r * k;
  const int b = a.row_req[r];
  const int len = a.row_len[r];
  if (b < 0) {
    for (int i = tid; i < k; i += 256) out[i] = -1;
    return;
  }
  const int nb = (len + kPage - 1) / kPage;
  if (len <= 0 || nb > a.max_blocks) {
    if (tid == 0) set_status(a.status, kDevBadLength);
    for (int i = tid; i < k; i += 256) out[i] = -1;
    return;
  }
  if (nb <= k) {
    for (int i = tid; i < k; i += 256) out[i] = i < nb ? i : -1;
    return;
  }
  const int th = a.tie_high;
  const float* sc = a.ws_score + (int64_t)r * a.max_blocks;
  const float* bd = a.ws_bound + (int64_t)r * a.max_blocks;
  float dmax = 0.f;
  for (int j = tid; j < nb; j += 256) {
    sh.key[j] = ord_f32(sc[j]);
    sh.flag[j] = 0;
    dmax = fmaxf(dmax, bd[j]);
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) dmax = fmaxf(dmax, __shfl_xor(dmax, m, 64));
  if (lane == 0) sh.redf[wid] = dmax;
  if (tid == 0) { sh.misc[3] = 0; sh.redi[0] = 0; sh.redi[1] = 0; }
  __syncthreads();
  dmax = fmaxf(fmaxf(sh.redf[0], sh.redf[1]), fmaxf(sh.redf[2], sh.redf[3]));

  // (k+1)-th and k-th largest composite keys
  const uint64_t K1 = select_kth(sh, nb, k + 1, th);
  uint64_t mn = ~(uint64_t)0;
  for (int j = tid; j < nb; j += 256) {
    const uint64_t c = comp_key(sh.key[j], j, th);
    if (c > K1 && c < mn) mn = c;
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const uint64_t o = shfl_xor_u64(mn, m);
    mn = o < mn ? o : mn;
  }
  if (lane == 0) sh.red64[wid] = mn;
  __syncthreads();
  uint64_t Kk = sh.red64[0];
  for (int w = 1; w < 4; ++w) Kk = sh.red64[w] < Kk ? sh.red64[w] : Kk;
  __syncthreads();

  bool by_key = dmax == 0.f;  // exact scores: select by composite key directly
  if (!by_key) {
    const double T = (double)unord_f32((uint32_t)(Kk >> 32));
    const double S1 = (double)unord_f32((uint32_t)(K1 >> 32));
    const double lo = T - 2.0 * (double)dmax, hi = S1 + 2.0 * (double)dmax;
    for (int j = tid; j < nb; j += 256) {
      const double s = (double)unord_f32(sh.key[j]);
      if (s > hi) {
        sh.flag[j] = 1;
        atomicAdd(&sh.redi[0], 1);
      } else if (s >= lo) {
        const int slot = atomicAdd(&sh.redi[1], 1);
        if (slot < kBandCap) sh.band[slot] = j;
      }
    }
    __syncthreads();
    const int nin = sh.redi[0], nband = sh.redi[1];
    const int need = k - nin;
    if (nband == need) {
      for (int i = tid; i < nband; i += 256) sh.flag[sh.band[i]] = 1;
    } else if (nband > kBandCap || need < 0) {
      if (tid == 0) set_status(a.status, kDevBandOverflow);
      for (int j = tid; j < nb; j += 256) sh.flag[j] = 0;
      by_key = true;
    } else {
      // exact rescore of the band
      const uint16_t* qp = a.q_idx + (int64_t)r * a.q_stride;
      int lqv = INT_MAX;
      if (tid < kDim) {
        const uint32_t bits = qp[tid];
        sh.q[tid] = (double)bf16_bits_to_f32(bits);
        const uint32_t m = bits & 0x7FFFu;
        if (m) {
          const uint32_t ex = m >> 7, mant = m & 0x7Fu;
          const uint32_t M = ex ? (mant | 0x80u) : mant;
          const int e = ex ? (int)ex - 134 : -133;
          lqv = e + __builtin_ctz(M);
        }
      }
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) lqv = min(lqv, __shfl_xor(lqv, m, 64));
      if (lane == 0) sh.redi[2 + wid] = lqv;
      __syncthreads();
      const int lq = min(min(sh.redi[2], sh.redi[3]), min(sh.redi[4], sh.redi[5]));
      for (int i = 0; i < nband; ++i) {
        const double e = exact_block_score<FMT>(a, sh, b, sh.band[i], len, lq == INT_MAX ? 0 : lq);
        if (tid == 0) sh.exact[i] = e + 0.0;
      }
      __syncthreads();
      for (int i = tid; i < nband; i += 256) {
        const double ei = sh.exact[i];
        const int ji = sh.band[i];
        const uint32_t ki = th ? (uint32_t)ji : ~(uint32_t)ji;
        int rank = 0;
        for (int m = 0; m < nband; ++m) {
          const double em = sh.exact[m];
          const uint32_t km = th ? (uint32_t)sh.band[m] : ~(uint32_t)sh.band[m];
          rank += (em > ei) || (em == ei && km > ki);
        }
        if (rank < need) sh.flag[ji] = 1;
      }
    }
  }
  __syncthreads();
  if (by_key) {
    for (int j = tid; j < nb; j += 256) sh.flag[j] = comp_key(sh.key[j], j, th) >= Kk ? 1 : 0;
    __syncthreads();
  }

  // ascending compaction of the selected ids
  const int per = (nb + 255) / 256;
  const int j0 = min(nb, tid * per), j1 = min(nb, j0 + per);
  int cnt = 0;
  for (int j = j0; j < j1; ++j) cnt += sh.flag[j];
  int incl = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) sh.scan[wid] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wid; ++w) base += sh.scan[w];
  const int total = sh.scan[0] + sh.scan[1] + sh.scan[2] + sh.scan[3];
  int pos = base + incl - cnt;
  for (int j = j0; j < j1; ++j)
    if (sh.flag[j]) {
      if (pos < k) out[pos] = j;
      ++pos;
    }
  for (int i = total + tid; i < k; i += 256) out[i] = -1;
}

size_t index_ws_bytes(int32_t num_rows, int32_t max_blocks) {
  const size_t one = ((size_t)num_rows * (size_t)max_blocks * sizeof(float) + 255) & ~(size_t)255;
  return 2 * one;
}

hipError_t launch_index_topk(const IndexArgs& a0, hipStream_t stream) {
  IndexArgs a = a0;
  if (a.num_rows == 0) return hipSuccess;
  if (a.num_reqs > 0) {
    const int64_t units_upper = (int64_t)a.num_reqs * a.max_blocks;
    int64_t grid = (units_upper + 3) / 4;
    if (grid > a.scan_grid) grid = a.scan_grid;
    if (grid < 1) grid = 1;
    if (a.format == 1)
      hipLaunchKernelGGL(index_scan_kernel<1>, dim3((unsigned)grid), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(index_scan_kernel<2>, dim3((unsigned)grid), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.format == 1)
    hipLaunchKernelGGL(index_select_kernel<1>, dim3((unsigned)a.num_rows), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(index_select_kernel<2>, dim3((unsigned)a.num_rows), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace m3s
