// The split pass of the sparse attention as a device function, shared by the
// m3s_sparse_attend split kernel and the fused top-k + attention kernel.
// Workgroup (row, split): 8 waves, two per selected block, each taking 64 of
// its tokens (so a split covers 4 of the row's k blocks). Per wave:
//   S^T = K Q^T on 16-bit MFMA (K tile of 16 tokens as A, the G <= 16 query
//     heads as B); K is decoded exactly: NVFP4 to fp16 (the query scaled by a
//     power of two into fp16 range), MXFP4 to bf16 (the bf16 query as is),
//     since only bf16 holds code * 2^(b - 127) for every E8M0 byte.
//   online softmax in fp32 over the block's causal tokens;
//   O += P V on 16-bit MFMA: P comes out of the S^T registers as the A
//     operand (NVFP4: one fp16 term; MXFP4: P = hi + lo, two bf16 terms and
//     two MFMAs, so P keeps 16 significant bits); V is decoded into LDS
//     token-major and read back transposed with ds_read_b64_tr_b16 as the B
//     operand.
// An output element that is not finite in fp32 (a logit or sum beyond the
// fp32 range, e.g. MXFP4 scale bytes 253 and 254, which no store writes) is
// written as 0 and sets the range status bit.
// The 8 waves merge through LDS and write one (m, l, O) partial per head (or,
// with a single split, the normalized output).
#pragma once

#include <float.h>

#include "fp4.hpp"
#include "launch.hpp"

namespace m3s {

typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kBlocks = 4;                  // selected blocks per split (workgroup)
constexpr int kHalves = 2;                  // waves per block
constexpr int kWaves = kBlocks * kHalves;   // 8
constexpr int kTiles = 8 / kHalves;         // 16-token tiles per wave
constexpr int kVRow = kDim + 8;  // LDS row of one token's decoded V (fp16), padded
constexpr int kVChunk = 32;      // tokens of V staged per step (one MFMA k-step)

struct AttendShared {
  union {
    _Float16 v[kWaves][kVChunk][kVRow];       // 69,632 B
    struct {
      float o[kWaves][16][kDim];              // 65,536 B
      float m[kWaves][16];
      float l[kWaves][16];
    } mrg;
  };
};

__device__ __forceinline__ s16x4 lds_tr16(const _Float16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) void*)p));
}

// B operand of 8 16-bit values from two transposing reads (bits as read).
template <typename OP>
__device__ __forceinline__ OP tr16_pair(s16x4 lo, s16x4 hi) {
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(OP, v);
}

__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) { return mfma_f16(a, b, c); }
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) { return mfma_bf16(a, b, c); }

// An output value, or 0 with the range flag set when it is not finite.
__device__ __forceinline__ float finite_or_zero(float v, bool& bad) {
  const bool ok = __builtin_isfinite(v);
  bad |= !ok;
  return ok ? v : 0.f;
}

// Workgroup b of a (row, split) grid -> its row and split, with all splits of a
// row on one XCD. The 8 XCDs take a launch's workgroups round-robin, so rows are
// dealt in groups of 8, one row per XCD, its splits 8 workgroups apart. A row's
// splits then share that XCD's L2 for the row's common inputs, and the combine
// workgroup of row r (workgroup r: XCD r mod 8) finds the row's partials there.
// Rows past the last full group of 8 take the plain row-major order. Used by the
// split kernel when all its workgroups are resident at once (xcd_rows).
__device__ __forceinline__ void row_split_of(int b, int nsplit, int num_rows, int& r, int& sp) {
  const int grp = 8 * nsplit;
  const int full = num_rows >> 3;
  const int g = b / grp;
  if (g < full) {
    const int o = b - g * grp;
    r = 8 * g + (o & 7);
    sp = o >> 3;
  } else {
    const int t = b - full * grp;
    r = 8 * full + t / nsplit;
    sp = t - (t / nsplit) * nsplit;
  }
}

// Split (row r, split sp) of the attention, run by kWaves waves. The selected
// block ids come from topk_ids and their pages from the block table, or from
// sel_pages when the select wrote them (loaded beside the ids: no dependent
// lookup), or, when s_ids is given (the select ran in the same workgroup), the
// ids, their pages and the row's request and length come from the caller (LDS /
// registers). LDS_IDS: the caller passes s_ids (the fused kernel); the paths that read
// the ids and pages from global memory are then not compiled, so no wait for them (or
// for the query loads issued before them) stands between the ids and the K/V loads.
template <int FMT, int REPS = 1, bool LDS_IDS = false>
__device__ __forceinline__ void attend_split_body(const AttendArgs& a, int r, int sp, AttendShared& sh,
                                                  const int* s_ids, const int* s_pages, int b_in, int len_in) {
  constexpr int SB = FMT == 1 ? 8 : 4;
  typedef Decode<FMT> Dec;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = lane & 15, G = lane >> 4;
  const int half = w % kHalves;  // tokens [64 half, 64 half + 64) of the block

  // ---- which blocks this wave attends; the row map, the ids and the query are
  // independent loads, issued together
  const int b = LDS_IDS ? b_in : a.row_req[r];
  const int len = LDS_IDS ? len_in : a.row_len[r];
  int id[REPS], pg_sel[REPS];
#pragma unroll
  for (int rep = 0; rep < REPS; ++rep) {
    const int slot = (sp * REPS + rep) * kBlocks + w / kHalves;
    if constexpr (LDS_IDS) {
      id[rep] = slot < a.topk ? s_ids[slot] : -1;
      pg_sel[rep] = -1;
    } else {
      id[rep] = slot < a.topk ? a.topk_ids[(int64_t)r * a.topk + slot] : -1;
      pg_sel[rep] = (a.sel_pages && slot < a.topk) ? a.sel_pages[(int64_t)r * a.topk + slot] : -1;
    }
  }
  u32x4 raw[4] = {};
  if (n < a.num_heads) {
    const uint16_t* qp = a.q + (int64_t)r * a.q_row_stride + (int64_t)n * a.q_head_stride + 32 * G;
#pragma unroll
    for (int s = 0; s < 4; ++s) raw[s] = *reinterpret_cast<const u32x4*>(qp + 8 * s);
  }
  int page[REPS], blk[REPS];
#pragma unroll
  for (int rep = 0; rep < REPS; ++rep) {
    const int slot = (sp * REPS + rep) * kBlocks + w / kHalves;
    page[rep] = -1;
    blk[rep] = -1;
    if (b >= 0 && len > 0 && slot < a.topk) {
      const int nbr = (len + kPage - 1) / kPage;
      if (id[rep] >= 0) {
        if (id[rep] >= nbr || id[rep] >= a.max_blocks) {
          if (lane == 0) set_status(a.status, kDevBadBlockId);
        } else {
          int pg;
          if constexpr (LDS_IDS) pg = s_pages[slot];
          else pg = a.sel_pages ? pg_sel[rep] : a.block_table[(int64_t)b * a.bt_stride + id[rep]];
          if (pg < 0 || pg >= a.num_pages) {
            if (lane == 0) set_status(a.status, kDevBadPage);
          } else {
            page[rep] = pg;
            blk[rep] = id[rep];
          }
        }
      }
    }
  }

  // ---- query heads as the B operand, the same for all of the wave's blocks: NVFP4
  // scaled by 2^P into fp16 range (built once per wave); MXFP4 the bf16 values as they
  // are. With one block per wave it is built after the block's K/V loads are issued,
  // so that waiting for the query does not hold them back; with several blocks, before
  // the first block (measured faster there).
  typedef typename Dec::op_t op_t;
  op_t qop[4];
  float c = 0.f;  // logits in log2 units: x = S' * c
  auto build_qop = [&]() {
    if constexpr (FMT == 1) {
      uint32_t mx = 0;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) mx = max(mx, max(raw[s][q4] & 0x7FFFu, (raw[s][q4] >> 16) & 0x7FFFu));
      mx = lane_max<1, 64>(mx);
      int P = 0;
      if (mx) {
        const uint32_t ex = mx >> 7, mant = mx & 0x7Fu;
        const int fl = ex ? (int)ex - 127 : (31 - __builtin_clz(mant)) - 133;
        P = 13 - fl;
        P = P > 64 ? 64 : (P < -64 ? -64 : P);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t bits = (e & 1) ? (raw[s][e >> 1] >> 16) : (raw[s][e >> 1] & 0xFFFFu);
          qop[s][e] = (_Float16)__builtin_ldexpf(bf16_bits_to_f32(bits), P);
        }
      c = a.sm_scale * 1.4426950408889634f * __builtin_ldexpf(1.0f, -P);
    }
  };
  if constexpr (REPS > 1) build_qop();

  float m_run = -INFINITY, l_run = 0.f;  // per head n (replicated over G)
  f32x4 o[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- the wave's blocks, one after another (REPS > 1: online softmax across them)
#pragma unroll
  for (int rep = 0; rep < REPS; ++rep) {
    const bool active = page[rep] >= 0;

    if (active) {
      // ---- K and V loads for the whole block (lane: token 16 i + n, dims [32G, 32G + 32))
      const uint8_t* kp = a.k_data + (int64_t)page[rep] * (kPage * kPayload);
      const uint8_t* vp = a.v_data + (int64_t)page[rep] * (kPage * kPayload);
      const uint8_t* ksp = a.k_scale + (int64_t)page[rep] * (kPage * SB);
      const uint8_t* vsp = a.v_scale + (int64_t)page[rep] * (kPage * SB);
      u32x4 kr[kTiles];
      uint32_t ks[kTiles];
      const int t0 = 16 * kTiles * half;  // first token of the wave's tiles
#pragma unroll
      for (int i = 0; i < kTiles; ++i)
        kr[i] = *reinterpret_cast<const u32x4*>(kp + (t0 + 16 * i + n) * kPayload + 16 * G);
#pragma unroll
      for (int i = 0; i < kTiles; ++i) {
        if (FMT == 1) ks[i] = *reinterpret_cast<const uint16_t*>(ksp + (t0 + 16 * i + n) * SB + 2 * G);
        else ks[i] = ksp[(t0 + 16 * i + n) * SB + G];
      }

      // ---- V loads, issued with the K loads (same lane mapping)
      u32x4 vr[kTiles];
      uint32_t vs[kTiles];
#pragma unroll
      for (int i = 0; i < kTiles; ++i)
        vr[i] = *reinterpret_cast<const u32x4*>(vp + (t0 + 16 * i + n) * kPayload + 16 * G);
#pragma unroll
      for (int i = 0; i < kTiles; ++i) {
        if (FMT == 1) vs[i] = *reinterpret_cast<const uint16_t*>(vsp + (t0 + 16 * i + n) * SB + 2 * G);
        else vs[i] = vsp[(t0 + 16 * i + n) * SB + G];
      }

      if constexpr (REPS == 1) build_qop();
      if constexpr (FMT == 2) {  // MXFP4: the bf16 words as they are, set per block (set once before the loop, the two-block build spills)
#pragma unroll
        for (int s = 0; s < 4; ++s) qop[s] = __builtin_bit_cast(bf16x8, raw[s]);
        c = a.sm_scale * 1.4426950408889634f;
      }
      // ---- S^T tiles: st[i][v] = logit of token t0 + 16 i + 4 G + v for head n
      f32x4 st[kTiles];
#pragma unroll
      for (int i = 0; i < kTiles; ++i) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        typename Dec::scale_t s0, s1;
        Dec::scales(ks[i], s0, s1);
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma16(Dec::run(kr[i][s], s < 2 ? s0 : s1), qop[s], acc);
        st[i] = acc * c;
      }
      const int tok_base = blk[rep] * kPage + t0;
      if (tok_base + 16 * kTiles > len) {
#pragma unroll
        for (int i = 0; i < kTiles; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (tok_base + 16 * i + 4 * G + v >= len) st[i][v] = -INFINITY;
      }
      float mx_l = -INFINITY;
#pragma unroll
      for (int i = 0; i < kTiles; ++i) mx_l = fmaxf(mx_l, fmaxf(fmaxf(st[i][0], st[i][1]), fmaxf(st[i][2], st[i][3])));
      mx_l = lane_fmax<16, 64>(mx_l);
      // a wave's 64 tokens can all lie past the row's length: it then stays empty
      if (tok_base < len) {
        // mx_l is finite: the wave's tokens include a causal one. Over several
        // blocks the running sum and O are rescaled to a new running max, but only
        // when some head's block maximum exceeds its running max by more than 2^8:
        // otherwise the running max stays (the weights are then below 2^8, in range
        // for the 16-bit P operand, and the sums are the same up to rounding) and the
        // rescale is skipped. The decision is the wave's, so O is rescaled for all
        // heads or none.
        const bool grow = REPS == 1 || rep == 0 || __builtin_amdgcn_ballot_w64(mx_l > m_run + 8.f) != 0;
        const float m_new = REPS == 1 ? mx_l : (grow ? fmaxf(m_run, mx_l) : m_run);
        float lsum = 0.f;
#pragma unroll
        for (int i = 0; i < kTiles; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float p = __builtin_amdgcn_exp2f(st[i][v] - m_new);
            st[i][v] = p;
            lsum += p;
          }
        lsum = lane_sum<16, 64>(lsum);
        if (REPS == 1 || rep == 0) {  // the wave's first block: nothing to rescale
          l_run = lsum;
        } else if (!grow) {
          l_run += lsum;
        } else {
          const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // head n; 0 while m_run is -inf
          l_run = l_run * alpha + lsum;
          // o[t][v] is head 4G + v: its factor comes from lane 4G + v (n = 4G + v)
          float av[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) av[v] = __shfl(alpha, 4 * G + v, 64);
#pragma unroll
          for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) o[t][v] *= av[v];
        }
        m_run = m_new;

        // ---- O += P V, kVChunk tokens staged per step, 32 per MFMA
        _Float16(*vb)[kVRow] = sh.v[w];
#pragma unroll
        for (int cidx = 0; cidx < 16 * kTiles / kVChunk; ++cidx) {
#pragma unroll
          for (int h4 = 0; h4 < kVChunk / 16; ++h4) {
            const int i = (kVChunk / 16) * cidx + h4;
            typename Dec::scale_t s0, s1;
            Dec::scales(vs[i], s0, s1);
            _Float16* dst = &vb[16 * h4 + n][32 * G];
#pragma unroll
            for (int s = 0; s < 4; ++s)
              *reinterpret_cast<op_t*>(dst + 8 * s) = Dec::run(vr[i][s], s < 2 ? s0 : s1);
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
          for (int ks = 0; ks < kVChunk / 32; ++ks) {
            const int i0 = (kVChunk / 16) * cidx + 2 * ks;
            // A operand: head n, tokens {4G..4G+3} of tile i0 then of tile i0 + 1
            // B operand for N tile t: V[those 8 tokens][16 t + n]; lane n of a 16-lane
            // group points at token (4G + n / 4), dims 16 t + 4 (n % 4) .. + 3.
            const int r0 = 32 * ks + 4 * G + (n >> 2);
            if constexpr (FMT == 1) {
              f16x8 pa;
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                pa[v] = (_Float16)st[i0][v];
                pa[4 + v] = (_Float16)st[i0 + 1][v];
              }
#pragma unroll
              for (int t = 0; t < 8; ++t) {
                const f16x8 bv = tr16_pair<f16x8>(lds_tr16(&vb[r0][16 * t + 4 * (n & 3)]),
                                                  lds_tr16(&vb[r0 + 16][16 * t + 4 * (n & 3)]));
                o[t] = mfma_f16(pa, bv, o[t]);
              }
            } else {
              // P = hi + lo in bf16 (the remainder is exact in fp32): 16 significant bits
              bf16x8 ph, pl;
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                const float p0 = st[i0][v], p1 = st[i0 + 1][v];
                const __bf16 h0 = (__bf16)p0, h1 = (__bf16)p1;
                ph[v] = h0;
                ph[4 + v] = h1;
                pl[v] = (__bf16)(p0 - (float)h0);
                pl[4 + v] = (__bf16)(p1 - (float)h1);
              }
#pragma unroll
              for (int t = 0; t < 8; ++t) {
                const bf16x8 bv = tr16_pair<bf16x8>(lds_tr16(&vb[r0][16 * t + 4 * (n & 3)]),
                                                    lds_tr16(&vb[r0 + 16][16 * t + 4 * (n & 3)]));
                o[t] = mfma_bf16(ph, bv, o[t]);
                o[t] = mfma_bf16(pl, bv, o[t]);
              }
            }
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        }
      }
    }
  }

  // ---- merge the waves: o[t][v] is head 4G + v, dim 16 t + n
  __syncthreads();
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) sh.mrg.o[w][4 * G + v][16 * t + n] = o[t][v];
  if (G == 0) {
    sh.mrg.m[w][n] = m_run;
    sh.mrg.l[w][n] = l_run;
  }
  __syncthreads();
  // thread: head tid / kPerHead, kOut dims from (tid % kPerHead) * kOut
  constexpr int kOut = 16 * kDim / (64 * kWaves);
  constexpr int kPerHead = kDim / kOut;
  const int tid = threadIdx.x;
  const int hh = tid / kPerHead;
  const int d0 = (tid % kPerHead) * kOut;
  float M = -INFINITY;
#pragma unroll
  for (int q = 0; q < kWaves; ++q) M = fmaxf(M, sh.mrg.m[q][hh]);
  float L = 0.f;
  float acc[kOut];
#pragma unroll
  for (int e = 0; e < kOut; ++e) acc[e] = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int q = 0; q < kWaves; ++q) {
      const float f = __builtin_amdgcn_exp2f(sh.mrg.m[q][hh] - M);
      L += f * sh.mrg.l[q][hh];
#pragma unroll
      for (int e = 0; e < kOut; ++e) acc[e] += f * sh.mrg.o[q][hh][d0 + e];
    }
  }
  if (hh < a.num_heads) {
    if (a.nsplit == 1) {
      const float inv = L > 0.f ? 1.0f / L : 0.f;
      float* dst = a.out + ((int64_t)r * a.num_heads + hh) * kDim + d0;
      bool bad = false;
#pragma unroll
      for (int e = 0; e < kOut; ++e) dst[e] = finite_or_zero(acc[e] * inv, bad);
      if (bad) set_status(a.status, kDevRange);
    } else {
      float* dst = a.part_o + (((int64_t)r * a.nsplit + sp) * 16 + hh) * kDim + d0;
#pragma unroll
      for (int e = 0; e < kOut; ++e) dst[e] = acc[e];
      if (tid % kPerHead == 0) {
        float* ml = a.part_ml + (((int64_t)r * a.nsplit + sp) * 16 + hh) * 2;
        ml[0] = M;
        ml[1] = L;
      }
    }
  }
}

}  // namespace m3s
