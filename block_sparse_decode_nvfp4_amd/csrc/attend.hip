// m3s_sparse_attend: GQA softmax attention of each row's G query heads over
// only the row's top-k blocks of the FP4 K/V cache, then a combine pass.
//
// Pages: [ATOM-2746] Summary, Attention (rows addressed through the top-k
// block ids and the request block table); [ATOM-2744] Design, Attention, and
// the review note that an invalid block id must not wrap onto a valid page.
//
// split kernel - workgroup (row, split), 8 waves, two per selected block, each
//   taking 64 of its tokens (so a split covers 4 of the row's k blocks; with
//   many more split workgroups than fit the GPU at once, each wave takes two or
//   four blocks in turn and a split covers 8 or 16). Per wave and block:
//     S^T = K Q^T on 16-bit MFMA (K tile of 16 tokens as A, the G <= 16
//       query heads as B); K is decoded exactly (NVFP4 to fp16, MXFP4 to
//       bf16).
//     online softmax in fp32 over the block's causal tokens;
//     O += P V on 16-bit MFMA: P comes out of the S^T registers as the A
//       operand; V is decoded into LDS token-major and read back transposed
//       with ds_read_b64_tr_b16 as the B operand.
//   The 8 waves merge through LDS and write one (m, l, O) partial per head.
// combine kernel - one workgroup per row merges the splits:
//   out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s (log2 domain).
// With a single split the split kernel writes the normalized output itself.
// (Merging in the split kernel's last workgroup instead needs a device-scope
// release of the partials, an L2 writeback per wave on this GPU; measured, it
// cost more than the separate launch.)
#include "attend_body.hpp"

namespace m3s {

// Two or four blocks per wave are kept to four waves per SIMD (128 VGPRs), so
// two workgroups still share a CU.
template <int FMT, int REPS>
__global__ __launch_bounds__(kWaves * 64, REPS == 1 ? 1 : 4) void attend_split_kernel(AttendArgs a) {
  __shared__ AttendShared sh;
  int r, sp;
  if (a.xcd_rows) {
    row_split_of(blockIdx.x, a.nsplit, a.num_rows, r, sp);
  } else {
    r = blockIdx.x / a.nsplit;
    sp = blockIdx.x - r * a.nsplit;
  }
  attend_split_body<FMT, REPS>(a, r, sp, sh, nullptr, nullptr, 0, 0);
}

// All partials of the row are loaded before any is used (one round trip): NS
// (4 or 16, >= nsplit) loads per thread with no branch between them, split s past
// nsplit reading split 0 again (unused). Loads guarded by a branch each were issued
// one round trip after another: the compiler waited for each split's (m, l) before
// the branch to the next split's loads.
constexpr int kMaxSplits = (64 + kBlocks - 1) / kBlocks;

// Workgroups per row of the combine for up to four splits: P = 2 takes half the row's
// heads each (128 threads), so twice the CUs issue the row's partial loads. Workgroup
// b is row b mod num_rows, half b / num_rows: when num_rows is a multiple of 8, both
// halves sit on the XCD of row r (r mod 8), where the XCD-dealt split kernel left the
// partials. Same-box A/B at 64 rows: the step 41.95 -> 41.79 us, m3s_sparse_attend
// 12.44 -> 12.32 us; P = 4 was no faster than one workgroup per row.
constexpr int kCombineWgs = 2;

template <int NS, int P = 1>
__global__ __launch_bounds__(256 / P) void attend_combine_kernel(AttendArgs a) {
  const int nr = a.num_rows;
  const int r = P == 1 ? (int)blockIdx.x : (int)blockIdx.x % nr;
  const int q = P == 1 ? 0 : (int)blockIdx.x / nr;
  const int tid = threadIdx.x;
  const int hh = q * (16 / P) + (tid >> 4), d0 = (tid & 15) * 8;
  if (hh >= a.num_heads) return;
  const int ns = a.nsplit;
  float mv[NS], lv[NS];
  f32x4 ov[NS][2];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int sl = s < ns ? s : 0;
    const float* ml = a.part_ml + (((int64_t)r * ns + sl) * 16 + hh) * 2;
    const f32x4* po = reinterpret_cast<const f32x4*>(a.part_o + (((int64_t)r * ns + sl) * 16 + hh) * kDim + d0);
    mv[s] = ml[0];
    lv[s] = ml[1];
    ov[s][0] = po[0];
    ov[s][1] = po[1];
  }
  // no branch between the loads and their use either (a branch lets the compiler sink
  // the O loads past the wait for m): splits past nsplit get weight 0, and a row with
  // no causal token (every m = -inf) gets weights 2^-inf = 0
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < NS; ++s) M = fmaxf(M, s < ns ? mv[s] : -INFINITY);
  const float Mr = M == -INFINITY ? 0.f : M;
  float L = 0.f;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float f = s < ns ? __builtin_amdgcn_exp2f(mv[s] - Mr) : 0.f;
    L += f * lv[s];
    acc0 += f * ov[s][0];
    acc1 += f * ov[s][1];
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  f32x4* dst = reinterpret_cast<f32x4*>(a.out + ((int64_t)r * a.num_heads + hh) * kDim + d0);
  bool bad = false;
  f32x4 o0, o1;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o0[e] = finite_or_zero(acc0[e] * inv, bad);
    o1[e] = finite_or_zero(acc1[e] * inv, bad);
  }
  dst[0] = o0;
  dst[1] = o1;
  if (bad) set_status(a.status, kDevRange);
}

int32_t attend_nsplit(int32_t topk) { return (topk + kBlocks - 1) / kBlocks; }

size_t attend_ws_bytes(int32_t num_rows, int32_t nsplit) {
  if (nsplit <= 1) return 0;
  const size_t po = ((size_t)num_rows * nsplit * 16 * kDim * sizeof(float) + 255) & ~(size_t)255;
  const size_t ml = ((size_t)num_rows * nsplit * 16 * 2 * sizeof(float) + 255) & ~(size_t)255;
  return po + ml;
}

hipError_t launch_sparse_attend(const AttendArgs& a, hipStream_t stream) {
  if (a.num_rows == 0) return hipSuccess;
  const unsigned grid = (unsigned)((int64_t)a.num_rows * a.nsplit);
  if (a.reps == 4) {
    if (a.format == 1)
      hipLaunchKernelGGL((attend_split_kernel<1, 4>), dim3(grid), dim3(kWaves * 64), 0, stream, a);
    else
      hipLaunchKernelGGL((attend_split_kernel<2, 4>), dim3(grid), dim3(kWaves * 64), 0, stream, a);
  } else if (a.reps == 2) {
    if (a.format == 1)
      hipLaunchKernelGGL((attend_split_kernel<1, 2>), dim3(grid), dim3(kWaves * 64), 0, stream, a);
    else
      hipLaunchKernelGGL((attend_split_kernel<2, 2>), dim3(grid), dim3(kWaves * 64), 0, stream, a);
  } else {
    if (a.format == 1)
      hipLaunchKernelGGL((attend_split_kernel<1, 1>), dim3(grid), dim3(kWaves * 64), 0, stream, a);
    else
      hipLaunchKernelGGL((attend_split_kernel<2, 1>), dim3(grid), dim3(kWaves * 64), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  return launch_attend_combine(a, stream);
}

hipError_t launch_attend_combine(const AttendArgs& a, hipStream_t stream) {
  if (a.nsplit <= 4)
    hipLaunchKernelGGL((attend_combine_kernel<4, kCombineWgs>), dim3((unsigned)a.num_rows * kCombineWgs), dim3(256 / kCombineWgs), 0, stream, a);
  else
    hipLaunchKernelGGL(attend_combine_kernel<kMaxSplits>, dim3((unsigned)a.num_rows), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace m3s
