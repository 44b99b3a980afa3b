// The store's per-row body (quantize one 128-element bf16 row and write it at its
// slot), shared by the m3s_store kernels and the decode step's scan kernel.
// 16 lanes per row, 8 elements (one 16-byte load) per lane; row index
// rr = token * 3 + tensor (K, V, index K). A row is split in two: store_issue
// issues its loads (the slot and the bf16 row, independent of each other) and
// store_commit quantizes and writes, so that a workgroup can have several rows'
// loads in flight before it waits for any.
#pragma once

#include "fp4.hpp"
#include "launch.hpp"
#include "quant.hpp"

namespace m3s {

struct StoreLoad {
  u32x4 raw;
  int64_t rr;    // -1: no row
  int32_t slot;  // -1: not loaded
};

// The row's tensor pointers are chosen among values held in scalar registers: left to
// the compiler, the choice by a per-lane index became a vector load from the kernel's
// argument block, a dependent round trip ahead of the row's own loads.
__device__ __forceinline__ const uint16_t* store_src(const StoreArgs& a, int ten) {
  const uint16_t* k = a.k;
  const uint16_t* v = a.v;
  const uint16_t* x = a.idx;
  asm volatile("" : "+s"(k), "+s"(v), "+s"(x));
  return ten == 0 ? k : (ten == 1 ? v : x);
}

// Loads of row rr (rr < 0: none). Every lane of the row's 16-lane group calls it.
__device__ __forceinline__ void store_issue(const StoreArgs& a, int64_t rr, int lane16, StoreLoad& ld) {
  ld.rr = rr;
  ld.slot = -1;
  ld.raw = {0u, 0u, 0u, 0u};
  if (rr < 0) return;
  const int64_t tok = rr / 3;
  const uint16_t* src = store_src(a, (int)(rr - tok * 3));
  if (tok < a.num_tokens && src != nullptr) {
    ld.slot = a.slots[tok];
    ld.raw = *reinterpret_cast<const u32x4*>(src + tok * a.row_stride + 8 * lane16);
  }
}

// Quantize and write a row whose loads store_issue issued (every lane of the group
// calls it, also for no row: the quantizer exchanges values across the group).
template <int FMT>
__device__ __forceinline__ void store_commit(const StoreArgs& a, int lane16, const StoreLoad& ld) {
  const int64_t tok = ld.rr >= 0 ? ld.rr / 3 : 0;
  const int ten = ld.rr >= 0 ? (int)(ld.rr - tok * 3) : 0;
  bool live = ld.slot >= 0;
  if (live && (int64_t)ld.slot >= (int64_t)a.num_pages * kPage) {
    if (lane16 == 0) set_status(a.status, kDevBadSlot);
    live = false;
  }
  uint32_t bits[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bits[2 * i] = ld.raw[i] & 0xFFFFu;
    bits[2 * i + 1] = ld.raw[i] >> 16;
  }
  uint32_t packed, scale_byte;
  quantize_lane<FMT>(bits, packed, scale_byte);
  if (live) {
    uint8_t* kd = a.k_data;
    uint8_t* vd = a.v_data;
    uint8_t* xd = a.idx_data;
    uint8_t* ks = a.k_scale;
    uint8_t* vs = a.v_scale;
    uint8_t* xs = a.idx_scale;
    asm volatile("" : "+s"(kd), "+s"(vd), "+s"(xd), "+s"(ks), "+s"(vs), "+s"(xs));
    uint8_t* dd = ten == 0 ? kd : (ten == 1 ? vd : xd);
    uint8_t* ds = ten == 0 ? ks : (ten == 1 ? vs : xs);
    write_lane<FMT>(dd, ds, ld.slot, lane16, packed, scale_byte);
  }
}

// Row rr of the store (every lane of the row's 16-lane group calls it together).
template <int FMT>
__device__ __forceinline__ void store_row(const StoreArgs& a, int64_t rr, int lane16) {
  StoreLoad ld;
  store_issue(a, rr, lane16, ld);
  store_commit<FMT>(a, lane16, ld);
}

// The 16 rows of store block `block` (a 256-thread workgroup).
template <int FMT>
__device__ __forceinline__ void store_body(const StoreArgs& a, int64_t block) {
  store_row<FMT>(a, block * 16 + (threadIdx.x >> 4), threadIdx.x & 15);
}

}  // namespace m3s
