// Device helpers shared by the gfx950 decode kernels (decode_fast.hip), and
// in part by the dense and prefill kernels: the cache-row slot layout in LDS,
// the DMA and L2-touch loads, the LDS operand reads and the cross-lane
// reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "mla_internal.h"

namespace mla {
namespace dec {

constexpr int kRowBytes = kDq * 2;                 // 1152: one cached row [c^KV | k^R]
constexpr int kSliceTok = 32;                      // tokens per LDS slot
constexpr int kSlotBytes = kSliceTok * kRowBytes;  // 36,864
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Slot layout: 4 x 9 tiles of 8 rows x 128 bytes.  Row t, logical 16-byte
// chunk c sits at (9 (t / 8) + c / 8) KiB + 128 (t % 8) + 16 ((c % 8) ^ swz(t));
// rows t and t + 16 are kRowGroup2 bytes apart.
constexpr uint32_t kTileRowGroup = 9 * 1024;
constexpr uint32_t kRowGroup2 = 2 * kTileRowGroup;

#define MLA_VMCNT(n) (((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

// Row swizzle: logical 16-byte chunk `ch` of LDS row `t` sits at chunk position
// ch ^ swz(t), a permutation inside aligned groups of 8 chunks (a row has 72).
// LDS has 64 four-byte banks; a 1152-byte row moves the bank position by half
// of the 256-byte period, so row parity picks the half.  How gfx950 services a
// wave (measured with the SQ_LDS_BANK_CONFLICT counter): ds_read_b128 takes 16
// lanes per cycle, namely the lanes of one half-wave whose lane-index bits 2..4
// have equal parity; ds_read_b64_tr_b16 takes one half-wave per cycle.
// With swz(t) = 2 ((t >> 1) & 3):
//  * QK^T reads, lane 16g + q reading row q, chunk 4k + g: in one cycle
//    (q0, g0, q1 ^ g1, q2) takes all 16 values, so the 16 lanes hit 16
//    distinct bank groups;
//  * PV reads, row 4g + q/4, chunk 2c + q1, half q0: over a half-wave the
//    8-byte bank pair (q2, q1, q3 ^ c0, g0 ^ c1, q0) takes all 32 values.
__device__ __forceinline__ int swz(int t) { return ((t >> 1) & 3) << 1; }

// Maximum / sum over the four lanes q, q+16, q+32, q+48 (the 16-lane rows of
// a wave) with the gfx950 row-swap permutes: v_permlane16_swap exchanges rows
// 0<->1 and 2<->3 between its two operands, v_permlane32_swap the two halves.
__device__ __forceinline__ float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 16 bytes per lane from `base + voff` into LDS at m0 + 16 * lane.  (The
// instruction's immediate offset is left at 0: it would move the LDS
// destination as well.)  The compiler cannot count these loads: every use of
// the data waits with an explicit s_waitcnt vmcnt.
#ifndef MLA_DMA_POLICY
#define MLA_DMA_POLICY ""
#endif
__device__ __forceinline__ void dma16(const char* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, %1" MLA_DMA_POLICY ::"v"(voff), "s"(base), "{m0}"(lds_addr)
               : "memory");
}

// The same with the non-temporal bit (rows with a single reader).
__device__ __forceinline__ void dma16_nt(const char* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(base), "{m0}"(lds_addr) : "memory");
}

// 4 bytes per lane from `base + voff` into LDS at m0 + 4 * lane: used only to
// pull rows into the L2 ahead of their DMA (the LDS bytes are never read).  No
// register receives the data, so nothing waits for it until the epilogue.
__device__ __forceinline__ void touch4(const char* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("global_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds_addr) : "memory");
}

__device__ __forceinline__ bf16x8 lds_read128(const char* lds, uint32_t off) {
  return *reinterpret_cast<const bf16x8*>(lds + off);
}

__device__ __forceinline__ bf16x4 lds_read_tr(const char* lds, uint32_t off) {
  short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4_t*)((__attribute__((address_space(3))) const char*)lds + off));
  return __builtin_bit_cast(bf16x4, v);
}

template <typename T>
__device__ __forceinline__ uint32_t lds_addr_of(T* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) T*)p));
}

// Work item and query token of a workgroup: an item has `per` workgroups
// (its query tokens, times `halves` head halves), numbered so that all of an
// item's workgroups run on one XCD (blocks go to the XCDs round-robin) and
// are dispatched together: blocks 8 per m + 8 r + j (j < 8, r < per) take part r
// of item 8m + j; a last incomplete group of items is laid out the same way
// over the blocks that remain.
__device__ __forceinline__ void block_to_item(int blk, int num_items, int per, int& it, int& part) {
  const int full = num_items & ~7;
  if (blk < per * full) {
    it = (blk / (8 * per)) * 8 + (blk & 7);
    part = (blk >> 3) % per;
  } else {
    const int j = blk - per * full, rest = num_items - full;
    it = full + j % rest;
    part = j / rest;
  }
}

// The work item of dispatch slot `slot`: with a dispatch order the record of
// item `slot` is read together with order[slot] (longest-first orders are
// mostly the identity), and only a slot that holds another item reads that
// item's record after the order arrives.  On return `slot` is the item.
__device__ __forceinline__ void load_item(const int32_t* items, const int32_t* order, int& slot,
                                          int& b, int& p0, int& p1) {
  b = items[4 * slot];
  p0 = items[4 * slot + 2];
  p1 = items[4 * slot + 3];
  if (order) {
    const int o = order[slot];
    if (o != slot) {
      slot = o;
      b = items[4 * o];
      p0 = items[4 * o + 2];
      p1 = items[4 * o + 3];
    }
  }
}

// Table entry of the item's first page, read as soon as the item is known:
// an ordered (relaxed) load stays where it is written, so it is in flight
// together with the sequence length instead of after the checks that need
// the length.
__device__ __forceinline__ int first_page(const int32_t* bt, int p0) {
  return __hip_atomic_load(bt + p0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace dec
}  // namespace mla
