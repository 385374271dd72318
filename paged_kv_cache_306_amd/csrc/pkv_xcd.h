// Workgroup slots to work units for the decode attention launches, weighted between the
// XCDs of the chip (host and device).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// The dispatcher deals workgroup b to XCD b % 8, and each XCD holds as many workgroups at
// once as any other.  Where the even XCDs stream K/V faster than the odd ones, units are
// dealt in proportion: over the longest-first unit list, unit g goes to the even XCDs iff
// floor((g + 1) P / 1024) > floor(g P / 1024), P = `split`, so both halves of the chip move
// through the list at the same relative pace, each in list order.  Inside a half, position
// pos goes to XCD pair member pos % 4 as its (pos / 4)-th workgroup, so slot b = 8 k + x runs
// position 4 k + x / 2 of half x % 2.  Every unit lands in exactly one slot; slots past a
// half's share get -1 (nothing to do).
constexpr int kXcds = 8;
constexpr int64_t kXcdSplitOne = 1024;  // split P is a fraction of this; P = 512: no bias

__host__ __device__ inline int64_t xcd_slot_unit(int64_t slot, int64_t units, int split) {
  const int64_t x = slot % kXcds, k = slot / kXcds;
  const int64_t pos = (kXcds / 2) * k + (x >> 1);
  // even half: the pos-th g with floor((g + 1) P / Q) = pos + 1, i.e. ceil((pos + 1) Q / P) - 1;
  // odd half: the pos-th g with (g + 1) - floor((g + 1) P / Q) = pos + 1, floor(pos Q / (Q - P))
  const int64_t g = (x & 1) == 0 ? ((pos + 1) * kXcdSplitOne + split - 1) / split - 1
                                 : pos * kXcdSplitOne / (kXcdSplitOne - split);
  return g < units ? g : -1;
}

// Workgroups a launch of `units` units needs under `split` (0 < split < 1024).
__host__ __device__ inline int64_t xcd_grid(int64_t units, int split) {
  const int64_t even = units * split / kXcdSplitOne, odd = units - even;
  const int64_t most = even > odd ? even : odd;
  return kXcds * ((most + kXcds / 2 - 1) / (kXcds / 2));
}

}  // namespace pkv
