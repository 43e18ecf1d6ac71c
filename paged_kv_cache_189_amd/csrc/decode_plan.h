// Work division of paged decode attention, shared by the plan, pass-1 and
// merge kernels (kernels.hip, decode_merge.hip).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

// ---------------------------------------------------------------- planning
// Work division, rebuilt on the device every call from context_lens.  All
// (kv head, sequence) pairs lie on one line, head major: pair P = g * S + s
// holds blocks [g*T + cb[s], g*T + cb[s+1]) of it, T = blocks of one head
// (cb = prefix sums of blocks per sequence).  The line is cut into R equal
// ranges of blocks, one per pass-1 wave.  Segments are the pieces between
// cut points: pair starts, range starts, and (with partitions) every
// part_blocks blocks from a pair's start.  The segment starting at position
// x has slot  K(x) + range_of(x),  K(x) = global index of the partition
// holding x (cp = prefix sums of partitions per sequence; a pair without
// partition cuts is one partition).  Every cut raises K or the range index,
// so slots grow strictly along the line: unique, and below
// partitions + R.  A pair inside one range and one partition is finished in
// pass 1; the others leave one partial state per segment for pass 2.
__device__ __forceinline__ int64_t range_start(int64_t r, int64_t total, int R) {
  return r * total / R;
}
// The last range starting at or before block position x (0 <= x < total).
__device__ __forceinline__ int range_of(int64_t x, int64_t total, int R) {
  return (int)(((x + 1) * R + total - 1) / total) - 1;
}
__device__ __forceinline__ int seq_blocks(const DecodeArgs& a, int s) {
  int L = a.context_lens[s];
  L = L < 0 ? 0 : (L > a.max_context_len ? a.max_context_len : L);
  return (L + kBS - 1) / kBS;
}
__device__ __forceinline__ int parts_of(int nblk, int pb) {
  return pb > 0 ? (nblk + pb - 1) / pb : (nblk > 0 ? 1 : 0);
}

}  // namespace
}  // namespace pkv
