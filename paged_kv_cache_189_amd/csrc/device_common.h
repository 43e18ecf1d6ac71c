// Device helpers shared by the HIP kernels of the library (gfx950): element
// kinds, vector types, the shape of a 16-token K/V tile in the pool, exact
// fp8 -> bf16 and round-to-nearest-even fp32 -> bf16 conversions,
// address-space views, the lazy-max threshold of the online softmax and a
// block-wide scan.  Everything sits in an unnamed namespace: each kernel
// source gets its own copy.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pkv {
namespace {

constexpr int kF32 = 0, kBF16 = 1, kFP8 = 2;
constexpr int kBS = 16;  // tokens per tile: one MFMA step; a physical block holds 1 or 2 tiles
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From& x) {
  static_assert(sizeof(To) == sizeof(From), "bitcast size");
  return __builtin_bit_cast(To, x);
}

template <int KIND>
struct ElemSize;
template <>
struct ElemSize<kF32> {
  static constexpr int value = 4;
};
template <>
struct ElemSize<kBF16> {
  static constexpr int value = 2;
};
template <>
struct ElemSize<kFP8> {
  static constexpr int value = 1;
};

template <int VB>
struct VecOf;
template <>
struct VecOf<4> {
  using T = uint32_t;
};
template <>
struct VecOf<8> {
  using T = u32x2;
};
template <>
struct VecOf<16> {
  using T = u32x4;
};

// Shape of one (block, kv head) tile and of a lane's share of it.
template <int KIND, int D>
struct Tile {
  static constexpr int ES = ElemSize<KIND>::value;
  static constexpr int BYTES = kBS * D * ES;  // one K (or V) tile
  static constexpr int NK = BYTES / 1024;      // 16-byte K loads per lane
  static constexpr int NQ = KIND == kFP8 ? 2 * NK : NK;  // 16-byte Q fragments per lane
  static constexpr int NT = D / 16;            // 16-wide d tiles of V and O
  static constexpr int VB = 4 * ES;            // V bytes per lane per d tile
  using V = typename VecOf<VB>::T;
  static_assert(NK >= 1, "tile smaller than one wave load");
};

// ---------------------------------------------------------------- conversions
// 4 E4M3 codes (one dword, byte i = element i) -> 4 bf16, exact.
__device__ __forceinline__ s16x4 fp8x4_to_bf16x4(uint32_t w) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  u32x2 r = {bitcast<uint32_t>(lo), bitcast<uint32_t>(hi)};
  return bitcast<s16x4>(r);
}

// 16 E4M3 codes -> two groups of 8 bf16 (codes 0..7 and 8..15).
__device__ __forceinline__ void fp8x16_to_bf16(const u32x4& w, u32x4& lo, u32x4& hi) {
  u32x2 a = bitcast<u32x2>(fp8x4_to_bf16x4(w.x));
  u32x2 b = bitcast<u32x2>(fp8x4_to_bf16x4(w.y));
  u32x2 c = bitcast<u32x2>(fp8x4_to_bf16x4(w.z));
  u32x2 d = bitcast<u32x2>(fp8x4_to_bf16x4(w.w));
  lo = u32x4{a.x, a.y, b.x, b.y};
  hi = u32x4{c.x, c.y, d.x, d.y};
}

// fp32 -> bf16, round to nearest even (NaN -> quiet NaN with its sign).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)(((u >> 16) & 0x8000u) | 0x7FC0u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// O^T accumulators: o[nt][i] = O^T[d = nt*16 + 4*(lane/16) + i][head lane%16].
template <int KIND, int D>
struct Acc {
  f32x4 o[Tile<KIND, D>::NT];
};

// Global-memory (address space 1) views, so loads are `global_load` with a
// scalar base, never FLAT loads (which also hold the LDS wait counter).
typedef const __attribute__((address_space(1))) char* gchar_p;
template <typename T>
using gptr = const __attribute__((address_space(1))) T*;

// Read-only kernel inputs (tables, lengths, plans) seen through the constant
// address space: uniform reads of them become scalar loads, which count on
// their own wait counter and do not hold up the K/V stream.
template <typename T>
using cptr = const __attribute__((address_space(4))) T*;
template <typename T>
__device__ __forceinline__ cptr<T> as_const(const T* p) {
  return (cptr<T>)p;
}

// A global pointer the whole wave agrees on, moved to scalar registers.
__device__ __forceinline__ gchar_p uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<gchar_p>(((uint64_t)hi << 32) | lo);
}

// The running max moves only when a block's max exceeds it by more than this
// (log2 units).  Weights are then bounded by 2^kLazyMax; numerator and
// normaliser share the same stale max, so the result is unchanged while the
// O^T rescale (32 accumulators) is skipped for almost every block.
constexpr float kLazyMax = 8.0f;

// Block-wide exclusive scan of one int per thread (blockDim.x == 64 * NWV);
// returns the prefix and writes the block total to *total.
template <int NWV>
__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_sums, int* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int k = 1; k < 64; k <<= 1) {
    const int y = __shfl_up(x, k);
    if (lane >= k) x += y;
  }
  if (lane == 63) wave_sums[wv] = x;
  __syncthreads();
  if (wv == 0) {
    int t = lane < NWV ? wave_sums[lane] : 0;
#pragma unroll
    for (int k = 1; k < NWV; k <<= 1) {
      const int y = __shfl_up(t, k);
      if (lane >= k) t += y;
    }
    if (lane < NWV) wave_sums[lane] = t;  // inclusive wave prefix
  }
  __syncthreads();
  const int base = wv > 0 ? wave_sums[wv - 1] : 0;
  *total = wave_sums[NWV - 1];
  __syncthreads();
  return base + x - v;
}

}  // namespace
}  // namespace pkv
