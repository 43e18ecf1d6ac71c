// The KV cache write and the device block copy for CDNA4 (gfx950).
//
// A new token's K and V are appended to its sequence by writing them into the
// slot the block manager assigned ("Optimizing Llama 3.1 405B Inference with
// vLLM PagedAttention", PagedAttention Mechanics); an fp8 cache stores the
// E4M3 code of each value ("vLLM PagedAttention Optimization: Complete
// Step-by-Step Tuning Guide for Low-Latency Inference", Step 3).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

// fp32 -> OCP E4M3FN code, satfinite round to nearest even: magnitudes at or
// beyond 448 (infinity included) give +-448, NaN gives NaN.  Integer form:
// below 2^-6 the code is the integer nearest to |x| * 2^9 (ties to even);
// above, the fp32 mantissa is rounded to 3 bits and a carry moves into the
// exponent field, which is what the code's bit layout expects.
__device__ __forceinline__ uint8_t f32_to_e4m3_sat(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return (uint8_t)(sign | 0x7Fu);
  if (a >= 0x43E00000u) return (uint8_t)(sign | 0x7Eu);  // 448
  if (a < 0x3C800000u) {                                  // 2^-6
    float f = __uint_as_float(a) * 512.0f;                // exact
    return (uint8_t)(sign | (uint32_t)__builtin_rintf(f));
  }
  uint32_t code = (((a >> 23) - 120u) << 3) | ((a >> 20) & 7u);
  uint32_t rem = a & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (code & 1u))) code += 1u;
  return (uint8_t)(sign | code);
}

// ---------------------------------------------------------------- cache write
// One workgroup per new token; threads stride over (kv head, 16-byte chunk).
// With B = block_size: K chunk c of head h goes to block[h][c][slot % B][0..X);
// V element d goes to block[h][d][slot % B].  As a decode append (tables
// given), token t is sequence t's token at position p = context_lens[t] - 1
// and entry p / B of its table row is set to the slot's block, the value the
// host block manager holds there.
template <int SRC, int CACHE, int D>
__global__ __launch_bounds__(128) void cache_write_kernel(CacheWriteArgs a) {
  constexpr int ES = ElemSize<CACHE>::value;
  constexpr int X = 16 / ES;
  constexpr int CH = D / X;
  constexpr int SES = SRC == kF32 ? 4 : 2;       // source element bytes
  constexpr int KR = X * SES / 16;               // 16-byte source pieces per item
  struct Raw {
    u32x4 q[KR];
  };
  const int t = blockIdx.x;
  const int items = a.num_kv_heads * CH;
  // A thread's first item's sources are loaded before the slot is known, so
  // the two loads overlap.
  auto load_raw = [&](const void* base, int e, Raw& r) {
    const int h = e / CH, c = e % CH;
    const int64_t src0 = ((int64_t)t * a.num_kv_heads + h) * D + c * X;
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const char*>(base) + src0 * SES);
#pragma unroll
    for (int i = 0; i < KR; ++i) r.q[i] = p[i];
  };
  Raw k0, v0;
  if ((int)threadIdx.x < items) {
    load_raw(a.k_new, threadIdx.x, k0);
    load_raw(a.v_new, threadIdx.x, v0);
  }
  const int64_t slot = a.slot_mapping[t];
  const int B = a.block_size;
  if (slot < 0 || slot >= a.num_blocks * B) return;
  const int64_t blk = slot / B;
  const int off = (int)(slot % B);
  if (a.block_tables != nullptr && threadIdx.x == 0) {
    const int p = a.context_lens[t] - 1;
    if (p >= 0 && p / B < a.max_blocks) a.block_tables[(int64_t)t * a.max_blocks + p / B] = (int32_t)blk;
  }
  // element x of a source piece as bits (same dtype) or as a float
  auto bits16 = [](const Raw& r, int x) -> uint16_t {
    return reinterpret_cast<const uint16_t*>(&r)[x];
  };
  auto bits32 = [](const Raw& r, int x) -> uint32_t {
    return reinterpret_cast<const uint32_t*>(&r)[x];
  };
  auto val = [&](const Raw& r, int x) -> float {
    if constexpr (SRC == kF32) return __uint_as_float(bits32(r, x));
    else return __uint_as_float((uint32_t)bits16(r, x) << 16);
  };
  constexpr bool kStream = CACHE != kFP8;  // store policy (below)
  auto put = [](auto* p, auto v) {
    if constexpr (kStream)
      __builtin_nontemporal_store(v, p);
    else
      *p = v;
  };
  for (int e = threadIdx.x; e < items; e += blockDim.x) {
    Raw kr = k0, vr = v0;
    if (e != (int)threadIdx.x) {
      load_raw(a.k_new, e, kr);
      load_raw(a.v_new, e, vr);
    }
    const int h = e / CH, c = e % CH;
    const int64_t tile = (blk * a.num_kv_heads + h);
    const int64_t kdst = ((tile * CH + c) * B + off) * X;  // element index
    const int64_t vdst = (tile * D + c * X) * B + off;     // element index, stride B
    // Cache policy of the stores, measured per cache dtype on the decode
    // step (this write, then the attention over the new tokens).  bf16 and
    // fp32 stores stream past the L2 (non-temporal), so the attention meets
    // no dirty lines of theirs (steps 2.4-2.8% faster on the 70B-shaped
    // shared-prefix bf16 batch, within 1% on the others).  Streamed fp8
    // stores (single bytes of V) slowed this kernel more than they saved the
    // attention, so the L2 takes them; a word of every destination line is
    // read first so that it holds those lines whole (0.4-0.5% faster steps
    // on the 70B-shaped fp8 batch than with either plain or streamed stores).
    if constexpr (!kStream) {
      uint32_t old = *reinterpret_cast<const uint32_t*>(static_cast<const char*>(a.k_cache) + kdst * ES);
#pragma unroll
      for (int x = 0; x < X; ++x) old += static_cast<const uint8_t*>(a.v_cache)[(vdst + x * B) * ES];
      asm volatile("" ::"v"(old));
    }
    if constexpr (CACHE == SRC) {
      // same dtype: copy bits
      static_assert(KR == 1, "one 16-byte piece per item");
      if constexpr (ES == 4) {
        uint32_t* kc = static_cast<uint32_t*>(a.k_cache);
        uint32_t* vc = static_cast<uint32_t*>(a.v_cache);
        put(reinterpret_cast<u32x4*>(kc + kdst), kr.q[0]);
#pragma unroll
        for (int x = 0; x < X; ++x) put(vc + vdst + x * B, bits32(vr, x));
      } else {
        uint16_t* kc = static_cast<uint16_t*>(a.k_cache);
        uint16_t* vc = static_cast<uint16_t*>(a.v_cache);
        put(reinterpret_cast<u32x4*>(kc + kdst), kr.q[0]);
#pragma unroll
        for (int x = 0; x < X; ++x) put(vc + vdst + x * B, bits16(vr, x));
      }
    } else if constexpr (CACHE == kBF16) {  // f32 -> bf16
      uint16_t* kc = static_cast<uint16_t*>(a.k_cache);
      uint16_t* vc = static_cast<uint16_t*>(a.v_cache);
      uint16_t kv[X];
#pragma unroll
      for (int x = 0; x < X; ++x) kv[x] = f32_to_bf16_rne(val(kr, x));
      put(reinterpret_cast<u32x4*>(kc + kdst), bitcast<u32x4>(kv));
#pragma unroll
      for (int x = 0; x < X; ++x) put(vc + vdst + x * B, f32_to_bf16_rne(val(vr, x)));
    } else {  // -> fp8 E4M3 of fp32(x / scale)
      uint8_t* kc = static_cast<uint8_t*>(a.k_cache);
      uint8_t* vc = static_cast<uint8_t*>(a.v_cache);
      uint8_t kv[X];
#pragma unroll
      for (int x = 0; x < X; ++x) kv[x] = f32_to_e4m3_sat(val(kr, x) / a.k_scale);
      put(reinterpret_cast<u32x4*>(kc + kdst), bitcast<u32x4>(kv));
#pragma unroll
      for (int x = 0; x < X; ++x) put(vc + vdst + x * B, f32_to_e4m3_sat(val(vr, x) / a.v_scale));
    }
  }
}

// ---------------------------------------------------------------- block copy
// Whole physical blocks, K and V (blockIdx.y), one workgroup per pair:
// 16-byte copies of the block's bytes (a multiple of 1 KiB).
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyBlocksArgs a) {
  const int i = blockIdx.x;
  const int64_t src = a.src[i], dst = a.dst[i];
  if (src < 0 || dst < 0 || src >= a.num_blocks || dst >= a.num_blocks) return;
  char* base = static_cast<char*>(blockIdx.y == 0 ? a.k_cache : a.v_cache);
  const u32x4* from = reinterpret_cast<const u32x4*>(base + src * a.block_bytes);
  u32x4* to = reinterpret_cast<u32x4*>(base + dst * a.block_bytes);
  for (int64_t k = threadIdx.x; k < a.block_bytes / 16; k += blockDim.x) to[k] = from[k];
}

}  // namespace

// ---------------------------------------------------------------- launchers
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream) {
  if (a.n == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(a.n, 2), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_cache_write(const CacheWriteArgs& a, int src, int cache, int D,
                              hipStream_t stream, bool* supported) {
  *supported = true;
  if (a.num_tokens == 0) return hipSuccess;
  dim3 grid(a.num_tokens), block(128);
#define PKV_CW(S_, C_, D_)                                                              \
  if (src == S_ && cache == C_ && D == D_) {                                            \
    hipLaunchKernelGGL((cache_write_kernel<S_, C_, D_>), grid, block, 0, stream, a);    \
    return hipGetLastError();                                                           \
  }
  PKV_CW(kF32, kF32, 64) PKV_CW(kF32, kF32, 128)
  PKV_CW(kBF16, kBF16, 64) PKV_CW(kBF16, kBF16, 128)
  PKV_CW(kF32, kBF16, 64) PKV_CW(kF32, kBF16, 128)
  PKV_CW(kBF16, kFP8, 64) PKV_CW(kBF16, kFP8, 128)
  PKV_CW(kF32, kFP8, 64) PKV_CW(kF32, kFP8, 128)
#undef PKV_CW
  *supported = false;
  return hipSuccess;
}

}  // namespace pkv
