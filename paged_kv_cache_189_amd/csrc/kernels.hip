// Paged decode attention and the KV cache write for CDNA4 (gfx950).
//
// What is computed ("vLLM PagedAttention: Memory Optimization &
// High-Throughput LLM Inference Tuning", §1 and §2): one new query per
// sequence attends to every cached token of its sequence; the kernel reaches
// each token's K and V by walking the sequence's block table over a pool of
// 16-token physical blocks, shared blocks included ("Optimizing Llama 3.1
// 405B Inference with vLLM PagedAttention", PagedAttention Mechanics).  The
// fp8 E4M3 cache of "vLLM PagedAttention Optimization: Complete Step-by-Step
// Tuning Guide for Low-Latency Inference" (Step 3) is dequantized in-kernel.
//
// Design for gfx950:
//  * one workgroup = NW wave64s = one (sequence, kv head, partition); wave w
//    takes blocks w, w+NW, ... of the partition; the block id is read once
//    per wave with a scalar load (wave-uniform indirection);
//  * the pool layout puts 16 bytes of one token's K next to the same 16 bytes
//    of the next token, so lane l's 16-byte load is at l*16 + j*1024 within a
//    (block, head) tile: every load instruction of a wave reads 1 KiB
//    contiguously and lands directly in the A-operand layout of the MFMA;
//  * scores S^T[token][head] = K . Q^T come from v_mfma_f32_16x16x32_bf16
//    (16 tokens x up to 16 query heads of the GQA group), so lane l holds
//    head l%16 and tokens 4*(l/16)..+3: the row max needs two cross-lane
//    steps and P is already in the B-operand layout of O^T = V^T . P^T
//    (v_mfma_f32_16x16x16_bf16), which keeps head l%16 in lane l for the
//    online-softmax rescale;
//  * fp8 E4M3 K/V become bf16 exactly (v_cvt_scalef32_pk_bf16_fp8, scale 1);
//    the per-tensor scales fold into the score scale and the output;
//  * fp32 caches take the v_mfma_f32_16x16x4_f32 path (P stays fp32);
//  * NW partial states are merged through LDS; a sequence that spans one
//    partition writes its final row, longer ones write fp32 partials that a
//    second kernel merges by log-sum-exp.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kF32 = 0, kBF16 = 1, kFP8 = 2;
constexpr int kBS = 16;  // tokens per block
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

template <int SRC>
__device__ __forceinline__ float load_src(const void* p, int64_t i) {
  if constexpr (SRC == kF32) {
    return static_cast<const float*>(p)[i];
  } else {
    return __uint_as_float((uint32_t) static_cast<const uint16_t*>(p)[i] << 16);
  }
}

// ---------------------------------------------------------------- cache write
// One workgroup per new token; threads stride over (kv head, 16-byte chunk).
// K chunk c of head h goes to tile[c][slot % 16][0..X); V element d goes to
// tile[d][slot % 16].
template <int SRC, int CACHE, int D>
__global__ __launch_bounds__(128) void cache_write_kernel(CacheWriteArgs a) {
  constexpr int ES = ElemSize<CACHE>::value;
  constexpr int X = 16 / ES;
  constexpr int CH = D / X;
  const int t = blockIdx.x;
  const int64_t slot = a.slot_mapping[t];
  if (slot < 0 || slot >= a.num_blocks * kBS) return;
  const int64_t blk = slot / kBS;
  const int off = (int)(slot % kBS);
  for (int e = threadIdx.x; e < a.num_kv_heads * CH; e += blockDim.x) {
    const int h = e / CH, c = e % CH;
    const int64_t src0 = ((int64_t)t * a.num_kv_heads + h) * D + c * X;
    const int64_t tile = (blk * a.num_kv_heads + h);
    const int64_t kdst = ((tile * CH + c) * kBS + off) * X;  // element index
    const int64_t vdst = (tile * D + c * X) * kBS + off;     // element index, stride kBS
    if constexpr (CACHE == SRC) {
      // same dtype: copy bits
      if constexpr (ES == 4) {
        const uint32_t* ks = static_cast<const uint32_t*>(a.k_new) + src0;
        const uint32_t* vs = static_cast<const uint32_t*>(a.v_new) + src0;
        uint32_t* kc = static_cast<uint32_t*>(a.k_cache);
        uint32_t* vc = static_cast<uint32_t*>(a.v_cache);
        *reinterpret_cast<u32x4*>(kc + kdst) = *reinterpret_cast<const u32x4*>(ks);
#pragma unroll
        for (int x = 0; x < X; ++x) vc[vdst + x * kBS] = vs[x];
      } else {
        const uint16_t* ks = static_cast<const uint16_t*>(a.k_new) + src0;
        const uint16_t* vs = static_cast<const uint16_t*>(a.v_new) + src0;
        uint16_t* kc = static_cast<uint16_t*>(a.k_cache);
        uint16_t* vc = static_cast<uint16_t*>(a.v_cache);
        *reinterpret_cast<u32x4*>(kc + kdst) = *reinterpret_cast<const u32x4*>(ks);
#pragma unroll
        for (int x = 0; x < X; ++x) vc[vdst + x * kBS] = vs[x];
      }
    } else if constexpr (CACHE == kBF16) {  // f32 -> bf16
      uint16_t* kc = static_cast<uint16_t*>(a.k_cache);
      uint16_t* vc = static_cast<uint16_t*>(a.v_cache);
      uint16_t kv[X];
#pragma unroll
      for (int x = 0; x < X; ++x) kv[x] = f32_to_bf16_rne(load_src<SRC>(a.k_new, src0 + x));
      *reinterpret_cast<u32x4*>(kc + kdst) = bitcast<u32x4>(kv);
#pragma unroll
      for (int x = 0; x < X; ++x) vc[vdst + x * kBS] = f32_to_bf16_rne(load_src<SRC>(a.v_new, src0 + x));
    } else {  // -> fp8 E4M3 of fp32(x / scale)
      uint8_t* kc = static_cast<uint8_t*>(a.k_cache);
      uint8_t* vc = static_cast<uint8_t*>(a.v_cache);
      uint8_t kv[X];
#pragma unroll
      for (int x = 0; x < X; ++x) kv[x] = f32_to_e4m3_sat(load_src<SRC>(a.k_new, src0 + x) / a.k_scale);
      *reinterpret_cast<u32x4*>(kc + kdst) = bitcast<u32x4>(kv);
#pragma unroll
      for (int x = 0; x < X; ++x)
        vc[vdst + x * kBS] = f32_to_e4m3_sat(load_src<SRC>(a.v_new, src0 + x) / a.v_scale);
    }
  }
}

// ---------------------------------------------------------------- pass 1
template <int KIND, int D>
struct Frags {
  using T = Tile<KIND, D>;
  u32x4 k[T::NK];
  typename T::V v[T::NT];
};

// O^T accumulators: o[nt][i] = O^T[d = nt*16 + 4*(lane/16) + i][head lane%16].
template <int KIND, int D>
struct Acc {
  f32x4 o[Tile<KIND, D>::NT];
};

// K/V tiles are streamed once per step: non-temporal loads (the nt bit)
// keep them from displacing reusable lines in L2 and measured ~12% more
// read bandwidth on MI355X for randomly placed 4-8 KiB tiles.
template <int KIND, int D>
__device__ __forceinline__ void load_tile(Frags<KIND, D>& f, const char* kt, const char* vt,
                                          int lane, int r, int q4) {
  using T = Tile<KIND, D>;
  using V = typename T::V;
#pragma unroll
  for (int j = 0; j < T::NK; ++j)
    f.k[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kt + (j * 64 + lane) * 16));
#pragma unroll
  for (int nt = 0; nt < T::NT; ++nt)
    f.v[nt] = __builtin_nontemporal_load(
        reinterpret_cast<const V*>(vt + ((nt * 16 + r) * kBS + 4 * q4) * T::ES));
}

// S^T[token 4*q4+i][head r] for i = 0..3.
template <int KIND, int D>
__device__ __forceinline__ f32x4 scores(const Frags<KIND, D>& f, const u32x4 (&qf)[Tile<KIND, D>::NQ]) {
  using T = Tile<KIND, D>;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (KIND == kBF16) {
#pragma unroll
    for (int j = 0; j < T::NK; ++j)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(f.k[j]), bitcast<bf16x8>(qf[j]), acc, 0, 0, 0);
  } else if constexpr (KIND == kFP8) {
#pragma unroll
    for (int j = 0; j < T::NK; ++j) {
      u32x4 lo, hi;
      fp8x16_to_bf16(f.k[j], lo, hi);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(lo), bitcast<bf16x8>(qf[2 * j]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(hi), bitcast<bf16x8>(qf[2 * j + 1]), acc, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int j = 0; j < T::NK; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(f.k[j][e]), __uint_as_float(qf[j][e]), acc, 0, 0, 0);
  }
  return acc;
}

// The lane's four weights P as multiplied into V: bf16 (round to nearest
// even) except on the fp32 path.
template <int KIND>
struct Weights {
  float p[4];   // exact fp32 weights
  s16x4 pb;     // bf16 weights (unused on the fp32 path)
  float used;   // sum of the weights as multiplied (normalises the output)
  float exact;  // sum of the fp32 weights (feeds the log-sum-exp)
};

template <int KIND>
__device__ __forceinline__ Weights<KIND> make_weights(const float (&p)[4]) {
  Weights<KIND> w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w.p[i] = p[i];
  w.exact = (p[0] + p[1]) + (p[2] + p[3]);
  if constexpr (KIND == kF32) {
    w.pb = s16x4{0, 0, 0, 0};
    w.used = w.exact;
  } else {
    bf16x2 p01 = __builtin_convertvector(f32x2{p[0], p[1]}, bf16x2);
    bf16x2 p23 = __builtin_convertvector(f32x2{p[2], p[3]}, bf16x2);
    u32x2 pp = {bitcast<uint32_t>(p01), bitcast<uint32_t>(p23)};
    w.pb = bitcast<s16x4>(pp);
    w.used = ((float)p01[0] + (float)p01[1]) + ((float)p23[0] + (float)p23[1]);
  }
  return w;
}

// O^T[d][head r] += V^T . P^T over the block's 16 tokens.  `valid` masks the
// lane's 4 tokens (slots past the sequence end may hold anything, NaN too, so
// they are selected away, not multiplied by a zero weight).
template <int KIND, int D, bool MASK>
__device__ __forceinline__ void accumulate_pv(Acc<KIND, D>& acc, const Frags<KIND, D>& f,
                                              const Weights<KIND>& wt, const bool (&valid)[4]) {
  using T = Tile<KIND, D>;
  f32x4* o = acc.o;
  if constexpr (KIND == kF32) {
#pragma unroll
    for (int nt = 0; nt < T::NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = __uint_as_float(f.v[nt][i]);
        if (MASK) v = valid[i] ? v : 0.f;
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(v, wt.p[i], o[nt], 0, 0, 0);
      }
  } else {
#pragma unroll
    for (int nt = 0; nt < T::NT; ++nt) {
      s16x4 v;
      if constexpr (KIND == kBF16)
        v = bitcast<s16x4>(f.v[nt]);
      else
        v = fp8x4_to_bf16x4(f.v[nt]);
      if (MASK) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = valid[i] ? v[i] : (short)0;
      }
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v, wt.pb, o[nt], 0, 0, 0);
    }
  }
}

// Lanes l, l^16, l^32 and l^48 hold the same query head: reduce over them
// with the gfx950 row-swap permutes (no LDS round trip).
__device__ __forceinline__ float max_across_groups(float v) {
  uint32_t u = __float_as_uint(v);
  auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
  u = __float_as_uint(v);
  auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
}

__device__ __forceinline__ float sum_across_groups(float v) {
  uint32_t u = __float_as_uint(v);
  auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
  u = __float_as_uint(v);
  auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
}

// The running max moves only when a block's max exceeds it by more than this
// (log2 units).  Weights are then bounded by 2^kLazyMax; numerator and
// normaliser share the same stale max, so the result is unchanged while the
// O^T rescale (32 accumulators) is skipped for almost every block.
constexpr float kLazyMax = 8.0f;

// One wave's online-softmax state for its 16 head rows.
template <int KIND, int D>
struct RunState {
  float m, l, e;  // running max (log2 units), sum of used weights, sum of fp32 weights
  Acc<KIND, D> acc;
  __device__ __forceinline__ void init() {
    m = -INFINITY;
    l = 0.f;
    e = 0.f;
#pragma unroll
    for (int nt = 0; nt < Tile<KIND, D>::NT; ++nt) acc.o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
};

// Scores, online softmax and P.V for logical block b of the sequence.
template <int KIND, int D>
__device__ __forceinline__ void process_block(RunState<KIND, D>& st, const Frags<KIND, D>& f,
                                              const u32x4 (&qf)[Tile<KIND, D>::NQ], int b, int L,
                                              float score_scale_log2, int q4) {
  using T = Tile<KIND, D>;
  const f32x4 sc = scores<KIND, D>(f, qf);
  const int tok0 = b * kBS + 4 * q4;
  float x[4];
  bool valid[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    valid[i] = tok0 + i < L;
    x[i] = valid[i] ? sc[i] * score_scale_log2 : -INFINITY;
  }
  const float mx = max_across_groups(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
  const bool bump = mx > st.m + kLazyMax;  // always true on the first block
  if (__builtin_amdgcn_ballot_w64(bump)) {
    const float m_new = bump ? mx : st.m;   // mx >= st.m whenever bump
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
    st.m = m_new;
    st.l *= alpha;
    st.e *= alpha;
#pragma unroll
    for (int nt = 0; nt < T::NT; ++nt) st.acc.o[nt] *= alpha;
  }
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - st.m);
  const Weights<KIND> wt = make_weights<KIND>(p);
  st.l += wt.used;
  st.e += wt.exact;
  if ((b + 1) * kBS > L)
    accumulate_pv<KIND, D, true>(st.acc, f, wt, valid);
  else
    accumulate_pv<KIND, D, false>(st.acc, f, wt, valid);
}

template <int KIND, int D, int NW>
__global__ __launch_bounds__(NW * 64) void decode_partitions_kernel(DecodeArgs a) {
  using T = Tile<KIND, D>;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, q4 = lane >> 4;
  const int g = blockIdx.x % a.num_kv_heads;
  const int s = blockIdx.x / a.num_kv_heads;
  const int part = blockIdx.y;

  int L = a.context_lens[s];
  L = L < 0 ? 0 : (L > a.max_context_len ? a.max_context_len : L);
  const int nblk = (L + kBS - 1) / kBS;
  const int nparts = (nblk + a.part_blocks - 1) / a.part_blocks;
  if (part >= (nparts > 0 ? nparts : 1)) return;

  const int G = a.group;
  const int Hq = a.num_q_heads;

  // Q^T fragments of the lane's head (zero rows pad the group to 16).
  u32x4 qf[T::NQ];
  {
    const int head = g * G + r;
    constexpr int QES = KIND == kF32 ? 4 : 2;
    const char* qrow = static_cast<const char*>(a.q) + ((int64_t)s * Hq + head) * D * QES;
#pragma unroll
    for (int j = 0; j < T::NQ; ++j) {
      int off;
      if constexpr (KIND == kFP8)
        off = ((j >> 1) * 4 + q4) * 32 + (j & 1) * 16;
      else
        off = (j * 4 + q4) * 16;
      qf[j] = r < G ? *reinterpret_cast<const u32x4*>(qrow + off) : u32x4{0u, 0u, 0u, 0u};
    }
  }

  const int b_begin = part * a.part_blocks;
  const int b_end = min(b_begin + a.part_blocks, nblk);
  const int32_t* tbl = a.block_tables + (int64_t)s * a.max_blocks;
  const char* kbase = static_cast<const char*>(a.k_cache) + (int64_t)g * T::BYTES;
  const char* vbase = static_cast<const char*>(a.v_cache) + (int64_t)g * T::BYTES;
  const int64_t bstride = (int64_t)a.num_kv_heads * T::BYTES;
  const int64_t last_block = a.num_blocks - 1;

  auto tile_of = [&](int b, const char*& kt, const char*& vt) {
    int64_t phys = __builtin_amdgcn_readfirstlane(tbl[b]);
    phys = phys < 0 ? 0 : (phys > last_block ? last_block : phys);
    kt = kbase + phys * bstride;
    vt = vbase + phys * bstride;
  };

  // Ping-pong register buffers: block b+NW is loaded while block b is
  // processed.  The prefetch index is clamped (the last block is re-read from
  // cache) so every iteration issues the same loads and the waits stay partial.
  RunState<KIND, D> st;
  st.init();
  int b = b_begin + w;
  if (b < b_end) {
    Frags<KIND, D> fa, fb;
    const char *kt, *vt;
    tile_of(b, kt, vt);
    load_tile<KIND, D>(fa, kt, vt, lane, r, q4);
    for (;;) {
      tile_of(min(b + NW, b_end - 1), kt, vt);
      load_tile<KIND, D>(fb, kt, vt, lane, r, q4);
      process_block<KIND, D>(st, fa, qf, b, L, a.score_scale_log2, q4);
      b += NW;
      if (b >= b_end) break;
      tile_of(min(b + NW, b_end - 1), kt, vt);
      load_tile<KIND, D>(fa, kt, vt, lane, r, q4);
      process_block<KIND, D>(st, fb, qf, b, L, a.score_scale_log2, q4);
      b += NW;
      if (b >= b_end) break;
    }
  }
  const float m_run = st.m;
  const float l_run = sum_across_groups(st.l);
  const float e_run = sum_across_groups(st.e);
  const f32x4* o = st.acc.o;

  // ---- merge the NW wave states through LDS
  __shared__ float sm_o[NW][D][17];
  __shared__ float sm_m[NW][16];
  __shared__ float sm_l[NW][16];
  __shared__ float sm_e[NW][16];
  if (q4 == 0) {
    sm_m[w][r] = m_run;
    sm_l[w][r] = l_run;
    sm_e[w][r] = e_run;
  }
#pragma unroll
  for (int nt = 0; nt < T::NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm_o[w][nt * 16 + 4 * q4 + i][r] = o[nt][i];
  __syncthreads();

  const bool final_row = nparts <= 1;
  for (int e = threadIdx.x; e < G * D; e += NW * 64) {
    const int h = e / D, d = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < NW; ++k) M = fmaxf(M, sm_m[k][h]);
    float num = 0.f, den = 0.f, ex = 0.f;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      const float mk = sm_m[k][h];
      const float c = mk == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mk - M);
      num += c * sm_o[k][d][h];
      den += c * sm_l[k][h];
      ex += c * sm_e[k][h];
    }
    const int64_t row = (int64_t)s * Hq + g * G + h;
    if (final_row) {
      const float val = den > 0.f ? num / den * a.v_scale : 0.f;
      if constexpr (KIND == kF32)
        static_cast<float*>(a.out)[row * D + d] = val;
      else
        static_cast<uint16_t*>(a.out)[row * D + d] = f32_to_bf16_rne(val);
      if (d == 0 && a.lse)
        a.lse[row] = ex > 0.f ? (M + __builtin_amdgcn_logf(ex)) * kLn2 : -INFINITY;
    } else {
      const int64_t pr = row * a.max_parts + part;
      a.ws_o[pr * D + d] = num * a.v_scale;
      if (d == 0) {
        a.ws_m[pr] = M;
        a.ws_l[pr] = den;
        a.ws_e[pr] = ex;
      }
    }
  }
}

// ---------------------------------------------------------------- pass 2
// One workgroup per (sequence, query head) whose sequence spans more than one
// partition: M = max m_p, Lambda = sum l_p 2^{m_p - M},
// out = sum 2^{m_p - M} o_p / Lambda, lse = (M + log2 sum e_p 2^{m_p - M}) ln 2,
// where l_p sums the weights as multiplied into V and e_p the fp32 weights.
template <int OUT, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecodeArgs a) {
  extern __shared__ float sm_c[];  // max_parts weights
  __shared__ float sm_red[D / 64];
  __shared__ float sm_ex[D / 64];
  const int row = blockIdx.x;  // s * Hq + h
  const int s = row / a.num_q_heads;
  const int tid = threadIdx.x;
  int L = a.context_lens[s];
  L = L < 0 ? 0 : (L > a.max_context_len ? a.max_context_len : L);
  const int nblk = (L + kBS - 1) / kBS;
  int np = (nblk + a.part_blocks - 1) / a.part_blocks;
  if (np <= 1) return;
  np = np < a.max_parts ? np : a.max_parts;
  const float* mrow = a.ws_m + (int64_t)row * a.max_parts;
  const float* lrow = a.ws_l + (int64_t)row * a.max_parts;
  const float* erow = a.ws_e + (int64_t)row * a.max_parts;

  float mx = -INFINITY;
  for (int p = tid; p < np; p += D) mx = fmaxf(mx, mrow[p]);
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) mx = fmaxf(mx, __shfl_xor(mx, k));
  if ((tid & 63) == 0) sm_red[tid >> 6] = mx;
  __syncthreads();
  float M = sm_red[0];
#pragma unroll
  for (int k = 1; k < D / 64; ++k) M = fmaxf(M, sm_red[k]);
  __syncthreads();

  float lam = 0.f, ex = 0.f;
  for (int p = tid; p < np; p += D) {
    const float m = mrow[p];
    const float c = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M);
    sm_c[p] = c;
    lam += c * lrow[p];
    ex += c * erow[p];
  }
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) {
    lam += __shfl_xor(lam, k);
    ex += __shfl_xor(ex, k);
  }
  if ((tid & 63) == 0) {
    sm_red[tid >> 6] = lam;
    sm_ex[tid >> 6] = ex;
  }
  __syncthreads();
  float Lam = 0.f, Ex = 0.f;
#pragma unroll
  for (int k = 0; k < D / 64; ++k) {
    Lam += sm_red[k];
    Ex += sm_ex[k];
  }

  const float* orow = a.ws_o + (int64_t)row * a.max_parts * D + tid;
  float acc0 = 0.f, acc1 = 0.f;
  int p = 0;
  for (; p + 1 < np; p += 2) {
    acc0 += sm_c[p] * orow[(int64_t)p * D];
    acc1 += sm_c[p + 1] * orow[(int64_t)(p + 1) * D];
  }
  if (p < np) acc0 += sm_c[p] * orow[(int64_t)p * D];
  const float val = Lam > 0.f ? (acc0 + acc1) / Lam : 0.f;
  if constexpr (OUT == kF32)
    static_cast<float*>(a.out)[(int64_t)row * D + tid] = val;
  else
    static_cast<uint16_t*>(a.out)[(int64_t)row * D + tid] = f32_to_bf16_rne(val);
  if (tid == 0 && a.lse) a.lse[row] = Ex > 0.f ? (M + __builtin_amdgcn_logf(Ex)) * kLn2 : -INFINITY;
}

}  // namespace

// ---------------------------------------------------------------- launchers
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

hipError_t launch_decode_partitions(const DecodeArgs& a, int cache, int D, hipStream_t stream,
                                    bool* supported) {
  *supported = true;
  if (a.num_seqs == 0) return hipSuccess;
  dim3 grid(a.num_seqs * a.num_kv_heads, a.max_parts), block(kWavesPerGroup * 64);
#define PKV_P1(C_, D_)                                                                          \
  if (cache == C_ && D == D_) {                                                                 \
    hipLaunchKernelGGL((decode_partitions_kernel<C_, D_, kWavesPerGroup>), grid, block, 0, stream, a); \
    return hipGetLastError();                                                                   \
  }
  PKV_P1(kF32, 64) PKV_P1(kF32, 128) PKV_P1(kBF16, 64) PKV_P1(kBF16, 128) PKV_P1(kFP8, 64)
  PKV_P1(kFP8, 128)
#undef PKV_P1
  *supported = false;
  return hipSuccess;
}

hipError_t launch_decode_merge(const DecodeArgs& a, int out, int D, hipStream_t stream,
                               bool* supported) {
  *supported = true;
  if (a.num_seqs == 0 || a.max_parts <= 1) return hipSuccess;
  dim3 grid(a.num_seqs * a.num_q_heads), block(D);
  const size_t lds = (size_t)a.max_parts * sizeof(float);
#define PKV_P2(O_, D_)                                                                      \
  if (out == O_ && D == D_) {                                                               \
    hipLaunchKernelGGL((decode_merge_kernel<O_, D_>), grid, block, lds, stream, a);         \
    return hipGetLastError();                                                               \
  }
  PKV_P2(kF32, 64) PKV_P2(kF32, 128) PKV_P2(kBF16, 64) PKV_P2(kBF16, 128)
#undef PKV_P2
  *supported = false;
  return hipSuccess;
}

}  // namespace pkv
