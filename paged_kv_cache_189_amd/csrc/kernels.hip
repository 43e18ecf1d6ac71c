// Paged decode attention, pass 1 and its plan, for CDNA4 (gfx950).
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
//  * pass 1 is persistent: every resident wave owns one of R equal ranges of
//    the line of all (kv head, sequence) pairs' tiles (decode_plan.h), dealt
//    so that each XCD works through one contiguous eighth of the line; the
//    block id of each tile is read with a scalar load (wave-uniform);
//  * the pool layout puts 16 bytes of one token's K next to the same 16 bytes
//    of the next token, so lane l's 16-byte load is at l*16 + j*1024 within a
//    (block, head) tile: every load instruction of a wave reads 1 KiB
//    contiguously and lands directly in the A-operand layout of the MFMA;
//  * scores S^T[token][head] = K . Q^T come from v_mfma_f32_16x16x32_bf16
//    (16 tokens x up to 16 query heads of the GQA group), so lane l holds
//    head l%16 and tokens 4*(l/16)..+3: the row max needs two cross-lane
//    steps and P is already in the B-operand layout of O^T = V^T . P^T,
//    which keeps head l%16 in lane l for the online-softmax rescale;
//  * fp8 E4M3 K/V become bf16 exactly (v_cvt_scalef32_pk_bf16_fp8, scale 1),
//    two 16-token blocks per stage; the per-tensor scales fold into the
//    score scale and the output; fp32 caches take v_mfma_f32_16x16x4_f32;
//  * a pair's pieces in the four ranges of one workgroup are merged in LDS;
//    a pair inside one workgroup writes its final row, the others leave
//    partial states that pass 2 (decode_merge.hip) merges by log-sum-exp.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <type_traits>

#include "decode_plan.h"
#include "device_common.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

// ---------------------------------------------------------------- pass 1
template <int KIND, int D>
struct Frags {
  using T = Tile<KIND, D>;
  u32x4 k[T::NK];
  typename T::V v[T::NT];
};

// Most K/V tiles are read once per step: non-temporal loads (the nt bit)
// keep them from displacing reusable lines in L2 and measured ~12% more
// read bandwidth on MI355X for randomly placed 4-8 KiB tiles.  The leading
// tiles of each sequence are the exception (HotTiles below).
// Lane offsets into one 16-token tile of a block of B = 16 << shift tokens:
// K is [D/X][B][X] per (block, head), so lane l reads 16 bytes of token l % 16
// in d-chunk 4j + l / 16; V is [D][B], lane (r, q4) reads tokens 4 q4 .. +3 of
// dimension 16 nt + r.  Strides between the lane's loads: kj (K), vn (V).
struct TileOffsets {
  uint32_t koff, voff, kj, vn;
};
template <int KIND, int D>
__device__ __forceinline__ TileOffsets tile_offsets(int lane, int r, int q4, int shift) {
  using T = Tile<KIND, D>;
  const uint32_t B = 16u << shift;
  TileOffsets o;
  o.koff = (((uint32_t)lane >> 4) * B + ((uint32_t)lane & 15u)) * 16u;
  o.voff = ((uint32_t)r * B + 4u * (uint32_t)q4) * T::ES;
  o.kj = 64u * B;
  o.vn = 16u * B * T::ES;
  return o;
}

// With 32-token blocks a tile reads half of each V row (and of each 128-byte
// K line pair); the other half is the next tile's, read one stage later, so
// those loads keep the default cache policy and find it in L2.
template <int KIND, int D, bool STREAM>
__device__ __forceinline__ void load_tile(Frags<KIND, D>& f, gchar_p kt, gchar_p vt,
                                          const TileOffsets& o) {
  using T = Tile<KIND, D>;
  using V = typename T::V;
#pragma unroll
  for (int j = 0; j < T::NK; ++j) {
    gptr<u32x4> p = reinterpret_cast<gptr<u32x4>>(kt + j * o.kj + o.koff);
    f.k[j] = STREAM ? __builtin_nontemporal_load(p) : *p;
  }
#pragma unroll
  for (int nt = 0; nt < T::NT; ++nt) {
    gptr<V> p = reinterpret_cast<gptr<V>>(vt + nt * o.vn + o.voff);
    f.v[nt] = STREAM ? __builtin_nontemporal_load(p) : *p;
  }
}

// Q^T fragments of one segment's query group, staged once per segment in the
// wave's own LDS slot: qf[j][lane] is the 16 bytes lane `lane` feeds to MFMA
// step j.
template <int KIND, int D>
struct QLds {
  u32x4 qf[Tile<KIND, D>::NQ][64];
#if PKV_DECODE_VALU_SCORES
  float sx[16][16];  // scores S[head][token] of the tile, vector-unit variant
#endif
};

// S^T[token 4*q4+i][head r] for i = 0..3.
template <int KIND, int D>
__device__ __forceinline__ f32x4 scores(const Frags<KIND, D>& f, const QLds<KIND, D>& q, int lane) {
  using T = Tile<KIND, D>;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (KIND == kBF16) {
#pragma unroll
    for (int j = 0; j < T::NK; ++j)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(f.k[j]), bitcast<bf16x8>(q.qf[j][lane]), acc, 0, 0, 0);
  } else if constexpr (KIND == kFP8) {
#pragma unroll
    for (int j = 0; j < T::NK; ++j) {
      u32x4 lo, hi;
      fp8x16_to_bf16(f.k[j], lo, hi);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(lo), bitcast<bf16x8>(q.qf[2 * j][lane]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(hi), bitcast<bf16x8>(q.qf[2 * j + 1][lane]), acc, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int j = 0; j < T::NK; ++j) {
      const u32x4 qj = q.qf[j][lane];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(f.k[j][e]), __uint_as_float(qj[e]), acc, 0, 0, 0);
    }
  }
  return acc;
}

// The q.K contraction on the vector unit instead of the matrix cores, for
// the comparison that decides which unit runs it (built with
// -DPKV_DECODE_VALU_SCORES=1; the 16-token tile path of bf16 and fp8 caches;
// 32-token blocks and fp8 block pairs keep MFMA).  Lane (t, c) holds token
// t's K dims in the chunks of MFMA step j (the same dims lane (h, c) holds of
// head h's Q); it dots them with every head's Q chunk read from the wave's
// LDS slot (v_dot2_f32_bf16, fp32 accumulation), the four lanes of a token
// add their parts, and the scores go through LDS to the layout scores()
// returns: S^T[token 4 q4 + i][head r], zero for the padding rows r >= G.
// The result differs from the MFMA one only in fp32 summation order.
#ifndef PKV_DECODE_VALU_SCORES
#define PKV_DECODE_VALU_SCORES 0
#endif
#if PKV_DECODE_VALU_SCORES
__device__ __forceinline__ float sum_across_groups(float v);
template <int KIND, int D>
__device__ __forceinline__ f32x4 scores_valu(const Frags<KIND, D>& f, QLds<KIND, D>& q, int lane, int G) {
  using T = Tile<KIND, D>;
  static_assert(KIND != kF32, "fp32 keeps the MFMA contraction");
  const int t = lane & 15, c = lane >> 4;
  u32x4 kb[T::NQ];  // token t's K as bf16 pairs, chunk jq as Q fragment jq
  if constexpr (KIND == kBF16) {
#pragma unroll
    for (int j = 0; j < T::NK; ++j) kb[j] = f.k[j];
  } else {
#pragma unroll
    for (int j = 0; j < T::NK; ++j) fp8x16_to_bf16(f.k[j], kb[2 * j], kb[2 * j + 1]);
  }
#pragma unroll
  for (int h = 0; h < 16; ++h) {
    if (h >= G) break;  // wave-uniform
    float acc = 0.f;
#pragma unroll
    for (int jq = 0; jq < T::NQ; ++jq) {
      const u32x4 qv = q.qf[jq][h + 16 * c];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2>(kb[jq][e]), bitcast<bf16x2>(qv[e]), acc, false);
    }
    acc = sum_across_groups(acc);  // the four dim quarters of token t
    if ((h & 3) == c) q.sx[h][t] = acc;
  }
  // A wave's LDS accesses complete in order: the row is the one just written.
  const int r = lane & 15, q4 = lane >> 4;
  const f32x4 v = *reinterpret_cast<const f32x4*>(&q.sx[r][4 * q4]);
  return r < G ? v : f32x4{0.f, 0.f, 0.f, 0.f};
}
#endif

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

// Scores, online softmax and P.V for tile b (16 tokens) of the sequence.  L:
// tokens the lane's query row may see; Lv: tokens of the sequence (wave-
// uniform; decode passes the same length for both).  Scores past L get
// weight 0; V rows past Lv may hold anything (NaN too) and are selected away.
// In the P.V product a lane holds V of dimension r, not query row r, so V
// masking uses the sequence bound only.
template <int KIND, int D>
__device__ __forceinline__ void process_block(RunState<KIND, D>& st, const Frags<KIND, D>& f,
                                              QLds<KIND, D>& q, int b, int L, int Lv,
                                              float score_scale_log2, int lane, int q4, int G) {
  using T = Tile<KIND, D>;
#if PKV_DECODE_VALU_SCORES
  f32x4 sc;
  if constexpr (KIND == kF32)
    sc = scores<KIND, D>(f, q, lane);
  else
    sc = scores_valu<KIND, D>(f, q, lane, G);
#else
  (void)G;
  const f32x4 sc = scores<KIND, D>(f, q, lane);
#endif
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
  if ((b + 1) * kBS > Lv) {
    bool vvalid[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) vvalid[i] = tok0 + i < Lv;
    accumulate_pv<KIND, D, true>(st.acc, f, wt, vvalid);
  } else {
    accumulate_pv<KIND, D, false>(st.acc, f, wt, valid);
  }
}

// ---- 32-token blocks: one stage per block
// A 16-token tile reads half of every 64-byte V row of a 32-token block, so
// the block is taken whole.  Its K fragments are loaded as two 16-row halves
// whose MFMA row m is token 8 (m / 4) + 4 h + m % 4 (half h): lane (r, q4)
// then holds the scores of tokens 8 q4 .. 8 q4 + 7, the eight consecutive
// tokens whose V it reads per dimension in one load, and P.V runs as
// 16x16x32 MFMAs over whole V rows.
template <int KIND, int D>
struct Frags32 {
  using T = Tile<KIND, D>;
  static constexpr int VB8 = 8 * T::ES;               // V bytes of 8 tokens of one dim
  static constexpr int VN = VB8 > 16 ? VB8 / 16 : 1;  // 16-byte pieces of them (fp32: 2)
  using VP = typename VecOf<(VB8 > 16 ? 16 : VB8)>::T;
  u32x4 k[2][T::NK];
  VP v[T::NT][VN];
};

struct Offsets32 {
  uint32_t koff[2], voff;
};
template <int KIND, int D>
__device__ __forceinline__ Offsets32 offsets32(int lane, int r, int q4) {
  Offsets32 o;
  const uint32_t m = (uint32_t)lane & 15u, cq = (uint32_t)lane >> 4;
#pragma unroll
  for (int h = 0; h < 2; ++h) o.koff[h] = cq * 512u + (8u * (m >> 2) + 4u * h + (m & 3u)) * 16u;
  o.voff = ((uint32_t)r * 32u + 8u * (uint32_t)q4) * Tile<KIND, D>::ES;
  return o;
}

// Two consecutive 16-token blocks A (tokens 0-15) and B (16-31) taken as one
// 32-token stage: the same MFMA row order, so K lane-row m < 8 and V lanes
// with q4 < 2 read A, the others B, each at its offset in a 16-token block
// (K chunk stride 256 bytes, V row 16 * ES bytes).
template <int KIND, int D>
__device__ __forceinline__ Offsets32 offsets_pair(int lane, int r, int q4) {
  Offsets32 o;
  const uint32_t m = (uint32_t)lane & 15u, cq = (uint32_t)lane >> 4;
#pragma unroll
  for (int h = 0; h < 2; ++h) o.koff[h] = cq * 256u + ((8u * (m >> 2) + 4u * h + (m & 3u)) & 15u) * 16u;
  o.voff = ((uint32_t)r * 16u + 8u * ((uint32_t)q4 & 1u)) * Tile<KIND, D>::ES;
  return o;
}

// A block's K chunk j of lane-row cq sits at (4 j + cq) * 512 bytes; V row d
// at d * 32 * ES bytes.  Every line of the block is read in this stage.
// (PAIR: a 16-token block pair, K chunk j at (4 j + cq) * 256 bytes and V
// row d at d * 16 * ES bytes of the lane's block.)
// Cache policy measured per dtype: fp8 blocks stream (non-temporal, +10% on
// the 70B-shaped fp8 workload); bf16 blocks keep the default policy, which
// lets the blocks of a shared prefix stay in L2 for the other sequences
// (+12% on the shared-prefix workload, within 1% elsewhere).
template <int KIND, int D, bool STREAM, bool PAIR = false>
__device__ __forceinline__ void load_block32(Frags32<KIND, D>& f, gchar_p kt, gchar_p vt,
                                             const Offsets32& o) {
  using T = Tile<KIND, D>;
  using F = Frags32<KIND, D>;
  constexpr int KJ = PAIR ? 1024 : 2048;                // K bytes per chunk group j
  constexpr int VNT = (PAIR ? 256 : 512) * T::ES;       // V bytes per 16 dims
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < T::NK; ++j)
    {
      gptr<u32x4> pk = reinterpret_cast<gptr<u32x4>>(kt + j * KJ + o.koff[h]);
      f.k[h][j] = STREAM ? __builtin_nontemporal_load(pk) : *pk;
    }
#pragma unroll
  for (int nt = 0; nt < T::NT; ++nt)
#pragma unroll
    for (int pc = 0; pc < F::VN; ++pc)
    {
      gptr<typename F::VP> pv = reinterpret_cast<gptr<typename F::VP>>(vt + nt * VNT + o.voff + pc * 16);
      f.v[nt][pc] = STREAM ? __builtin_nontemporal_load(pv) : *pv;
    }
}

// S^T of one 32-token block: sc[h][i] = score of token 8 q4 + 4 h + i.
template <int KIND, int D>
__device__ __forceinline__ void scores32(const Frags32<KIND, D>& f, const QLds<KIND, D>& q,
                                         int lane, f32x4 (&sc)[2]) {
  using T = Tile<KIND, D>;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (KIND == kBF16) {
#pragma unroll
      for (int j = 0; j < T::NK; ++j)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(f.k[h][j]), bitcast<bf16x8>(q.qf[j][lane]), acc, 0, 0, 0);
    } else if constexpr (KIND == kFP8) {
#pragma unroll
      for (int j = 0; j < T::NK; ++j) {
        u32x4 lo, hi;
        fp8x16_to_bf16(f.k[h][j], lo, hi);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(lo), bitcast<bf16x8>(q.qf[2 * j][lane]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(hi), bitcast<bf16x8>(q.qf[2 * j + 1][lane]), acc, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < T::NK; ++j) {
        const u32x4 qj = q.qf[j][lane];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(f.k[h][j][e]), __uint_as_float(qj[e]), acc, 0, 0, 0);
      }
    }
    sc[h] = acc;
  }
}

// Online softmax and P.V for one 32-token block starting at token tok0,
// from its scores.  MASK: tokens outside [tmin, tmax) get weight 0 and V of
// tokens at or past L (slots past the sequence may hold NaN) is selected
// away.
template <int KIND, int D, bool MASK>
__device__ __forceinline__ void finish_block32(RunState<KIND, D>& st, const Frags32<KIND, D>& f,
                                               const f32x4 (&sc)[2], int tok0, int tmin, int tmax,
                                               int L, float score_scale_log2, int q4) {
  using T = Tile<KIND, D>;
  const int t8 = tok0 + 8 * q4;  // the lane's tokens: t8 .. t8 + 7
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[i] = sc[i >> 2][i & 3] * score_scale_log2;
    if (MASK) x[i] = t8 + i >= tmin && t8 + i < tmax ? x[i] : -INFINITY;
  }
  const float mx = max_across_groups(fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                                           fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7]))));
  const bool bump = mx > st.m + kLazyMax;  // always true on the first block
  if (__builtin_amdgcn_ballot_w64(bump)) {
    const float m_new = bump ? mx : st.m;
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
    st.m = m_new;
    st.l *= alpha;
    st.e *= alpha;
#pragma unroll
    for (int nt = 0; nt < T::NT; ++nt) st.acc.o[nt] *= alpha;
  }
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - st.m);
  st.e += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  if constexpr (KIND == kF32) {
    st.l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
#pragma unroll
    for (int nt = 0; nt < T::NT; ++nt)
#pragma unroll
      for (int pc = 0; pc < 2; ++pc)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = __uint_as_float(f.v[nt][pc][i]);
          if (MASK) v = t8 + 4 * pc + i < L ? v : 0.f;
          st.acc.o[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(v, p[4 * pc + i], st.acc.o[nt], 0, 0, 0);
        }
  } else {
    bf16x2 pb[4];
    float used = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pb[i] = __builtin_convertvector(f32x2{p[2 * i], p[2 * i + 1]}, bf16x2);
      used += (float)pb[i][0] + (float)pb[i][1];
    }
    st.l += used;
    const bf16x8 pw = bitcast<bf16x8>(u32x4{bitcast<uint32_t>(pb[0]), bitcast<uint32_t>(pb[1]),
                                            bitcast<uint32_t>(pb[2]), bitcast<uint32_t>(pb[3])});
#pragma unroll
    for (int nt = 0; nt < T::NT; ++nt) {
      s16x4 va, vb;  // tokens t8 .. t8 + 3 and t8 + 4 .. t8 + 7
      if constexpr (KIND == kBF16) {
        const u32x4 w = f.v[nt][0];
        va = bitcast<s16x4>(u32x2{w[0], w[1]});
        vb = bitcast<s16x4>(u32x2{w[2], w[3]});
      } else {
        const u32x2 w = f.v[nt][0];
        va = fp8x4_to_bf16x4(w[0]);
        vb = fp8x4_to_bf16x4(w[1]);
      }
      if (MASK) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          va[i] = t8 + i < L ? va[i] : (short)0;
          vb[i] = t8 + 4 + i < L ? vb[i] : (short)0;
        }
      }
      const bf16x8 vv = bitcast<bf16x8>(u32x4{bitcast<u32x2>(va)[0], bitcast<u32x2>(va)[1],
                                              bitcast<u32x2>(vb)[0], bitcast<u32x2>(vb)[1]});
      st.acc.o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, pw, st.acc.o[nt], 0, 0, 0);
    }
  }
}

// A SIMD issues for its oldest wave first, so waves given equal work finish
// in the order they started, the youngest far behind.  Each wave lowers its
// own priority as it gets through its work (`done` of `total` blocks, in
// four steps), which lets the waves that are behind catch up.
__device__ __forceinline__ void pace(int done, int total) {
  if (done * 4 < total)
    __builtin_amdgcn_s_setprio(3);
  else if (done * 2 < total)
    __builtin_amdgcn_s_setprio(2);
  else if (done * 4 < 3 * total)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
}

// A wave's un-reduced online-softmax state (per lane), handed to the wave
// of the previous range through LDS.
template <int KIND, int D>
struct FoldLds {
  f32x4 o[Tile<KIND, D>::NT][64];
  float m[64], l[64], e[64];
};

// One segment, processed by one wave: logical blocks [b_begin, b_end) of
// sequence s under kv head g.  slot < 0: the segment is the whole sequence
// and writes the final row; otherwise it writes partial state `slot`.
// done / total: the wave's progress through its range before this segment.
// absorb >= 0: before writing, wait for the state published in fold[absorb]
// (the same pair's piece in the next range) and merge it in.  publish >= 0:
// instead of writing, hand the state to the previous range's wave through
// fold[publish] and raise flag[publish].
// Partial O^T rows of a segment slot in the workspace, row major
// [slot][G][D]: element (slot, head row r, dims nt*16 ..).  The fp32 path
// keeps sum_t e^{s_t - m} v_t in fp32.  Where the output is bf16 the row is
// stored normalised by its own weight sum l, in bf16 (round to nearest even):
// half the bytes pass 1 writes among its reads (partition cuts of long
// contexts write one row set per partition), and a row of constant V stays
// exactly that constant through the merge.
__device__ __forceinline__ int64_t ws_o_at(int64_t slot, int nt, int G, int r, int D) {
  return ((int64_t)slot * G + r) * D + nt * 16;
}

// Write lane (r, q4)'s part of partial row (slot, r): O^T[nt*16 + 4 q4 + i].
template <int KIND, int D>
__device__ __forceinline__ void store_partial(const DecodeArgs& a, int64_t slot, int G, int r,
                                              int q4, const f32x4 (&o)[Tile<KIND, D>::NT],
                                              float l_run) {
  const float f = KIND == kF32 ? a.v_scale : (l_run > 0.f ? a.v_scale / l_run : 0.f);
#pragma unroll
  for (int nt = 0; nt < Tile<KIND, D>::NT; ++nt) {
    const f32x4 v = o[nt] * f;
    if constexpr (KIND == kF32) {
      *reinterpret_cast<f32x4*>(a.ws_o + ws_o_at(slot, nt, G, r, D) + 4 * q4) = v;
    } else {
      const bf16x2 lo = __builtin_convertvector(f32x2{v[0], v[1]}, bf16x2);
      const bf16x2 hi = __builtin_convertvector(f32x2{v[2], v[3]}, bf16x2);
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.ws_o) + ws_o_at(slot, nt, G, r, D) + 4 * q4) =
          u32x2{bitcast<uint32_t>(lo), bitcast<uint32_t>(hi)};
    }
  }
}

// Partial states of a wave's split-KV partitions, staged in LDS and written
// out NP at a time.  A global store joins the wave's single in-order
// vector-memory count, so each later wait for a K/V load also waits for the
// store, and under a saturated read stream a store takes about as long as a
// load: one store per partition cut costs one drain of the wave's load
// pipeline (workload 5, 512-token partitions: 556 us against 466 us without
// cuts).  Staged, a wave drains once per NP cuts.  Rows are kept as
// store_partial writes them (bf16, normalised by their own weight sum); the
// flush writes 1 KiB of contiguous rows per store instruction.
template <int KIND, int D>
struct alignas(16) PartStage {
  static constexpr int NP = KIND == kF32 ? 0 : (D == 128 ? 3 : 2);  // entries per wave
  static constexpr int N = NP > 0 ? NP : 1;
  uint16_t o[N][16][D];
  float m[N][16], l[N][16], e[N][16];
  int64_t slot[N];
};

// Stage partial state `slot` (lane (r, q4)'s share, as store_partial writes
// it) as entry n of the wave's area.
template <int KIND, int D>
__device__ __forceinline__ void stage_partial(PartStage<KIND, D>& ps, int n, const DecodeArgs& a, int64_t slot,
                                              int G, int r, int q4, int lane,
                                              const f32x4 (&o)[Tile<KIND, D>::NT], float m, float l_run,
                                              float e_run) {
  static_assert(KIND != kF32, "fp32 partial rows are stored directly");
  if (r < G) {
    const float f = l_run > 0.f ? a.v_scale / l_run : 0.f;
#pragma unroll
    for (int nt = 0; nt < Tile<KIND, D>::NT; ++nt) {
      const f32x4 v = o[nt] * f;
      const bf16x2 lo = __builtin_convertvector(f32x2{v[0], v[1]}, bf16x2);
      const bf16x2 hi = __builtin_convertvector(f32x2{v[2], v[3]}, bf16x2);
      *reinterpret_cast<u32x2*>(&ps.o[n][r][nt * 16 + 4 * q4]) = u32x2{bitcast<uint32_t>(lo), bitcast<uint32_t>(hi)};
    }
    if (q4 == 0) {
      ps.m[n][r] = m;
      ps.l[n][r] = l_run;
      ps.e[n][r] = e_run;
    }
  }
  if (lane == 0) ps.slot[n] = slot;
}

// Write the first n staged entries to the workspace.  A wave's LDS accesses
// complete in order, so its own staging writes are visible here.
template <int KIND, int D>
__device__ __forceinline__ void flush_partials(const PartStage<KIND, D>& ps, int n, const DecodeArgs& a,
                                               int G, int lane) {
  constexpr int RB = D * 2;            // bytes of a bf16 row
  constexpr int CH = 16 * RB / 1024;   // 1 KiB pieces of an entry's 16 rows
  for (int i = 0; i < n; ++i) {
    const int64_t slot = ps.slot[i];
    const char* src = reinterpret_cast<const char*>(ps.o[i]);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int byte = c * 1024 + lane * 16, row = byte / RB;
      if (row < G)
        *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(a.ws_o) + (slot * G + row) * RB + byte % RB) =
            *reinterpret_cast<const u32x4*>(src + byte);
    }
    if (lane < G) {
      const int64_t pr = slot * G + lane;
      a.ws_m[pr] = ps.m[i][lane];
      a.ws_l[pr] = ps.l[i][lane];
      a.ws_e[pr] = ps.e[i][lane];
    }
  }
}

// 16-token tiles at the start of every sequence loaded with the default
// cache policy in pass 1 (1024 tokens).  With a shared prefix the copy one
// sequence brings into L2 serves the others: on the 70B-shaped shared-prefix
// workload HBM reads fell from 1.097x to 1.018x of the unique bytes and pass
// 1 went from 0.70 to 0.76-0.80 of peak.  Without sharing the rule is neutral
// on cold caches (timing back-to-back steps of one layer shows a gain there
// that comes from these lines surviving in the MALL into the next step).
// 128 and more tiles lose, counting from each segment's start loses
// everywhere, and fp8 tiles measured flat to slightly slower, so they stream
// throughout.
template <int KIND>
struct HotTiles {
  static constexpr int value = KIND == kFP8 ? 0 : 64;
};

template <int KIND, int D, int S, int SH>
__device__ __forceinline__ void decode_segment(const DecodeArgs& a, QLds<KIND, D>& qs,
                                               FoldLds<KIND, D>* fold, int* flag, int s, int g,
                                               int b_begin, int b_end, int slot, int done,
                                               int total, int absorb, int publish, int pb,
                                               PartStage<KIND, D>* stage, int& staged) {
  static_assert(S >= 2 && S <= 4, "2 to 4 register buffers");
  using T = Tile<KIND, D>;
  constexpr int NW = 1;  // blocks of the segment are taken in order by this wave
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, q4 = lane >> 4;

  int L = as_const(a.context_lens)[s];
  L = L < 0 ? 0 : (L > a.max_context_len ? a.max_context_len : L);

  const int G = a.group;
  const int Hq = a.num_q_heads;

  // Q^T fragments of the lane's head (zero rows pad the group to 16).  They
  // are loaded first and written to this wave's LDS slot once the first K/V
  // tiles are on their way, so the three latencies (Q, table, tile) overlap.
  // A wave's LDS accesses complete in order: no barrier between segments.
  u32x4 qreg[T::NQ];
  {
    const int head = g * G + r;
    constexpr int QES = KIND == kF32 ? 4 : 2;
    const gchar_p qrow = (gchar_p) static_cast<const char*>(a.q) + ((int64_t)s * Hq + head) * D * QES;
#pragma unroll
    for (int j = 0; j < T::NQ; ++j) {
      int off;
      if constexpr (KIND == kFP8)
        off = ((j >> 1) * 4 + q4) * 32 + (j & 1) * 16;
      else
        off = (j * 4 + q4) * 16;
      qreg[j] = r < G ? *reinterpret_cast<gptr<u32x4>>(qrow + off) : u32x4{0u, 0u, 0u, 0u};
    }
  }

  // Tile b (16 tokens) lies in table entry b >> shift, half b & 1 of a
  // 32-token block.
  constexpr int shift = SH;
  const cptr<int32_t> tbl = as_const(a.block_tables) + (int64_t)s * a.max_blocks;
  const char* kbase = static_cast<const char*>(a.k_cache) + ((int64_t)g * T::BYTES << shift);
  const char* vbase = static_cast<const char*>(a.v_cache) + ((int64_t)g * T::BYTES << shift);
  const int64_t bstride = (int64_t)a.num_kv_heads * T::BYTES << shift;
  const int64_t last_block = a.num_blocks - 1;
  const TileOffsets toff = tile_offsets<KIND, D>(lane, r, q4, shift);

  // Tile bases are wave-uniform: keep them in scalar registers so each load
  // is a scalar base plus the lane's 32-bit offset.
  auto tile_of = [&](int b, gchar_p& kt, gchar_p& vt) {
    int64_t phys = __builtin_amdgcn_readfirstlane(tbl[b >> shift]);
    phys = phys < 0 ? 0 : (phys > last_block ? last_block : phys);
    const int half = b & ((1 << shift) - 1);
    kt = uniform_ptr(kbase + phys * bstride + half * (kBS * 16));
    vt = uniform_ptr(vbase + phys * bstride + half * (kBS * T::ES));
  };

  // S rotating register buffers: while block b is processed, the loads of
  // blocks b+NW .. b+(S-1)*NW are in flight.  Prefetch indices are clamped
  // (the last block is re-read from cache) so every stage issues the same
  // loads and the waits stay partial.
  RunState<KIND, D> st;
  st.init();
  // A range may hold several split-KV partitions of the pair: at each
  // partition boundary inside it the state so far goes out as the partial of
  // that partition (slot, slot + 1, ...) and a fresh state starts, while the
  // loads of the next tiles, already in flight, keep streaming.
  int to_cut = pb > 0 ? pb - b_begin % pb : 0x7fffffff;
  // Partial state `slot` out: staged when the kernel gave this wave an area
  // (flushed when it is full), else stored directly.
  auto put_partial = [&](float m_run, float l_run, float e_run) {
    if constexpr (PartStage<KIND, D>::NP > 0) {
      if (stage) {
        stage_partial<KIND, D>(*stage, staged, a, slot, G, r, q4, lane, st.acc.o, m_run, l_run, e_run);
        if (++staged == PartStage<KIND, D>::NP) {
          flush_partials<KIND, D>(*stage, staged, a, G, lane);
          staged = 0;
        }
        return;
      }
    }
    if (r < G) {
      const int64_t pr = (int64_t)slot * G + r;
      store_partial<KIND, D>(a, slot, G, r, q4, st.acc.o, l_run);
      if (q4 == 0) {
        a.ws_m[pr] = m_run;
        a.ws_l[pr] = l_run;
        a.ws_e[pr] = e_run;
      }
    }
  };
  auto cut = [&]() {
    const float l_run = sum_across_groups(st.l);
    const float e_run = sum_across_groups(st.e);
    put_partial(st.m, l_run, e_run);
    ++slot;
    st.init();
  };
  // fp8 16-token blocks are taken two at a time (a 2 KiB K tile per stage
  // leaves too little work per stage to cover a block's latency).
  // Pairs cut only at even tiles: with an odd number of tiles per partition
  // the segment takes the 16-token tile loop below instead.
  constexpr bool kPair = SH == 0 && KIND == kFP8;
  constexpr bool kWhole = (SH == 1 && KIND != kF32) || kPair;  // fp32 blocks would not fit in registers
  const bool whole = kWhole && !(kPair && (pb & 1));
  if constexpr (kWhole) if (whole) {
    // 32-token blocks (or 16-token block pairs): a stage per block.  The
    // segment's tiles [b_begin, b_end) may start or end mid-block; those
    // stages mask the other half.
    constexpr int S32 = KIND == kFP8 ? 3 : 2;  // register buffers (blocks)
    static_assert(KIND != kF32, "fp32 32-token blocks take the 16-token tile path");
    const Offsets32 o32 = kPair ? offsets_pair<KIND, D>(lane, r, q4) : offsets32<KIND, D>(lane, r, q4);
    const bool k_from_b = (lane & 15) >= 8, v_from_b = q4 >= 2;  // pair: lanes reading block B
    const int u0 = b_begin >> 1, u1 = (b_end - 1) >> 1;  // blocks, inclusive
    const int tmin = b_begin * kBS, tmax = b_end * kBS < L ? b_end * kBS : L;
    int next_cut = pb > 0 ? (b_begin / pb + 1) * pb : 0x7fffffff;  // in tiles
    int u = u0;
    auto block_of = [&](int ub, gchar_p& kt, gchar_p& vt) {
      if constexpr (kPair) {
        // tiles 2 ub and 2 ub + 1; past the segment's last tile B repeats A
        // (its tokens are masked), so no entry past the segment is read
        const int ib = 2 * ub + 1 < b_end ? 2 * ub + 1 : 2 * ub;
        int64_t pa = __builtin_amdgcn_readfirstlane(tbl[2 * ub]);
        int64_t pbk = __builtin_amdgcn_readfirstlane(tbl[ib]);
        pa = pa < 0 ? 0 : (pa > last_block ? last_block : pa);
        pbk = pbk < 0 ? 0 : (pbk > last_block ? last_block : pbk);
        kt = (gchar_p)(kbase + (k_from_b ? pbk : pa) * bstride);
        vt = (gchar_p)(vbase + (v_from_b ? pbk : pa) * bstride);
      } else {
        int64_t phys = __builtin_amdgcn_readfirstlane(tbl[ub]);
        phys = phys < 0 ? 0 : (phys > last_block ? last_block : phys);
        kt = uniform_ptr(kbase + phys * bstride);
        vt = uniform_ptr(vbase + phys * bstride);
      }
    };
    if (b_begin < b_end) {
      Frags32<KIND, D> g0, g1, g2;
      gchar_p kt, vt;
#define PKV_PREFETCH32(BUF, AHEAD)                 \
  block_of(min(u + (AHEAD), u1), kt, vt);          \
  load_block32<KIND, D, KIND == kFP8, kPair>(BUF, kt, vt, o32);
// The next block's loads go out once this block's scores are formed, so its
// K registers are free to take them: a block and a half in flight.
#define PKV_STAGE32(CUR, NXT)                                                                 \
  {                                                                                           \
    f32x4 sc[2];                                                                              \
    scores32<KIND, D>(CUR, qs, lane, sc);                                                     \
    PKV_PREFETCH32(NXT, S32 - 1)                                                              \
    if (u * 2 * kBS >= tmin && (u + 1) * 2 * kBS <= tmax)                                     \
      finish_block32<KIND, D, false>(st, CUR, sc, u * 2 * kBS, tmin, tmax, L, a.score_scale_log2, q4); \
    else                                                                                      \
      finish_block32<KIND, D, true>(st, CUR, sc, u * 2 * kBS, tmin, tmax, L, a.score_scale_log2, q4);  \
  }                                                                                           \
  pace(done + 2 * u - b_begin, total);                                                        \
  if (++u > u1) break;                                                                        \
  if (2 * u == next_cut) {                                                                    \
    cut();                                                                                    \
    next_cut += pb;                                                                           \
  }
      PKV_PREFETCH32(g0, 0)
      if constexpr (S32 >= 3) { PKV_PREFETCH32(g1, 1) }
#pragma unroll
      for (int j = 0; j < T::NQ; ++j) qs.qf[j][lane] = qreg[j];
      if constexpr (S32 == 2) {
        for (;;) { PKV_STAGE32(g0, g1) PKV_STAGE32(g1, g0) }
      } else {
        for (;;) { PKV_STAGE32(g0, g2) PKV_STAGE32(g1, g0) PKV_STAGE32(g2, g1) }
      }
#undef PKV_STAGE32
#undef PKV_PREFETCH32
    }
  }
  // 16-token tiles [b, b_stop) with cache policy STR (true: non-temporal);
  // a partition cut falling at b_stop is taken before the loop ends, so two
  // loops over one segment cut exactly where one would.
  int b = b_begin;
  auto run_tiles = [&](auto stream_tag, int b_stop) {
    constexpr bool STR = decltype(stream_tag)::value;
    if (b >= b_stop) return;
    Frags<KIND, D> f0, f1, f2, f3;
    gchar_p kt, vt;
#define PKV_PREFETCH(BUF, AHEAD)                          \
  tile_of(min(b + (AHEAD)*NW, b_stop - 1), kt, vt);       \
  load_tile<KIND, D, STR>(BUF, kt, vt, toff);
#define PKV_STAGE(CUR, NXT)                                              \
  PKV_PREFETCH(NXT, S - 1)                                               \
  process_block<KIND, D>(st, CUR, qs, b, L, L, a.score_scale_log2, lane, q4, G); \
  pace(done + (b - b_begin), total);                                     \
  b += NW;                                                               \
  if (b < b_end && --to_cut == 0) {                                      \
    cut();                                                               \
    to_cut = pb;                                                         \
  }                                                                      \
  if (b >= b_stop) break;
    PKV_PREFETCH(f0, 0)
    if constexpr (S >= 3) { PKV_PREFETCH(f1, 1) }
    if constexpr (S >= 4) { PKV_PREFETCH(f2, 2) }
#pragma unroll
    for (int j = 0; j < T::NQ; ++j) qs.qf[j][lane] = qreg[j];
    if constexpr (S == 2) {
      for (;;) { PKV_STAGE(f0, f1) PKV_STAGE(f1, f0) }
    } else if constexpr (S == 3) {
      for (;;) { PKV_STAGE(f0, f2) PKV_STAGE(f1, f0) PKV_STAGE(f2, f1) }
    } else {
      for (;;) { PKV_STAGE(f0, f3) PKV_STAGE(f1, f0) PKV_STAGE(f2, f1) PKV_STAGE(f3, f2) }
    }
#undef PKV_STAGE
#undef PKV_PREFETCH
  };
  if (!whole) {
    // The leading tiles of a sequence (where a shared prefix sits) take the
    // default cache policy, so that other sequences reading the same blocks
    // find them in L2; the rest streams with non-temporal loads.
    const int hot = b_end < HotTiles<KIND>::value ? b_end : HotTiles<KIND>::value;
    run_tiles(std::false_type{}, hot);
    run_tiles(std::integral_constant<bool, SH == 0>{}, b_end);
  }
  if (absorb >= 0) {
    // The publisher is the next wave of this workgroup, co-resident with
    // this one; it publishes right after its first piece, and a wait only
    // ever points to a higher wave (the last never waits), so the chain is at
    // most NW - 1 long and ends.  The bound (2^24 sleeps, about half a
    // second) only guards against a hang; if it ever ran out, the piece would
    // be lost, so the state becomes NaN and the row (or partial state) this
    // wave writes says so instead of holding a silently wrong value.
    bool got = false;
    for (int spin = 0; spin < (1 << 24); ++spin) {
      if (__hip_atomic_load(&flag[absorb], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != 0) {
        got = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    const FoldLds<KIND, D>& f = fold[absorb];
    const float mb = f.m[lane];
    const float M = fmaxf(st.m, mb);
    const float ca = st.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.m - M);
    const float cb = mb == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mb - M);
    st.m = M;
    st.l = ca * st.l + cb * f.l[lane];
    st.e = ca * st.e + cb * f.e[lane];
#pragma unroll
    for (int nt = 0; nt < T::NT; ++nt) st.acc.o[nt] = ca * st.acc.o[nt] + cb * f.o[nt][lane];
    if (!got) {
      st.m = __builtin_nanf("");
      st.l = st.m;
      st.e = st.m;
#pragma unroll
      for (int nt = 0; nt < T::NT; ++nt) st.acc.o[nt] = f32x4{st.m, st.m, st.m, st.m};
    }
  }
  if (publish >= 0) {
    FoldLds<KIND, D>& f = fold[publish];
#pragma unroll
    for (int nt = 0; nt < T::NT; ++nt) f.o[nt][lane] = st.acc.o[nt];
    f.m[lane] = st.m;
    f.l[lane] = st.l;
    f.e[lane] = st.e;
    __hip_atomic_store(&flag[publish], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    return;
  }
  const float m_run = st.m;
  const float l_run = sum_across_groups(st.l);
  const float e_run = sum_across_groups(st.e);
  const f32x4* o = st.acc.o;

  // ---- lane (r, q4) holds O^T[d = nt*16 + 4*q4 + i][head r]: write it out
  if (slot >= 0) {
    put_partial(m_run, l_run, e_run);
    return;
  }
  if (r >= G) return;
  const int64_t row = (int64_t)s * Hq + g * G + r;
  {
    const float inv = l_run > 0.f ? a.v_scale / l_run : 0.f;
#pragma unroll
    for (int nt = 0; nt < T::NT; ++nt) {
      const int d = nt * 16 + 4 * q4;
      if constexpr (KIND == kF32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + row * D + d) = o[nt] * inv;
      } else {
        const uint32_t lo = (uint32_t)f32_to_bf16_rne(o[nt][0] * inv) | ((uint32_t)f32_to_bf16_rne(o[nt][1] * inv) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16_rne(o[nt][2] * inv) | ((uint32_t)f32_to_bf16_rne(o[nt][3] * inv) << 16);
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + row * D + d) = u32x2{lo, hi};
      }
    }
    if (q4 == 0 && a.lse) a.lse[row] = !(e_run <= 0.f) ? (m_run + __builtin_amdgcn_logf(e_run)) * kLn2 : -INFINITY;
  }
}

// The pair holding block position st of the line (S * H past the end),
// searched in the prefix array cb[0..S].
template <typename CB>
__device__ __forceinline__ int pair_at(int64_t st, int64_t total, int T, int S, int H, CB cb) {
  if (st >= total) return S * H;
  const int g = (int)(st / T);
  const int x = (int)(st - (int64_t)g * T);
  int lo = 0, hi = S;  // largest s with cb[s] <= x (then cb[s+1] > x)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cb[mid] <= x) lo = mid; else hi = mid;
  }
  return g * S + lo;
}

// cb[S+1], cp[S+1] and, for every range, its first pair (pairs = S*Hkv for
// an empty range past the end).  One workgroup; the prefix array is searched
// in LDS when it fits.
constexpr int kPlanLds = 8192;
__global__ __launch_bounds__(1024) void decode_plan_kernel(DecodeArgs a) {
  __shared__ int wave_sums[16];
  __shared__ int carry_b, carry_p;
  __shared__ int lcb[kPlanLds];
  const int tid = threadIdx.x;
  const int S = a.num_seqs, H = a.num_kv_heads, R = a.num_ranges, pb = a.part_blocks;
  const bool in_lds = S + 1 <= kPlanLds;
  if (tid == 0) {
    carry_b = 0;
    carry_p = 0;
  }
  __syncthreads();
  for (int c0 = 0; c0 < S; c0 += 1024) {
    const int s = c0 + tid;
    const int nb = s < S ? seq_blocks(a, s) : 0;
    int tb, tp;
    const int eb = block_exclusive_scan<16>(nb, wave_sums, &tb);
    const int ep = block_exclusive_scan<16>(parts_of(nb, pb), wave_sums, &tp);
    if (s < S) {
      a.cum[s] = carry_b + eb;
      a.cum_parts[s] = carry_p + ep;
      if (in_lds) lcb[s] = carry_b + eb;
    }
    __syncthreads();
    if (tid == 0) {
      carry_b += tb;
      carry_p += tp;
    }
    __syncthreads();
  }
  const int T = carry_b;
  if (tid == 0) {
    a.cum[S] = T;
    a.cum_parts[S] = carry_p;
  }
  if (in_lds && tid == 0) lcb[S] = T;
  __syncthreads();
  const int64_t total = (int64_t)T * H;
  // (the fallback rereads this kernel's own global writes: volatile keeps
  // the reads from a stale vector L1 line)
  const volatile int* cb = in_lds ? lcb : a.cum;
  for (int r = tid; r < R; r += 1024)
    a.range_pair[r] = pair_at(range_start(r, total, R), total, T, S, H, cb);
}

// ---------------------------------------------------------------- pass 1
// Persistent: every wave owns one range.  Wave w of workgroup b takes range
// ((b mod 8) * (R / (8 NW)) + b / 8) * NW + w, so the ranges a dispatcher
// places on one XCD (workgroups are dealt to the 8 XCDs in turn) are one
// contiguous eighth of the line -- with 8 kv heads, one head per XCD,
// sharing that head's prefix blocks in the XCD's L2.  No atomics and no
// barrier beyond the plan's; a wave waits only for the next wave of its
// workgroup, when their ranges share a pair (folding, below).
// PLAN (up to kFusedPlanSeqs sequences): every workgroup builds the prefix
// arrays in its LDS from context_lens and each wave finds its first pair;
// workgroup 0 also stores them for pass 2.  Otherwise decode_plan_kernel
// has built them beforehand.
constexpr int kFusedPlanSeqs = 1024;
template <int KIND, int D, int NW, int S, bool PLAN, int SH>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void decode_partitions_kernel(DecodeArgs a) {
  __shared__ QLds<KIND, D> qs[NW];
  // Folding (no partition cuts) and partial staging (cuts) never run in one
  // launch: they share this area.
  constexpr size_t kFoldBytes = sizeof(FoldLds<KIND, D>) * (NW - 1);
  constexpr size_t kStageBytes = PartStage<KIND, D>::NP > 0 ? sizeof(PartStage<KIND, D>) * NW : 0;
  __shared__ __attribute__((aligned(16))) char fold_area[kFoldBytes > kStageBytes ? kFoldBytes : kStageBytes];
  FoldLds<KIND, D>* fold = reinterpret_cast<FoldLds<KIND, D>*>(fold_area);
  __shared__ int flag[NW - 1];
  __shared__ int lcb[PLAN ? kFusedPlanSeqs + 1 : 1];
  __shared__ int lcp[PLAN ? kFusedPlanSeqs + 1 : 1];
  __shared__ int wsums[NW];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int R = a.num_ranges;
  const int groups = R / NW;
  const int rg = ((blockIdx.x & 7) * (groups >> 3) + (blockIdx.x >> 3)) * NW + w;
  const int nseq = a.num_seqs, H = a.num_kv_heads, pb = a.part_blocks;
  if (threadIdx.x < NW - 1) flag[threadIdx.x] = 0;
  if constexpr (!PLAN) __syncthreads();
  if constexpr (PLAN) {
    const int tid = threadIdx.x;
    int carry_b = 0, carry_p = 0;
    for (int c0 = 0; c0 < nseq; c0 += NW * 64) {
      const int s = c0 + tid;
      const int nb = s < nseq ? seq_blocks(a, s) : 0;
      int tb, tp;
      const int eb = block_exclusive_scan<NW>(nb, wsums, &tb);
      const int ep = block_exclusive_scan<NW>(parts_of(nb, pb), wsums, &tp);
      if (s < nseq) {
        lcb[s] = carry_b + eb;
        lcp[s] = carry_p + ep;
      }
      carry_b += tb;
      carry_p += tp;
    }
    if (tid == 0) {
      lcb[nseq] = carry_b;
      lcp[nseq] = carry_p;
    }
    __syncthreads();
    if (blockIdx.x == 0)
      for (int s = tid; s <= nseq; s += NW * 64) {
        a.cum[s] = lcb[s];
        a.cum_parts[s] = lcp[s];
      }
  }
  const cptr<int32_t> gcb = as_const(a.cum);
  const cptr<int32_t> gcp = as_const(a.cum_parts);
  auto cb = [&](int i) -> int {
    if constexpr (PLAN) return lcb[i]; else return gcb[i];
  };
  auto cp = [&](int i) -> int {
    if constexpr (PLAN) return lcp[i]; else return gcp[i];
  };
  const int T = cb(nseq), PT = cp(nseq);
  const int64_t total = (int64_t)T * H;
  int64_t x = range_start(rg, total, R);
  const int64_t x1 = range_start(rg + 1, total, R);
  if (x >= x1) return;
  const int64_t x_first = x;
  // Folding needs every range non-empty and no partition cuts.
  const bool fold_on = pb == 0 && total >= R;
  int P;
  if constexpr (PLAN)
    P = pair_at(x, total, T, nseq, H, lcb);
  else
    P = as_const(a.range_pair)[rg];
  int g = P / nseq, s = P % nseq;
  PartStage<KIND, D>* stage = PartStage<KIND, D>::NP > 0 && pb > 0
                                  ? reinterpret_cast<PartStage<KIND, D>*>(fold_area) + w
                                  : nullptr;
  int staged = 0;
  while (x < x1 && g < H) {
    const int64_t ps = (int64_t)g * T + cb(s);
    const int nblk = cb(s + 1) - cb(s);
    if (ps + nblk <= x) {  // pair ends at or before x (empty pairs too): next pair
      if (++s == nseq) {
        s = 0;
        ++g;
      }
      continue;
    }
    const int lo = (int)(x - ps);
    const int pidx = pb > 0 ? lo / pb : 0;  // first partition of the segment
    int hi = nblk;  // the segment runs to the pair's or the range's end
    hi = (int64_t)hi < x1 - ps ? hi : (int)(x1 - ps);
    // Folding: a pair's pieces in the ranges of one workgroup are merged in
    // LDS into the leftmost one, which alone writes (the final row when the
    // pair starts there and ends in this workgroup).  A wave publishes its
    // first piece when the pair began in an earlier range; before writing
    // (or publishing) a last piece whose pair goes on into the next range of
    // the workgroup, it absorbs that range's first piece.  Waits only ever
    // point to the next wave, so they end.
    const int64_t pe = ps + nblk;
    const bool publish = fold_on && x == x_first && lo > 0 && w != 0;
    const bool absorb = fold_on && ps + hi == x1 && hi < nblk && w != NW - 1;
    const bool whole = fold_on ? lo == 0 && range_of(pe - 1, total, R) / NW == rg / NW
                               : lo == 0 && hi == nblk && (pb == 0 || nblk <= pb);
    const int slot = g * PT + cp(s) + pidx + rg;
    decode_segment<KIND, D, S, SH>(a, qs[w], fold, flag, s, g, lo, hi, whole ? -1 : slot,
                               (int)(x - x_first), (int)(x1 - x_first), absorb ? w : -1,
                               publish ? w - 1 : -1, pb, stage, staged);
    x = ps + hi;
  }
  if constexpr (PartStage<KIND, D>::NP > 0)
    if (staged > 0) flush_partials<KIND, D>(*stage, staged, a, a.group, threadIdx.x & 63);
}

// Register buffers (prefetch depth + 1) per cache dtype, at two waves per
// SIMD (eight per CU).  Three measured the same as two buffers at three
// waves per SIMD, and leave registers for the fold merge.
#ifndef PKV_DEPTH_F32
#define PKV_DEPTH_F32 2
#endif
#ifndef PKV_DEPTH_BF16
#define PKV_DEPTH_BF16 3
#endif
#ifndef PKV_DEPTH_FP8
#define PKV_DEPTH_FP8 3
#endif
template <int KIND>
struct Depth;
template <>
struct Depth<kF32> {
  static constexpr int value = PKV_DEPTH_F32;
};
template <>
struct Depth<kBF16> {
  static constexpr int value = PKV_DEPTH_BF16;
};
template <>
struct Depth<kFP8> {
  static constexpr int value = PKV_DEPTH_FP8;
};

}  // namespace

// ---------------------------------------------------------------- launchers
// Workgroups of `kernel` (NW waves each) that fit on the current device at
// once, cached per device and kernel variant (`variant` < 32 names it).  Computed from the kernel's
// register and LDS use against gfx950's limits (512 VGPRs per SIMD lane with
// the accumulation registers unified, 160 KiB LDS and at most 8 waves per
// SIMD): the runtime's occupancy query assumes 256 VGPRs here and would
// leave two thirds of the GPU idle for a 168-register kernel.
template <typename K>
static int resident_groups(K kernel, int nw, int variant, hipError_t* err) {
  static std::atomic<int> cache[64][32];
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return 0;
  const bool cached = dev >= 0 && dev < 64 && variant >= 0 && variant < 32;
  if (cached) {
    const int c = cache[dev][variant].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  hipFuncAttributes attr;
  *err = hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(kernel));
  if (*err != hipSuccess) return 0;
  int cus = 0;
  *err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (*err != hipSuccess) return 0;
  const int regs = attr.numRegs > 0 ? (attr.numRegs + 7) / 8 * 8 : 8;
  int waves_per_simd = 512 / regs;
  waves_per_simd = waves_per_simd > 8 ? 8 : (waves_per_simd < 1 ? 1 : waves_per_simd);
  int per_cu = waves_per_simd * 4 / nw;
  const size_t lds = attr.sharedSizeBytes;
  if (lds > 0) {
    const int by_lds = (int)((160u * 1024u) / lds);
    per_cu = per_cu < by_lds ? per_cu : by_lds;
  }
  per_cu = per_cu < 1 ? 1 : per_cu;
  const int n = per_cu * (cus > 0 ? cus : 1);
  if (cached) cache[dev][variant].store(n, std::memory_order_relaxed);
  return n;
}

int decode_ranges(int cache, int D, int num_seqs, int block_shift, int64_t max_blocks_total,
                  hipError_t* err) {
  *err = hipSuccess;
  int groups = 0;
  const bool plan = num_seqs <= kFusedPlanSeqs;
  const int variant = ((cache * 2 + (D == 128 ? 1 : 0)) * 2 + (plan ? 1 : 0)) * 2 + block_shift;
#define PKV_R(C_, D_, SH_)                                                                              \
  if (cache == C_ && D == D_ && block_shift == SH_)                                                     \
    groups = plan ? resident_groups(decode_partitions_kernel<C_, D_, kWavesPerGroup, Depth<C_>::value, true, SH_>, kWavesPerGroup, variant, err) \
                  : resident_groups(decode_partitions_kernel<C_, D_, kWavesPerGroup, Depth<C_>::value, false, SH_>, kWavesPerGroup, variant, err);
  PKV_R(kF32, 64, 0) PKV_R(kF32, 128, 0) PKV_R(kBF16, 64, 0) PKV_R(kBF16, 128, 0) PKV_R(kFP8, 64, 0)
  PKV_R(kFP8, 128, 0) PKV_R(kF32, 64, 1) PKV_R(kF32, 128, 1) PKV_R(kBF16, 64, 1) PKV_R(kBF16, 128, 1)
  PKV_R(kFP8, 64, 1) PKV_R(kFP8, 128, 1)
#undef PKV_R
  // one range per resident wave; workgroups in multiples of 8 (one per XCD);
  // never more ranges than the blocks that can exist
  groups = groups / 8 * 8;
  if (groups < 8) groups = 8;
  const int64_t cap_groups = ((max_blocks_total + 8 * kWavesPerGroup - 1) / (8 * kWavesPerGroup)) * 8;
  if (cap_groups < groups) groups = (int)(cap_groups < 8 ? 8 : cap_groups);
  const int n = groups * kWavesPerGroup;
  return n < kMaxRanges ? n : kMaxRanges / (8 * kWavesPerGroup) * (8 * kWavesPerGroup);
}

hipError_t launch_decode_partitions(const DecodeArgs& a, int cache, int D, hipStream_t stream,
                                    bool* supported) {
  *supported = true;
  if (a.num_seqs == 0) return hipSuccess;
  const int block = kWavesPerGroup * 64;
  const dim3 grid(a.num_ranges / kWavesPerGroup);
#define PKV_P1(C_, D_, SH_)                                                                     \
  if (cache == C_ && D == D_ && a.block_shift == SH_) {                                         \
    if (a.num_seqs <= kFusedPlanSeqs) {                                                         \
      hipLaunchKernelGGL((decode_partitions_kernel<C_, D_, kWavesPerGroup, Depth<C_>::value, true, SH_>), \
                         grid, dim3(block), 0, stream, a);                                      \
      return hipGetLastError();                                                                 \
    }                                                                                           \
    hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, stream, a);                  \
    hipError_t err = hipGetLastError();                                                         \
    if (err != hipSuccess) return err;                                                          \
    hipLaunchKernelGGL((decode_partitions_kernel<C_, D_, kWavesPerGroup, Depth<C_>::value, false, SH_>), \
                       grid, dim3(block), 0, stream, a);                                        \
    return hipGetLastError();                                                                   \
  }
  PKV_P1(kF32, 64, 0) PKV_P1(kF32, 128, 0) PKV_P1(kBF16, 64, 0) PKV_P1(kBF16, 128, 0)
  PKV_P1(kFP8, 64, 0) PKV_P1(kFP8, 128, 0) PKV_P1(kF32, 64, 1) PKV_P1(kF32, 128, 1)
  PKV_P1(kBF16, 64, 1) PKV_P1(kBF16, 128, 1) PKV_P1(kFP8, 64, 1) PKV_P1(kFP8, 128, 1)
#undef PKV_P1
  *supported = false;
  return hipSuccess;
}

}  // namespace pkv
