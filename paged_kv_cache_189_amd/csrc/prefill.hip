// Chunked-prefill attention over the paged KV cache for CDNA4 (gfx950).
//
// What is computed: the pages name chunked prefill only as an engine setting
// ("Optimizing vLLM Throughput with PagedAttention and Continuous Batching
// for Llama 3"; "vLLM PagedAttention Optimization: Complete Step-by-Step
// Tuning Guide for Low-Latency Inference", Step 2).  Read plainly: the query
// tokens of a prompt chunk attend causally to every cached token of their
// sequence up to their own position, through the same block tables and pool
// as decode, the chunk's own K and V already written to the cache.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "device_common.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

// ---------------------------------------------------------------- chunked prefill
// One workgroup of NWV waves per (kv head g, sequence s, item of NWV * NR
// query tiles).  A
// query tile holds tokens_per_tile = 16 / G query tokens of the chunk, row
// r = token r / G, head r % G, so the G heads of a token share every K/V
// fragment as in decode; wave w owns NR consecutive query tiles.  Row r's
// token sits at position p = L - C + j of its sequence and sees tokens 0..p
// (causal); the workgroup walks the context up to its last row's position in
// 32-token steps (two 16-token K/V tiles).  A step is copied from the pool
// straight into LDS (global_load_lds, 16 bytes a lane, no registers in
// between), an equal share by each wave, PD + 1 steps ahead of its P.V, into
// PD + 2 buffers with one barrier per step; all waves run their query tiles
// against it, so a K/V byte is fetched once per NWV * NR query tiles.
// Rows past the chunk copy the wave's last row and are not written; rows with
// p < 0 (chunk longer than the context) are written as zeros.
//
// Per step a row tile costs 2 x (D / 32) score MFMAs and D / 16 P.V MFMAs of
// 16x16x32.  The score MFMAs take the step's tokens in an order that leaves
// each lane the scores of 8 consecutive tokens of its row, exactly the P
// operand of one P.V MFMA, whose V operand is then 8 consecutive tokens of
// one dim: 16 contiguous bytes of a pool V row.  About 40 VALU instructions
// of online softmax go with them.  Steps every row of the item sees in full
// take a loop with no causal masking.
#ifndef PKV_PREFILL_WAVES
#define PKV_PREFILL_WAVES 4  // waves per workgroup where a step has copies for them all
#endif
template <int KIND, int D>
struct PrefillCfg {
  using T = Tile<KIND, D>;
  static constexpr int NR = KIND == kF32 ? 1 : 2;  // query tiles per wave
  static constexpr int NC = T::BYTES / 1024;        // 1 KiB copies per 16-token tile
  static constexpr int NWV = 4 * NC >= PKV_PREFILL_WAVES ? PKV_PREFILL_WAVES : 4;  // waves per workgroup
  static constexpr int PD = 2;                      // steps in flight past the one scored next
  static constexpr int NBUF = PD + 2;               // LDS step buffers
  static constexpr int NCW = 4 * NC / NWV;          // copies per wave per step
  static_assert(NWV == 4 || NWV == 8, "waves per workgroup");
  static_assert(NCW >= 1 && (4 * NC) % NWV == 0, "step split");
  static_assert(PD * NCW <= 63, "vmcnt range");
};

// One 32-token step (tiles 2u and 2u + 1) in LDS, in 16-byte units.  K: each
// tile as the pool holds a 16-token block, [D * ES / 16][16 tokens][16 bytes],
// the second tile 64 bytes further on, so a read of tokens of both tiles by 16
// lanes spreads over all banks.  V: unit (d, u) = V[tokens 16 * u / ES ..][d]
// (ES bytes a token, 16 / ES tokens a unit) at unit index ((d / 16) * ES + u) *
// 16 + d % 16 of its tile, so the units of one u and 16 consecutive d -- what
// 16 lanes of a P.V operand read -- are 256 contiguous bytes.
template <int KIND, int D>
struct PfStep {
  static constexpr int B = Tile<KIND, D>::BYTES;
  static constexpr int KPAD = 64;
  static constexpr int VOFS = 2 * B + KPAD;  // V's first byte
  u32x4 k[(2 * B + KPAD) / 16];
  u32x4 v[2][B / 16];
};

// Copy 16 bytes a lane from global memory (base + voff) to LDS at lds + lane
// * 16, tracked by vmcnt only.  Written as asm so the compiler, which does
// not follow these copies by buffer, adds no wait of its own before every
// LDS read: callers wait with vm_wait before the barrier that publishes a
// step.  No output register: the copy writes only LDS.
__device__ __forceinline__ void copy_to_lds(gchar_p base, uint32_t voff, uint32_t lds) {
  // (lds is wave-uniform; readfirstlane keeps it in a scalar register)
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(base),
               "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

template <int ES>
struct ElemOf;
template <>
struct ElemOf<1> {
  using T = uint8_t;
};
template <>
struct ElemOf<2> {
  using T = uint16_t;
};
template <>
struct ElemOf<4> {
  using T = uint32_t;
};

// Zero the elements of a V piece (consecutive tokens of one dim) from token
// index `lim` of the piece on: V rows past the sequence may hold anything.
template <int ES, typename PT>
__device__ __forceinline__ PT zero_from(PT v, int lim) {
  constexpr int N = sizeof(PT) / ES;
  struct A {
    typename ElemOf<ES>::T e[N];
  };
  A x = bitcast<A>(v);
#pragma unroll
  for (int e = 0; e < N; ++e)
    if (e >= lim) x.e[e] = 0;
  return bitcast<PT>(x);
}

// +inf in a scalar register the compiler cannot see through (a plain s_mov,
// no memory access): med3(a, b, +inf) = max(a, b) then stays one v_med3
// instead of being folded into a max that first quiets NaN operands.
__device__ __forceinline__ float opaque_inf() {
  float r;
  asm("s_mov_b32 %0, 0x7f800000" : "=s"(r));
  return r;
}

// max(a, b, c) in one instruction.  Written as asm: from fmaxf the compiler
// first quiets possible signalling NaNs of the MFMA results, one more
// instruction per operand.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Row max over the 16 lanes of a head (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float row_max(float v, float pinf) {
  uint32_t u = __float_as_uint(v);
  auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __builtin_amdgcn_fmed3f(__uint_as_float(s16[0]), __uint_as_float(s16[1]), pinf);
  u = __float_as_uint(v);
  auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_amdgcn_fmed3f(__uint_as_float(s32[0]), __uint_as_float(s32[1]), pinf);
}

// S^T[token 4*q4+i][row r] of one 16-token tile from its K fragments (LDS)
// and the row tile's Q^T fragments (registers).
template <int KIND, int D>
__device__ __forceinline__ f32x4 pf_scores(const u32x4 (&kf)[Tile<KIND, D>::NK],
                                           const u32x4 (&q)[Tile<KIND, D>::NQ]) {
  using T = Tile<KIND, D>;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (KIND == kBF16) {
#pragma unroll
    for (int j = 0; j < T::NK; ++j)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(kf[j]), bitcast<bf16x8>(q[j]), acc, 0, 0, 0);
  } else if constexpr (KIND == kFP8) {
#pragma unroll
    for (int j = 0; j < T::NK; ++j) {
      u32x4 lo, hi;
      fp8x16_to_bf16(kf[j], lo, hi);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(lo), bitcast<bf16x8>(q[2 * j]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(hi), bitcast<bf16x8>(q[2 * j + 1]), acc, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int j = 0; j < T::NK; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kf[j][e]), __uint_as_float(q[j][e]), acc, 0, 0, 0);
  }
  return acc;
}

// Online-softmax state of one row tile: running max m (log2 units), the
// bump threshold m + kLazyMax in raw-score units ((m + kLazyMax) / scale, so
// a raw max is compared without scaling it), the fp32 sum of the weights
// (for the lse), the sum of the weights as P.V multiplies them (rounded to
// bf16 for the MFMA; the output's normaliser, so that their rounding scales
// numerator and denominator alike), and O^T.
template <int KIND, int D>
struct PfState {
  float m, thr, l;
  f32x4 lr;  // (an MFMA of a ones operand with P: every element the row's sum)
  Acc<KIND, D> acc;
};

template <int KIND, int D, int SH>
__device__ __forceinline__ void prefill_item(const PrefillArgs& a, PfStep<KIND, D>* kv, int w,
                                             int s, int g, int item) {
  using T = Tile<KIND, D>;
  using C_ = PrefillCfg<KIND, D>;
  constexpr int NR = C_::NR, PD = C_::PD, NC = C_::NC, NCW = C_::NCW;
  constexpr int shift = SH;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, q4 = lane >> 4;
  const int G = a.group, NQ = a.tokens_per_tile, Hq = a.num_q_heads;
  const cptr<int32_t> qst = as_const(a.query_start);
  const int q0 = qst[s], C = qst[s + 1] - q0;
  int Ls = as_const(a.context_lens)[s];
  Ls = Ls < 0 ? 0 : (Ls > a.max_context_len ? a.max_context_len : Ls);
  const int per_wave = NQ * NR;
  constexpr int NWV = C_::NWV;
  const int ibase = item * NWV * per_wave;             // first chunk token of the item
  const int ilast = (ibase + NWV * per_wave < C ? ibase + NWV * per_wave : C) - 1;
  const int Lmax = Ls - C + ilast + 1;                  // tokens the item's last row sees
  const int Lmin = Ls - C + ibase + 1;                  // ... and its first row
  const int jbase = ibase + w * per_wave;               // this wave's first token
  const int jlast = jbase + per_wave - 1 < ilast ? jbase + per_wave - 1 : ilast;
  const int jfall = jlast >= jbase ? jlast : ilast;     // stand-in for rows past the chunk
  const int jl = r / G, hh = r % G;

  const float pinf = opaque_inf();
  const bool qneg = a.score_scale_log2 < 0.f;  // fold the sign into Q (exact)
  const float scl = qneg ? -a.score_scale_log2 : a.score_scale_log2;
  const float inv_scl = scl > 0.f ? 1.f / scl : INFINITY;  // scale 0: no bump after the first
  const uint32_t qflip = !qneg ? 0u : (KIND == kF32 ? 0x80000000u : 0x80008000u);
  int L[NR];
  bool row_ok[NR];
  gchar_p qrow[NR];
  constexpr int QES = KIND == kF32 ? 4 : 2;
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    const int j = jbase + k * NQ + jl;
    row_ok[k] = r < NQ * G && j <= jlast;
    const int jj = row_ok[k] ? j : jfall;
    const int Lrow = Ls - C + jj + 1;
    L[k] = Lrow > 1 ? Lrow : 1;  // empty rows look at token 0, then write zeros
    qrow[k] = (gchar_p) static_cast<const char*>(a.q) +
              ((int64_t)(q0 + jj) * Hq + g * G + (r < NQ * G ? hh : 0)) * D * QES;
  }
  u32x4 q[NR][T::NQ];  // Q^T fragments, kept in registers for the whole item
  auto load_q = [&]() {
#pragma unroll
    for (int k = 0; k < NR; ++k)
#pragma unroll
      for (int jq = 0; jq < T::NQ; ++jq) {
        int off;
        if constexpr (KIND == kFP8)
          off = ((jq >> 1) * 4 + q4) * 32 + (jq & 1) * 16;
        else
          off = (jq * 4 + q4) * 16;
        q[k][jq] = *reinterpret_cast<gptr<u32x4>>(qrow[k] + off) ^ qflip;
      }
  };

  // The copies of a step: 4 * NC of 1 KiB, copy idx = (kind * 2 + tile) *
  // NC + c for K (kind 0) and V (kind 1) of tiles 2u, 2u + 1 and the tile's
  // 1 KiB chunk c; wave w does idx = w + NWV * i.  With NC >= NWV copy i of
  // every wave has kind and tile (i * NWV / NC) >> 1 and & 1; with NC < NWV
  // (both powers of two) a wave copies from the one tile (w / NC) & 1, copy i
  // of kind (NWV * i / NC + w / NC) >> 1.  A lane copies LDS unit c * 64 +
  // lane of the tile (the step layout above); a pool of 2^shift * 16-token
  // blocks holds a tile's row
  // (K: 16 tokens x 16 bytes of one dim group; V: the 16 tokens of one dim)
  // at row * (row bytes << shift) from the tile's start.
  constexpr bool BOTH = NC >= NWV;  // each wave copies from both tiles of a step
  const int wtile = BOTH ? 0 : (w / NC) & 1;
  uint32_t csrc[NCW], cdst[NCW];
#pragma unroll
  for (int i = 0; i < NCW; ++i) {
    const int idx = w + NWV * i, kh = idx / NC, c = idx % NC;
    const uint32_t t = (uint32_t)(c * 1024 + lane * 16), un = t / 16;
    constexpr uint32_t VR = 16u * T::ES;  // V row bytes of a 16-token tile
    const uint32_t ks = ((t >> 8) << (8 + shift)) + (t & 255u);
    const uint32_t vd = un / (16 * T::ES) * 16 + un % 16, vu = un / 16 % T::ES;
    const uint32_t vs = vd * (VR << shift) + vu * 16;
    csrc[i] = kh >= 2 ? vs : ks;
    cdst[i] = (kh >= 2 ? (uint32_t)PfStep<KIND, D>::VOFS + (uint32_t)(kh & 1) * T::BYTES
                       : (uint32_t)(kh & 1) * (T::BYTES + PfStep<KIND, D>::KPAD)) + (uint32_t)c * 1024;
  }
  // LDS reads.  Score MFMA h takes step token 8 * (m / 4) + 4 * h + m % 4 as
  // its row m, so lane (q4, r) gets the scores of step tokens 8 * q4 + 4 * h +
  // i, i < 4: tokens 8 * q4 .. 8 * q4 + 7 of its row over h = 0, 1.  Its V
  // operand is then V[tokens 8 * q4 ..][d], in tile q4 / 2 from token 8 * (q4
  // % 2): unit u = (q4 % 2) * ES / 2 of dim d (fp8: half of unit 0).
  uint32_t koff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int sg = 8 * (r >> 2) + 4 * h + (r & 3);
    koff[h] = (uint32_t)((sg >> 4) * (T::BYTES + PfStep<KIND, D>::KPAD) + q4 * 256 + (sg & 15) * 16);
  }
  const uint32_t voff = (uint32_t)(PfStep<KIND, D>::VOFS + (q4 >> 1) * T::BYTES +
                                   (KIND == kFP8 ? r * 16 + (q4 & 1) * 8 : ((q4 & 1) * T::ES / 2 * 16 + r) * 16));

  const cptr<int32_t> tbl = as_const(a.block_tables) + (int64_t)s * a.max_blocks;
  const char* kbase = static_cast<const char*>(a.k_cache) + ((int64_t)g * T::BYTES << shift);
  const char* vbase = static_cast<const char*>(a.v_cache) + ((int64_t)g * T::BYTES << shift);
  // (the launcher refuses block strides of 2^32 bytes or more)
  const uint32_t bstride = (uint32_t)a.num_kv_heads * (uint32_t)(T::BYTES << shift);
  // (table entries are int32, so the clamp runs in 32 bits, on the scalar unit)
  const int last_block = a.num_blocks - 1 < INT32_MAX ? (int)(a.num_blocks - 1) : INT32_MAX;
  const int n16 = Lmax > 0 ? (Lmax + kBS - 1) / kBS : 0;  // 16-token tiles to read
  const int n32 = (n16 + 1) >> 1;                           // steps
  // Steps every row of the item sees in full (no causal masking needed).
  int u_full = Lmin > 0 ? Lmin / (2 * kBS) : 0;
  u_full = u_full < n32 ? u_full : n32;

  PfState<KIND, D> st[NR];
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    st[k].m = -INFINITY;
    st[k].thr = -INFINITY;
    st[k].l = 0.f;
    st[k].lr = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < T::NT; ++nt) st[k].acc.o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // Table entries of the tiles of step j this wave copies from (past the
  // context: its last tile).  Both tiles of a step share one entry when a
  // block holds 32 tokens.
  constexpr int NID = BOTH && shift == 0 ? 2 : 1;
  auto tile_of = [&](int j, int h) {
    const int t16 = 2 * j + h;
    return t16 < n16 - 1 ? t16 : n16 - 1;
  };
  auto ids_of = [&](int j, int (&id)[NID]) {
#pragma unroll
    for (int h = 0; h < NID; ++h)
      id[h] = __builtin_amdgcn_readfirstlane(tbl[(uint32_t)tile_of(j, BOTH ? h : wtile) >> shift]);
  };
  // Start the copies of step j into the LDS buffer at byte address lds.
  // Default cache policy: every item of the sequence reads these tiles, and
  // the items of a (head, sequence) pair run side by side on one XCD.
  auto copy_step = [&](int j, const int (&id)[NID], uint32_t lds) {
    constexpr int NT2 = BOTH ? 2 : 1;
    const char* kt[NT2];
    const char* vt[NT2];
#pragma unroll
    for (int h = 0; h < NT2; ++h) {
      const int t16 = tile_of(j, BOTH ? h : wtile);
      const int e = id[NID == 2 ? h : 0];
      const int p32 = e < 0 ? 0 : (e > last_block ? last_block : e);
      const int half = t16 & ((1 << shift) - 1);
      const uint64_t off = (uint64_t)(uint32_t)p32 * bstride;  // p32 >= 0
      kt[h] = kbase + off + half * (kBS * 16);
      vt[h] = vbase + off + half * (kBS * T::ES);
    }
#pragma unroll
    for (int i = 0; i < NCW; ++i) {
      const char* src;
      if constexpr (BOTH) {
        constexpr int NWV_ = C_::NWV;
        const int kh = i * NWV_ / NC;  // compile-time once unrolled
        src = (kh >> 1) ? vt[kh & 1] : kt[kh & 1];
      } else {
        constexpr int NWV_ = C_::NWV;
        src = ((NWV_ * i / NC + w / NC) >> 1) ? vt[0] : kt[0];
      }
      copy_to_lds(uniform_ptr(src), csrc[i], lds + cdst[i]);
    }
  };

  using PB = typename std::conditional<KIND == kF32, f32x4, bf16x8>::type;
  constexpr int NPB = KIND == kF32 ? 2 : 1;
  // S^T of a step for every row tile, from the step's K in LDS.
  auto scores_of = [&](const PfStep<KIND, D>& t, f32x4 (&sc)[NR][2]) {
    const char* kb = reinterpret_cast<const char*>(t.k);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 kf[T::NK];
#pragma unroll
      for (int j = 0; j < T::NK; ++j) kf[j] = *reinterpret_cast<const u32x4*>(kb + koff[h] + j * 1024);
#pragma unroll
      for (int k = 0; k < NR; ++k) sc[k][h] = pf_scores<KIND, D>(kf, q[k]);
    }
  };
  // Raw scores of step u (past each row's causal bound -> -inf when MASK),
  // each lane's max of them, and whether some row's running max must move.
  // The scale (> 0: a negative one was moved into Q) is applied inside the
  // exponent, p = 2^(s * scale - m).
  auto max_of = [&](const f32x4 (&sc)[NR][2], int u, auto masked, float (&x)[NR][8],
                    float (&mx)[NR]) {
    constexpr bool MASK = decltype(masked)::value;
    bool any = false;
#pragma unroll
    for (int k = 0; k < NR; ++k) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = sc[k][h][i];
          if (MASK) v = u * 2 * kBS + 8 * q4 + 4 * h + i < L[k] ? v : -INFINITY;
          x[k][h * 4 + i] = v;
        }
      const float m3a = max3(x[k][0], x[k][1], x[k][2]);
      const float m3b = max3(x[k][3], x[k][4], x[k][5]);
      const float m2c = __builtin_amdgcn_fmed3f(x[k][6], x[k][7], pinf);
      mx[k] = max3(m3a, m3b, m2c);  // this lane's max (raw); the row's below
      // always true on a row's first step; false for NaN
      any = any || mx[k] > st[k].thr;
    }
    return any;
  };
  // The row max across the 4 lanes of each row and which rows move their
  // running max: needed only when some lane's own max passed its row's
  // threshold (raw scores against a raw threshold: the row's max passes it
  // exactly when one of its lanes' does).
  auto row_bumps = [&](float (&mx)[NR], bool (&bump)[NR]) {
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      mx[k] = row_max(mx[k], pinf);
      bump[k] = mx[k] > st[k].thr;
      mx[k] *= scl;
    }
  };
  // Move the running max before a step's weights are formed; O must already
  // hold every earlier step.  Lanes without a bump rescale by 2^0 = 1.
  auto rescale = [&](const float (&mx)[NR], const bool (&bump)[NR]) {
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const float m_new = bump[k] ? mx[k] : st[k].m;
      const float alpha = __builtin_amdgcn_exp2f(st[k].m - m_new);
      st[k].m = m_new;
      st[k].thr = (m_new + kLazyMax) * inv_scl;
      st[k].l *= alpha;
      st[k].lr *= alpha;
#pragma unroll
      for (int nt = 0; nt < T::NT; ++nt) st[k].acc.o[nt] *= alpha;
    }
  };
  // Weights of a step, summed into l (fp32) and packed as P.V operands:
  // p[e] is the weight of step token 8 * q4 + e.
  auto weights_of = [&](const float (&x)[NR][8], auto masked, PB (&pw)[NR][NPB]) {
    constexpr bool MASK = decltype(masked)::value;
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[k][i], scl, -st[k].m));
        if (MASK) p[i] = x[k][i] == -INFINITY ? 0.f : p[i];
      }
      st[k].l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      if constexpr (KIND == kF32) {
        pw[k][0] = f32x4{p[0], p[1], p[2], p[3]};
        pw[k][1] = f32x4{p[4], p[5], p[6], p[7]};
      } else {
        const bf16x2 p01 = __builtin_convertvector(f32x2{p[0], p[1]}, bf16x2);
        const bf16x2 p23 = __builtin_convertvector(f32x2{p[2], p[3]}, bf16x2);
        const bf16x2 p45 = __builtin_convertvector(f32x2{p[4], p[5]}, bf16x2);
        const bf16x2 p67 = __builtin_convertvector(f32x2{p[6], p[7]}, bf16x2);
        const u32x4 pp = {bitcast<uint32_t>(p01), bitcast<uint32_t>(p23), bitcast<uint32_t>(p45),
                          bitcast<uint32_t>(p67)};
        pw[k][0] = bitcast<bf16x8>(pp);
      }
    }
  };
  // A lane's V operands of a step: for each 16-dim tile, V[tokens 8 * q4 ..
  // 8 * q4 + 7][d] (fp32: two halves of 4 tokens).  Read ahead of their use
  // so the stage's softmax work covers the LDS latency.
  using VR = typename std::conditional<KIND == kBF16, u32x4, typename std::conditional<KIND == kFP8, u32x2, u32x4>::type>::type;
  constexpr int NVR = KIND == kF32 ? 2 * T::NT : T::NT;
  auto read_v = [&](const PfStep<KIND, D>& t, VR (&vr)[NVR]) {
    const char* vb = reinterpret_cast<const char*>(t.k) + voff;  // V follows K in the step
#pragma unroll
    for (int nt = 0; nt < T::NT; ++nt) {
      if constexpr (KIND == kF32) {  // units u and u + 1: 4 tokens each
        vr[2 * nt] = *reinterpret_cast<const u32x4*>(vb + nt * 256 * T::ES);
        vr[2 * nt + 1] = *reinterpret_cast<const u32x4*>(vb + nt * 256 * T::ES + 256);
      } else {
        vr[nt] = *reinterpret_cast<const VR*>(vb + nt * 256 * T::ES);
      }
    }
  };
  // O^T[d][row] += V^T . P^T over the 32 tokens of step u.  On the step
  // holding the end of what the item reads, V past Lmax is zeroed: those
  // weights are 0 but the slots may hold NaN.
  auto pv_of = [&](const VR (&vr)[NVR], const PB (&pw)[NR][NPB], int u, bool tail) {
    const int lim = Lmax - (u * 2 * kBS + 8 * q4);  // valid tokens of this lane's 8
#pragma unroll
    for (int nt = 0; nt < T::NT; ++nt) {
      if constexpr (KIND == kF32) {
        u32x4 va = vr[2 * nt], vc = vr[2 * nt + 1];
        if (tail) {
          va = zero_from<4>(va, lim);
          vc = zero_from<4>(vc, lim - 4);
        }
#pragma unroll
        for (int k = 0; k < NR; ++k) {
          f32x4 o = st[k].acc.o[nt];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            o = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(va[i]), pw[k][0][i], o, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            o = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(vc[i]), pw[k][1][i], o, 0, 0, 0);
          st[k].acc.o[nt] = o;
        }
      } else {
        VR v = vr[nt];
        if (tail) v = zero_from<T::ES>(v, lim);
        u32x4 vv;
        if constexpr (KIND == kBF16) {
          vv = v;
        } else {
          const u32x2 lo = bitcast<u32x2>(fp8x4_to_bf16x4(v[0]));
          const u32x2 hi = bitcast<u32x2>(fp8x4_to_bf16x4(v[1]));
          vv = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
#pragma unroll
        for (int k = 0; k < NR; ++k)
          st[k].acc.o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(vv), pw[k][0], st[k].acc.o[nt], 0, 0, 0);
      }
    }
    if constexpr (KIND != kF32) {  // the rounded weights' row sums, in the same unit
      const bf16x8 one8 = bitcast<bf16x8>(u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
#pragma unroll
      for (int k = 0; k < NR; ++k)
        st[k].lr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(one8, pw[k][0], st[k].lr, 0, 0, 0);
    }
  };

  if (n32 > 0) {
    // Software pipeline over steps.  Stage u issues the MFMAs of step u + 1's
    // scores, then takes step u's row max (its scores finished a stage ago,
    // so neither the max nor the branch on a bump waits for an MFMA), forms
    // its weights on the VALU while those MFMAs run, and issues its P.V.  Step j
    // lives in LDS buffer j mod (PD + 2); its copies start right after the
    // barrier of stage j - PD - 1, into the buffer of step j - PD - 2, whose
    // last reads (stage j - PD - 2) precede that barrier.  Before the barrier
    // of stage u each wave waits for its own copies of step u + 1; those of
    // the PD - 1 steps after it stay in flight.
    constexpr uint32_t SB = sizeof(PfStep<KIND, D>);
    const uint32_t lds0 = (uint32_t)(uintptr_t)kv;  // LDS byte address of buffer 0
    float x[NR][8];
    int id[NID];
    // Step 0's copies and Q's loads overlap; an explicit wait that the
    // compiler sees then retires both, so its own wait for Q (it does not
    // count the asm copies) cannot later hold the copies of steps 1..PD.
    ids_of(0, id);
    copy_step(0, id, lds0);
    load_q();
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt, lgkmcnt unchecked
#pragma unroll
    for (int j = 1; j <= PD; ++j) {
      ids_of(j, id);
      copy_step(j, id, lds0 + j * SB);
    }
    ids_of(PD + 1, id);
    vm_wait<PD * NCW>();
    __syncthreads();
    // Raw scores of the current step (sc[J % 2] in stage J) and of the next.
    f32x4 sc[2][NR][2];
    scores_of(kv[0], sc[0]);
    int u = 0;
#define PKV_PF_STAGE(J, MASK)                                                            \
  {                                                                                      \
    constexpr int NB = C_::NBUF;                                                         \
    constexpr int BC = (J) % NB, BN = ((J) + 1) % NB, BI = ((J) + PD + 1) % NB;          \
    vm_wait<(PD - 1) * NCW>();                                                           \
    __syncthreads();                                                                     \
    copy_step(u + PD + 1, id, lds0 + BI * SB);                                           \
    ids_of(u + PD + 2, id);                                                              \
    VR vr[NVR];                                                                          \
    read_v(kv[BC], vr);                                                                  \
    scores_of(kv[BN], sc[((J) + 1) % 2]);                                                \
    float mx[NR];                                                                        \
    bool bump[NR];                                                                       \
    const bool any = max_of(sc[(J) % 2], u, std::integral_constant<bool, MASK>(), x, mx);  \
    if (__builtin_amdgcn_ballot_w64(any)) {                                              \
      row_bumps(mx, bump);                                                               \
      rescale(mx, bump);                                                                 \
    }                                                                                    \
    PB pw[NR][NPB];                                                                      \
    weights_of(x, std::integral_constant<bool, MASK>(), pw);                             \
    pv_of(vr, pw, u, MASK && (u + 1) * 2 * kBS > Lmax);                                  \
    ++u;                                                                                 \
  }
    // Stage u may skip masking when every row sees step u in full.
    constexpr int U = C_::NBUF;  // stages per unrolled round
    static_assert(U == 4 && U % 2 == 0, "the stage loops below are written for 4 stages a round");
    const int u_plain = u_full / U * U;
    while (u < u_plain) {
      PKV_PF_STAGE(0, false)
      PKV_PF_STAGE(1, false)
      PKV_PF_STAGE(2, false)
      PKV_PF_STAGE(3, false)
    }
    while (u < n32) {
      PKV_PF_STAGE(0, true)
      if (u >= n32) break;
      PKV_PF_STAGE(1, true)
      if (u >= n32) break;
      PKV_PF_STAGE(2, true)
      if (u >= n32) break;
      PKV_PF_STAGE(3, true)
      if (u >= n32) break;
    }
#undef PKV_PF_STAGE
    // No copy may still be writing LDS when the workgroup ends.
    vm_wait<0>();
  }

  // a row's sum over its four lanes (l, l ^ 16, l ^ 32, l ^ 48)
  auto row_sum = [](float v) {
    uint32_t u = __float_as_uint(v);
    auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    v = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
    u = __float_as_uint(v);
    auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
  };
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    const float lsum = row_sum(st[k].l);
    const float lnorm = KIND == kF32 ? lsum : st[k].lr[0];
    if (!row_ok[k]) continue;
    const int j = jbase + k * NQ + jl;
    const bool empty = Ls - C + j + 1 <= 0;
    const int64_t row = (int64_t)(q0 + j) * Hq + g * G + hh;
    const float inv = !empty && lnorm > 0.f ? a.v_scale / lnorm : 0.f;
#pragma unroll
    for (int nt = 0; nt < T::NT; ++nt) {
      const int d = nt * 16 + 4 * q4;
      const f32x4 o = st[k].acc.o[nt] * inv;
      if constexpr (KIND == kF32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + row * D + d) = o;
      } else {
        const uint32_t lo = (uint32_t)f32_to_bf16_rne(o[0]) | ((uint32_t)f32_to_bf16_rne(o[1]) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16_rne(o[2]) | ((uint32_t)f32_to_bf16_rne(o[3]) << 16);
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + row * D + d) = u32x2{lo, hi};
      }
    }
    if (q4 == 0 && a.lse)
      a.lse[row] = !empty && lsum > 0.f ? (st[k].m + __builtin_amdgcn_logf(lsum)) * kLn2 : -INFINITY;
  }
}

// Items (g, s, item) lie head major: item g * TQ + ct[s] + i, ct = prefix
// sums of the sequences' item counts, built in LDS by every workgroup.
// Workgroup b takes item (b mod 8) * (nWG / 8) + b / 8, so one XCD works
// through consecutive items of the same sequences and shares their K/V tiles
// in its L2.
template <int KIND, int D, int SH>
__global__ __launch_bounds__((64 * PrefillCfg<KIND, D>::NWV)) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_kernel(PrefillArgs a) {
  constexpr int NR = PrefillCfg<KIND, D>::NR;
  __shared__ PfStep<KIND, D> kv[PrefillCfg<KIND, D>::NBUF];
  __shared__ int lct[kPrefillMaxSeqs + 1];
  constexpr int NWV = PrefillCfg<KIND, D>::NWV;
  __shared__ int wsums[NWV];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nseq = a.num_seqs, H = a.num_kv_heads;
  const int per = a.tokens_per_tile * NR * NWV;  // query tokens per item
  {
    const int tid = threadIdx.x;
    int carry = 0;
    for (int c0 = 0; c0 < nseq; c0 += 64 * NWV) {
      const int s = c0 + tid;
      int C = s < nseq ? a.query_start[s + 1] - a.query_start[s] : 0;
      C = C < 0 ? 0 : C;
      int tot;
      const int e = block_exclusive_scan<NWV>((C + per - 1) / per, wsums, &tot);
      if (s < nseq) lct[s] = carry + e;
      carry += tot;
    }
    if (tid == 0) lct[nseq] = carry;
    __syncthreads();
  }
  const int TQ = lct[nseq];
  const int groups = gridDim.x;
  const int64_t k = (int64_t)(blockIdx.x & 7) * (groups >> 3) + (blockIdx.x >> 3);
  if (k >= (int64_t)H * TQ) return;  // the whole workgroup
  const int g = (int)(k / TQ), rem = (int)(k % TQ);
  int lo = 0, hi = nseq;  // largest s with lct[s] <= rem
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (lct[mid] <= rem) lo = mid; else hi = mid;
  }
  prefill_item<KIND, D, SH>(a, kv, w, lo, g, rem - lct[lo]);
}

}  // namespace

namespace {
// One workgroup per item of NWV * NR query tiles; items <= rows / tokens per
// item + one partial item per sequence.
template <int C_, int D_, int SH_>
hipError_t launch_prefill_cfg(const PrefillArgs& a, int64_t num_rows, hipStream_t stream,
                              bool* supported) {
  using Cfg = PrefillCfg<C_, D_>;
  const int per = a.tokens_per_tile * Cfg::NR * Cfg::NWV;
  const int64_t items = (num_rows + per - 1) / per + a.num_seqs;
  int64_t groups = (int64_t)a.num_kv_heads * items;
  groups = (groups + 7) / 8 * 8;
  if (groups > INT32_MAX) {
    *supported = false;
    return hipSuccess;
  }
  hipLaunchKernelGGL((prefill_kernel<C_, D_, SH_>), dim3((unsigned)groups), dim3(64 * Cfg::NWV), 0,
                     stream, a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int cache, int D, int64_t num_rows,
                          hipStream_t stream, bool* supported) {
  *supported = true;
  if (a.num_seqs == 0 || num_rows == 0) return hipSuccess;
  // the kernel computes block offsets as 32-bit stride x 32-bit block id
  const int64_t es = cache == kF32 ? 4 : (cache == kBF16 ? 2 : 1);
  const int64_t block_stride = ((int64_t)a.num_kv_heads * kBS * D * es) << a.block_shift;
  if (block_stride > (int64_t)UINT32_MAX) {
    *supported = false;
    return hipSuccess;
  }
#define PKV_PF(C_, D_, SH_)                                                           \
  if (cache == C_ && D == D_ && a.block_shift == SH_)                                 \
    return launch_prefill_cfg<C_, D_, SH_>(a, num_rows, stream, supported);
  PKV_PF(kF32, 64, 0) PKV_PF(kF32, 128, 0) PKV_PF(kBF16, 64, 0) PKV_PF(kBF16, 128, 0)
  PKV_PF(kFP8, 64, 0) PKV_PF(kFP8, 128, 0) PKV_PF(kF32, 64, 1) PKV_PF(kF32, 128, 1)
  PKV_PF(kBF16, 64, 1) PKV_PF(kBF16, 128, 1) PKV_PF(kFP8, 64, 1) PKV_PF(kFP8, 128, 1)
#undef PKV_PF
  *supported = false;
  return hipSuccess;
}

}  // namespace pkv
