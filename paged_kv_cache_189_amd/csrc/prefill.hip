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
// One workgroup per (kv head g, sequence s, item of 4 * NR query tiles).  A
// query tile holds tokens_per_tile = 16 / G query tokens of the chunk, row
// r = token r / G, head r % G, so the G heads of a token share every K/V
// fragment as in decode; wave w owns NR consecutive query tiles.  Row r's
// token sits at position p = L - C + j of its sequence and sees tokens 0..p
// (causal); the workgroup walks the context up to its last row's position in
// 32-token steps (two 16-token K/V tiles).  Each wave loads a quarter of every
// step into registers PD steps ahead and publishes it to LDS (two buffers,
// one barrier per step); all four waves run their query tiles against it, so
// a K/V byte is fetched once per 4 * NR query tiles.  Rows past the chunk copy
// the wave's last row and are not written; rows with p < 0 (chunk longer than
// the context) are written as zeros.
//
// Per step a row tile costs 2 x (D / 32) score MFMAs and D / 16 P.V MFMAs of
// 16x16x32 (the two tiles' 4-token fragments of a lane form one 8-element
// operand, so P.V runs at the full bf16 rate), against about 40 VALU
// instructions of online softmax.  Steps every row of the item sees in full
// take a loop with no causal masking.
template <int KIND, int D>
struct PrefillCfg {
  using T = Tile<KIND, D>;
  static constexpr int NR = KIND == kF32 ? 1 : 2;  // query tiles per wave
  static constexpr int PD = 2;                      // 32-token steps in flight per wave
  static constexpr int NWV = 4;                     // waves per workgroup (4 or 8)
  static constexpr int HPW = 8 / NWV;               // 16-token tiles of a step each wave loads
  // Each wave loads NL pieces of W bytes per lane of each 16-token K tile and
  // as many of the V tile, so the four waves split a step evenly, unbranched.
  static constexpr int W = T::BYTES / 256 < 16 ? T::BYTES / 256 : 16;
  static constexpr int NL = T::BYTES / (256 * W);
  static constexpr int FPC = W / T::VB;  // V fragments per loaded piece
  static constexpr int PER_STEP = 2 * NL;  // pieces of K (and of V) per lane per step
  static_assert(NL >= 1 && FPC >= 1, "tile split");
};

template <int KIND, int D>
struct KVLds {  // one 16-token K/V tile in fragment order: [chunk][lane]
  u32x4 k[Tile<KIND, D>::NK][64];
  typename Tile<KIND, D>::V v[Tile<KIND, D>::NT][64];
};

// One 32-token step (tiles 2u and 2u + 1) in LDS.  K: per tile, fragment
// order.  V: the two tiles' fragments of a lane side by side, v[nt][lane] =
// {tile 2u, tile 2u + 1}, so one LDS read yields a P.V operand.
template <int KIND, int D>
struct PfStep {
  using T = Tile<KIND, D>;
  u32x4 k[2][T::NK][64];
  typename T::V v[T::NT][64][2];
};

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
// bump threshold m + kLazyMax, the fp32 sum of the weights, and O^T.
template <int KIND, int D>
struct PfState {
  float m, thr, l;
  Acc<KIND, D> acc;
};

template <int KIND, int D, int SH>
__device__ __forceinline__ void prefill_item(const PrefillArgs& a, PfStep<KIND, D>* kv, int w,
                                             int s, int g, int item) {
  using T = Tile<KIND, D>;
  using C_ = PrefillCfg<KIND, D>;
  using VT = typename T::V;
  using PT = typename VecOf<C_::W>::T;
  struct Parts {
    VT p[C_::FPC];
  };
  constexpr int NR = C_::NR, PD = C_::PD, NL = C_::NL, W = C_::W, FPC = C_::FPC;
  constexpr int shift = SH;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, q4 = lane >> 4;
  const int G = a.group, NQ = a.tokens_per_tile, Hq = a.num_q_heads;
  const cptr<int32_t> qst = as_const(a.query_start);
  const int q0 = qst[s], C = qst[s + 1] - q0;
  int Ls = as_const(a.context_lens)[s];
  Ls = Ls < 0 ? 0 : (Ls > a.max_context_len ? a.max_context_len : Ls);
  const int per_wave = NQ * NR;
  constexpr int NWV = C_::NWV, HPW = C_::HPW;
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
  const uint32_t qflip = !qneg ? 0u : (KIND == kF32 ? 0x80000000u : 0x80008000u);
  int L[NR];
  bool row_ok[NR];
  u32x4 q[NR][T::NQ];  // Q^T fragments, kept in registers for the whole item
  {
    constexpr int QES = KIND == kF32 ? 4 : 2;
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const int j = jbase + k * NQ + jl;
      row_ok[k] = r < NQ * G && j <= jlast;
      const int jj = row_ok[k] ? j : jfall;
      const int Lrow = Ls - C + jj + 1;
      L[k] = Lrow > 1 ? Lrow : 1;  // empty rows look at token 0, then write zeros
      const gchar_p qrow = (gchar_p) static_cast<const char*>(a.q) +
                           ((int64_t)(q0 + jj) * Hq + g * G + (r < NQ * G ? hh : 0)) * D * QES;
#pragma unroll
      for (int jq = 0; jq < T::NQ; ++jq) {
        int off;
        if constexpr (KIND == kFP8)
          off = ((jq >> 1) * 4 + q4) * 32 + (jq & 1) * 16;
        else
          off = (jq * 4 + q4) * 16;
        q[k][jq] = *reinterpret_cast<gptr<u32x4>>(qrow + off) ^ qflip;
      }
    }
  }

  // This lane's pieces of a 16-token tile: byte t of the tile in pool order
  // lies at row * (row bytes << shift) + (t mod row bytes) from the tile's
  // start (K rows are 16 tokens x 16 bytes, V rows 16 tokens of one dim).  K
  // pieces land in LDS at t (pool order is fragment order); a V piece holds
  // FPC 4-token fragments of dim d, stored to [d / 16][q4 * 16 + d % 16].
  uint32_t ksrc[NL], kdst[NL], vsrc[NL], vdst[NL];
  int vtok[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const uint32_t t = (uint32_t)(((i * 4 + (w & 3)) * 64 + lane) * W);
    ksrc[i] = ((t >> 8) << (8 + shift)) + (t & 255u);
    kdst[i] = t;
    constexpr uint32_t VR = 16u * T::ES;  // V row bytes of a tile
    const uint32_t d = t / VR, tk = (t % VR) / T::ES;
    vsrc[i] = d * (VR << shift) + t % VR;
    vdst[i] = ((d >> 4) * 64u + (tk >> 2) * 16u + (d & 15u)) * (2 * T::VB);
    vtok[i] = (int)tk;
  }

  const cptr<int32_t> tbl = as_const(a.block_tables) + (int64_t)s * a.max_blocks;
  const char* kbase = static_cast<const char*>(a.k_cache) + ((int64_t)g * T::BYTES << shift);
  const char* vbase = static_cast<const char*>(a.v_cache) + ((int64_t)g * T::BYTES << shift);
  const int64_t bstride = (int64_t)a.num_kv_heads * T::BYTES << shift;
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
#pragma unroll
    for (int nt = 0; nt < T::NT; ++nt) st[k].acc.o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // With 8 waves, waves 0-3 load the step's first tile and 4-7 its second.
  const int h0 = HPW == 2 ? 0 : w >> 2;
  PT sk[PD][HPW][NL], sv[PD][HPW][NL];
  auto load_slot = [&](PT (&dk)[HPW][NL], PT (&dv)[HPW][NL], int u) {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const int h = h0 + hh;
      int t16 = 2 * u + h;
      t16 = t16 < n16 - 1 ? t16 : n16 - 1;
      int p32 = __builtin_amdgcn_readfirstlane(tbl[t16 >> shift]);
      p32 = p32 < 0 ? 0 : (p32 > last_block ? last_block : p32);
      const int64_t phys = p32;
      const int half = t16 & ((1 << shift) - 1);
      const gchar_p kt = uniform_ptr(kbase + phys * bstride + half * (kBS * 16));
      const gchar_p vt = uniform_ptr(vbase + phys * bstride + half * (kBS * T::ES));
      // Default cache policy: every item of the sequence reads these tiles,
      // and the items of a (head, sequence) pair run side by side on one XCD.
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        dk[hh][i] = *reinterpret_cast<gptr<PT>>(kt + ksrc[i]);
        dv[hh][i] = *reinterpret_cast<gptr<PT>>(vt + vsrc[i]);
      }
    }
  };
  // Publish a step to LDS.  On the step holding the sequence end V elements
  // past Lmax are zeroed: their weights are 0 but the slots may hold NaN.
  auto store_slot = [&](const PT (&dk)[HPW][NL], const PT (&dv)[HPW][NL], PfStep<KIND, D>& dst,
                        int u, bool tail) {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const int h = h0 + hh;
      char* kb = reinterpret_cast<char*>(dst.k[h]);
      char* vb = reinterpret_cast<char*>(dst.v) + h * T::VB;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        *reinterpret_cast<PT*>(kb + kdst[i]) = dk[hh][i];
        PT v = dv[hh][i];
        if (tail) v = zero_from<T::ES>(v, Lmax - (u * 2 + h) * kBS - vtok[i]);
        const Parts pp = bitcast<Parts>(v);
#pragma unroll
        for (int f = 0; f < FPC; ++f)
          *reinterpret_cast<VT*>(vb + vdst[i] + f * 16 * (2 * T::VB)) = pp.p[f];
      }
    }
  };

  using PB = typename std::conditional<KIND == kF32, f32x4, bf16x8>::type;
  constexpr int NPB = KIND == kF32 ? 2 : 1;
  // S^T of a step for every row tile, from the step's K in LDS.
  auto scores_of = [&](const PfStep<KIND, D>& t, f32x4 (&sc)[NR][2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 kf[T::NK];
#pragma unroll
      for (int j = 0; j < T::NK; ++j) kf[j] = t.k[h][j][lane];
#pragma unroll
      for (int k = 0; k < NR; ++k) sc[k][h] = pf_scores<KIND, D>(kf, q[k]);
    }
  };
  // Raw scores of step u (past each row's causal bound -> -inf when MASK),
  // each lane's max of them, and whether some row's running max must move.
  // The scale (> 0: a negative one was moved into Q) is applied inside the
  // exponent, p = 2^(s * scale - m).
  auto max_of = [&](const f32x4 (&sc)[NR][2], int u, auto masked, float (&x)[NR][8],
                    float (&mx)[NR], bool (&bump)[NR], bool live) {
    constexpr bool MASK = decltype(masked)::value;
    bool any = false;
#pragma unroll
    for (int k = 0; k < NR; ++k) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = sc[k][h][i];
          if (MASK) v = u * 2 * kBS + h * kBS + 4 * q4 + i < L[k] ? v : -INFINITY;
          x[k][h * 4 + i] = v;
        }
      const float m01 = __builtin_amdgcn_fmed3f(x[k][0], x[k][1], pinf);
      const float m23 = __builtin_amdgcn_fmed3f(x[k][2], x[k][3], pinf);
      const float m45 = __builtin_amdgcn_fmed3f(x[k][4], x[k][5], pinf);
      const float m67 = __builtin_amdgcn_fmed3f(x[k][6], x[k][7], pinf);
      mx[k] = fmaxf(fmaxf(m01, m23), fmaxf(m45, m67));  // this lane's max; the row's below
      // always true on a row's first step; false for NaN
      any = any || (live && mx[k] * scl > st[k].thr);
    }
    return any;
  };
  // The row max across the 4 lanes of each row and which rows move their
  // running max: needed only when some lane's own max passed its row's
  // threshold (scl > 0 keeps the scaling monotone, so the row's scaled max
  // passes it exactly when one of its lanes' does).
  auto row_bumps = [&](float (&mx)[NR], bool (&bump)[NR], bool live) {
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      mx[k] = row_max(mx[k], pinf) * scl;
      bump[k] = live && mx[k] > st[k].thr;
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
      st[k].thr = m_new + kLazyMax;
      st[k].l *= alpha;
#pragma unroll
      for (int nt = 0; nt < T::NT; ++nt) st[k].acc.o[nt] *= alpha;
    }
  };
  // Weights of a step, summed into l (fp32) and packed as P.V operands.
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
  // O^T[d][row] += V^T . P^T over a step's 32 tokens.
  auto pv_of = [&](const PfStep<KIND, D>& t, const PB (&pw)[NR][NPB]) {
#pragma unroll
    for (int nt = 0; nt < T::NT; ++nt) {
      const VT va = t.v[nt][lane][0], vb = t.v[nt][lane][1];
      if constexpr (KIND == kF32) {
#pragma unroll
        for (int k = 0; k < NR; ++k) {
          f32x4 o = st[k].acc.o[nt];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            o = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(va[i]), pw[k][0][i], o, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            o = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(vb[i]), pw[k][1][i], o, 0, 0, 0);
          st[k].acc.o[nt] = o;
        }
      } else {
        u32x2 lo, hi;
        if constexpr (KIND == kBF16) {
          lo = va;
          hi = vb;
        } else {
          lo = bitcast<u32x2>(fp8x4_to_bf16x4(va));
          hi = bitcast<u32x2>(fp8x4_to_bf16x4(vb));
        }
        const bf16x8 vv = bitcast<bf16x8>(u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
        for (int k = 0; k < NR; ++k)
          st[k].acc.o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, pw[k][0], st[k].acc.o[nt], 0, 0, 0);
      }
    }
  };

  if (n32 > 0) {
    // Software pipeline over steps.  Stage u publishes step u + 1 and runs
    // the MFMAs of step u + 1's scores and step u's P.V while the VALU forms
    // step u's weights and step u + 1's row max, so matrix and vector work
    // of one wave overlap.  Step j lives in LDS buffer j mod 3: stage u reads
    // buffers u and u + 1 and writes u + 1, last read at stage u - 2 (before
    // the previous stage's barrier), so one barrier per stage suffices.
    // Register slot j mod PD holds step j from its load, issued PD stages
    // ahead, until it is published.
    float x[NR][8];
#pragma unroll
    for (int i = 0; i < PD; ++i) load_slot(sk[i], sv[i], i);
    store_slot(sk[0], sv[0], kv[0], 0, 2 * kBS > Lmax);
    __syncthreads();
    load_slot(sk[0], sv[0], PD);
    {
      f32x4 sc[NR][2];
      scores_of(kv[0], sc);
      float mx[NR];
      bool bump[NR];
      if (__builtin_amdgcn_ballot_w64(max_of(sc, 0, std::true_type(), x, mx, bump, true))) {
        row_bumps(mx, bump, true);
        rescale(mx, bump);
      }
    }
    int u = 0;
#define PKV_PF_STAGE(J, MASK)                                                            \
  {                                                                                      \
    constexpr int BC = (J) % 3, BN = ((J) + 1) % 3, SL = ((J) + 1) % PD;                 \
    const bool live = u + 1 < n32;                                                       \
    store_slot(sk[SL], sv[SL], kv[BN], u + 1, MASK && (u + 2) * 2 * kBS > Lmax);         \
    __syncthreads();                                                                     \
    load_slot(sk[SL], sv[SL], u + 1 + PD);                                               \
    f32x4 scn[NR][2];                                                                    \
    scores_of(kv[BN], scn);                                                              \
    PB pw[NR][NPB];                                                                      \
    weights_of(x, std::integral_constant<bool, MASK>(), pw);                             \
    pv_of(kv[BC], pw);                                                                   \
    float mx[NR];                                                                        \
    bool bump[NR];                                                                       \
    const bool any = max_of(scn, u + 1, std::integral_constant<bool, MASK>(), x, mx, bump, live); \
    if (__builtin_amdgcn_ballot_w64(any)) {                                              \
      row_bumps(mx, bump, live);                                                         \
      rescale(mx, bump);                                                                 \
    }                                                                                    \
    ++u;                                                                                 \
  }
    // Stage u may skip masking when steps u and u + 1 are seen in full.
    constexpr int U = PD % 3 == 0 ? PD : 3 * PD;  // stages per unrolled round
    const int u_plain = u_full >= 1 ? (u_full - 1) / U * U : 0;
    static_assert(U <= 6, "the stage loops below are written for 6 stages a round");
    while (u < u_plain) {
      PKV_PF_STAGE(0, false)
      PKV_PF_STAGE(1, false)
      PKV_PF_STAGE(2, false)
      if constexpr (U == 6) {
        PKV_PF_STAGE(3, false)
        PKV_PF_STAGE(4, false)
        PKV_PF_STAGE(5, false)
      }
    }
    for (;;) {
      PKV_PF_STAGE(0, true)
      if (u >= n32) break;
      PKV_PF_STAGE(1, true)
      if (u >= n32) break;
      PKV_PF_STAGE(2, true)
      if (u >= n32) break;
      if constexpr (U == 6) {
        PKV_PF_STAGE(3, true)
        if (u >= n32) break;
        PKV_PF_STAGE(4, true)
        if (u >= n32) break;
        PKV_PF_STAGE(5, true)
        if (u >= n32) break;
      }
    }
#undef PKV_PF_STAGE
  }

#pragma unroll
  for (int k = 0; k < NR; ++k) {
    uint32_t lu = __float_as_uint(st[k].l);
    auto s16 = __builtin_amdgcn_permlane16_swap(lu, lu, false, false);
    float lsum = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
    lu = __float_as_uint(lsum);
    auto s32 = __builtin_amdgcn_permlane32_swap(lu, lu, false, false);
    lsum = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
    if (!row_ok[k]) continue;
    const int j = jbase + k * NQ + jl;
    const bool empty = Ls - C + j + 1 <= 0;
    const int64_t row = (int64_t)(q0 + j) * Hq + g * G + hh;
    const float inv = !empty && lsum > 0.f ? a.v_scale / lsum : 0.f;
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
  __shared__ PfStep<KIND, D> kv[3];
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

hipError_t launch_prefill(const PrefillArgs& a, int cache, int D, int64_t num_rows,
                          hipStream_t stream, bool* supported) {
  *supported = true;
  if (a.num_seqs == 0 || num_rows == 0) return hipSuccess;
  // one workgroup per item of 4 * NR query tiles; items <= rows / tokens per
  // item + one partial item per sequence
  const int nr = cache == kF32 ? PrefillCfg<kF32, 128>::NR : PrefillCfg<kBF16, 128>::NR;
  const int per = a.tokens_per_tile * nr * PrefillCfg<kBF16, 128>::NWV;
  const int64_t items = (num_rows + per - 1) / per + a.num_seqs;
  int64_t groups = (int64_t)a.num_kv_heads * items;
  groups = (groups + 7) / 8 * 8;
  if (groups > INT32_MAX) {
    *supported = false;
    return hipSuccess;
  }
  const dim3 grid((unsigned)groups), block(64 * PrefillCfg<kBF16, 128>::NWV);
#define PKV_PF(C_, D_, SH_)                                                           \
  if (cache == C_ && D == D_ && a.block_shift == SH_) {                               \
    hipLaunchKernelGGL((prefill_kernel<C_, D_, SH_>), grid, block, 0, stream, a);     \
    return hipGetLastError();                                                         \
  }
  PKV_PF(kF32, 64, 0) PKV_PF(kF32, 128, 0) PKV_PF(kBF16, 64, 0) PKV_PF(kBF16, 128, 0)
  PKV_PF(kFP8, 64, 0) PKV_PF(kFP8, 128, 0) PKV_PF(kF32, 64, 1) PKV_PF(kF32, 128, 1)
  PKV_PF(kBF16, 64, 1) PKV_PF(kBF16, 128, 1) PKV_PF(kFP8, 64, 1) PKV_PF(kFP8, 128, 1)
#undef PKV_PF
  *supported = false;
  return hipSuccess;
}

}  // namespace pkv
