// Pass 2 of paged decode attention for CDNA4 (gfx950): the log-sum-exp merge
// of the partial states pass 1 leaves when a (sequence, kv head) pair is
// split over several ranges or split-KV partitions.  Split-KV is the reading
// of the pages' statement that attention over a long context may be computed
// in pieces ("vLLM PagedAttention: Memory Optimization & High-Throughput LLM
// Inference Tuning", §2); the merge is exact up to rounding order.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "decode_plan.h"
#include "device_common.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

// ---------------------------------------------------------------- pass 2
// The segments of the pair at blocks [ps, pe), the same cut points pass 1
// uses, grouped into items: without partition cuts an item is one range
// r_lo + i touching the pair, with them an item is one partition, split at the
// starts of the ranges inside it.  A piece starting at a range start belongs
// to the last range starting there (earlier ones are empty).  With folding
// (no partition cuts, every range non-empty) a piece starting at range r's
// start, r not first in its workgroup, was merged by pass 1 into range
// r - 1's piece and holds no state of its own.
struct PairSegs {
  int64_t ps, pe, total;
  int k0, pb, R, r_lo, items;
  bool all_nonempty;  // every range holds a block
  bool fold;
  __device__ __forceinline__ bool nonempty(int r) const {
    return all_nonempty || range_start(r + 1, total, R) > range_start(r, total, R);
  }
  // (r > r_lo) the piece starting at range r's start was folded
  __device__ __forceinline__ bool folded(int r) const { return r % kWavesPerGroup != 0; }
  template <typename F>
  __device__ __forceinline__ void item(int i, F&& f) const {
    if (pb == 0) {
      const int r = r_lo + i;
      if (i == 0 || (fold ? !folded(r) : nonempty(r))) f(k0 + r);
      return;
    }
    const int64_t a = ps + (int64_t)i * pb;
    const int64_t b = a + pb < pe ? a + pb : pe;
    const int ra = range_of(a, total, R), rb = range_of(b - 1, total, R);
    f(k0 + i + ra);
    for (int r = ra + 1; r <= rb; ++r)
      if (nonempty(r)) f(k0 + i + r);
  }
};

constexpr int kMergeThreads = 256;  // 4 waves per (sequence, query head)
constexpr int kMergeWaves = kMergeThreads / 64;
constexpr int kMergeList = 2048;     // segments listed in LDS; more take a slower walk

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) v = fmaxf(v, __shfl_xor(v, k));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int k = 1; k < kMergeWaves; ++k) m = fmaxf(m, red[k]);
  __syncthreads();
  return m;
}

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) v += __shfl_xor(v, k);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int k = 0; k < kMergeWaves; ++k) t += red[k];
  __syncthreads();
  return t;
}

// One workgroup of kMergeThreads per (sequence, query head).  A sequence of
// length 0 gets a zero row and lse = -inf; one finished in pass 1 (inside
// one range and one partition) is skipped; otherwise the partial states of
// its segments are merged: M = max m_p, Lambda = sum l_p 2^{m_p - M},
// out = sum 2^{m_p - M} o_p / Lambda, lse = (M + log2 sum e_p 2^{m_p - M}) ln 2
// (l_p sums the weights as multiplied into V, e_p the fp32 weights).
// The segments are listed in LDS with their factors 2^{m_p - M}; each wave
// then takes every fourth entry, four rows per load (lane = D/16 dims), and
// the four waves' sums are added in LDS.
// Lane `lane`'s V = D / 64 dims of partial row pr (fp32 or bf16 workspace).
template <int OUT, int D>
__device__ __forceinline__ void load_partial(const DecodeArgs& a, int64_t pr, int lane,
                                             float (&x)[D / 64]) {
  constexpr int V = D / 64;
  const int64_t at = pr * D + lane * V;
  if constexpr (OUT == kF32) {
    if constexpr (V == 2) {
      const float2 t = *reinterpret_cast<const float2*>(a.ws_o + at);
      x[0] = t.x;
      x[1] = t.y;
    } else {
      x[0] = a.ws_o[at];
    }
  } else {
    const uint16_t* w = reinterpret_cast<const uint16_t*>(a.ws_o);
    if constexpr (V == 2) {
      const uint32_t t = *reinterpret_cast<const uint32_t*>(w + at);
      x[0] = __uint_as_float(t << 16);
      x[1] = __uint_as_float(t & 0xFFFF0000u);
    } else {
      x[0] = __uint_as_float((uint32_t)w[at] << 16);
    }
  }
}

// Dims l16 * D/16 .. + D/16 of partial row (slot, hh): 16 bytes of a bf16 row
// (32 of an fp32 one) for D = 128, half that for D = 64.
template <int OUT, int D>
__device__ __forceinline__ void load_row16(const DecodeArgs& a, int64_t slot, int hh, int G,
                                           int l16, float (&x)[D / 16]) {
  constexpr int DPL = D / 16;
  const int64_t at = (slot * G + hh) * D + l16 * DPL;
  if constexpr (OUT == kF32) {
#pragma unroll
    for (int k = 0; k < DPL / 4; ++k) {
      const f32x4 t = *reinterpret_cast<const f32x4*>(a.ws_o + at + 4 * k);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[4 * k + i] = t[i];
    }
  } else {
    const uint16_t* w = reinterpret_cast<const uint16_t*>(a.ws_o) + at;
    if constexpr (DPL == 8) {
      const u32x4 t = *reinterpret_cast<const u32x4*>(w);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(t[i] << 16);
        x[2 * i + 1] = __uint_as_float(t[i] & 0xFFFF0000u);
      }
    } else {
      const u32x2 t = *reinterpret_cast<const u32x2*>(w);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        x[2 * i] = __uint_as_float(t[i] << 16);
        x[2 * i + 1] = __uint_as_float(t[i] & 0xFFFF0000u);
      }
    }
  }
}

template <int OUT, int D>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeArgs a) {
  constexpr int V = D / 64;
  __shared__ int lslot[kMergeList];
  __shared__ float lcoef[kMergeList];
  __shared__ float red[kMergeWaves];
  __shared__ int wsum[kMergeWaves];
  __shared__ float psum[kMergeWaves][D];
  const int row = blockIdx.x;  // s * Hq + h
  const int S = a.num_seqs, H = a.num_kv_heads, R = a.num_ranges, pb = a.part_blocks;
  const int s = row / a.num_q_heads, h = row % a.num_q_heads;
  const int G = a.group;
  const int g = h / G, hh = h % G;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const cptr<int32_t> cb = as_const(a.cum);
  const cptr<int32_t> cp = as_const(a.cum_parts);
  const int T = cb[S], PT = cp[S];
  const int nblk = cb[s + 1] - cb[s];
  if (nblk == 0) {
    if (tid < D) {
      if constexpr (OUT == kF32)
        static_cast<float*>(a.out)[(int64_t)row * D + tid] = 0.f;
      else
        static_cast<uint16_t*>(a.out)[(int64_t)row * D + tid] = 0;
    }
    if (tid == 0 && a.lse) a.lse[row] = -INFINITY;
    return;
  }
  PairSegs ps;
  ps.total = (int64_t)T * H;
  ps.ps = (int64_t)g * T + cb[s];
  ps.pe = ps.ps + nblk;
  ps.k0 = g * PT + cp[s];
  ps.pb = pb;
  ps.R = R;
  ps.r_lo = range_of(ps.ps, ps.total, R);
  const int r_hi = range_of(ps.pe - 1, ps.total, R);
  ps.all_nonempty = ps.total >= R;
  ps.fold = pb == 0 && ps.all_nonempty;
  // finished in pass 1
  if (ps.r_lo == r_hi && (pb == 0 || nblk <= pb)) return;
  if (ps.fold && ps.r_lo / kWavesPerGroup == r_hi / kWavesPerGroup) return;
  ps.items = pb > 0 ? (nblk + pb - 1) / pb : r_hi - ps.r_lo + 1;
  const float* wm = a.ws_m;
  int cnt = 0;
  float mx = -INFINITY;
  for (int i = tid; i < ps.items; i += kMergeThreads)
    ps.item(i, [&](int slot) {
      ++cnt;
      mx = fmaxf(mx, wm[(int64_t)slot * G + hh]);
    });
  const float M = block_max(mx, red);
  int n;
  int off = block_exclusive_scan<kMergeWaves>(cnt, wsum, &n);
  float lam = 0.f, ex = 0.f;
  float acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = 0.f;
  if (n <= kMergeList) {
    for (int i = tid; i < ps.items; i += kMergeThreads)
      ps.item(i, [&](int slot) {
        const int64_t pr = (int64_t)slot * G + hh;
        const float m = wm[pr];
        const float c = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M);
        const float cl = c * a.ws_l[pr];
        lam += cl;
        ex += c * a.ws_e[pr];
        lslot[off] = slot;
        lcoef[off] = OUT == kF32 ? c : cl;  // bf16 rows are normalised by l
        ++off;
      });
    __syncthreads();
    // Four rows per load instruction: lane group q = lane / 16 takes every
    // fourth of the wave's listed entries, each lane D/16 dims of the row;
    // four loads in flight per lane.  The groups' sums are then added across
    // lanes.
    constexpr int DPL = D / 16;
    const int q = lane >> 4, l16 = lane & 15;
    float a8[DPL];
#pragma unroll
    for (int v = 0; v < DPL; ++v) a8[v] = 0.f;
    for (int e0 = wv + q * kMergeWaves; e0 < n; e0 += 16 * kMergeWaves) {
      float x[4][DPL], c[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + 4 * u * kMergeWaves;
        c[u] = 0.f;
        if (e < n) {
          c[u] = lcoef[e];
          load_row16<OUT, D>(a, lslot[e], hh, G, l16, x[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (c[u] != 0.f)
#pragma unroll
          for (int v = 0; v < DPL; ++v) a8[v] += c[u] * x[u][v];
    }
#pragma unroll
    for (int v = 0; v < DPL; ++v) {
      a8[v] += __shfl_xor(a8[v], 16);
      a8[v] += __shfl_xor(a8[v], 32);
    }
    if (q == 0)
#pragma unroll
      for (int v = 0; v < DPL; ++v) psum[wv][l16 * DPL + v] = a8[v];
  } else {
    // Too many segments to list: each wave walks its share of the items.
    for (int i = tid; i < ps.items; i += kMergeThreads)
      ps.item(i, [&](int slot) {
        const int64_t pr = (int64_t)slot * G + hh;
        const float m = wm[pr];
        const float c = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M);
        lam += c * a.ws_l[pr];
        ex += c * a.ws_e[pr];
      });
    for (int i = wv; i < ps.items; i += kMergeWaves)
      ps.item(i, [&](int slot) {
        const int64_t pr = (int64_t)slot * G + hh;
        const float m = wm[pr];
        if (m == -INFINITY) return;
        const float c = __builtin_amdgcn_exp2f(m - M) * (OUT == kF32 ? 1.f : a.ws_l[pr]);
        float x[V];
        load_partial<OUT, D>(a, pr, lane, x);
#pragma unroll
        for (int v = 0; v < V; ++v) acc[v] += c * x[v];
      });
#pragma unroll
    for (int v = 0; v < V; ++v) psum[wv][lane * V + v] = acc[v];
  }
  const float Lam = block_sum(lam, red);
  const float Ex = block_sum(ex, red);
  __syncthreads();
  if (tid < D) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < kMergeWaves; ++k) t += psum[k][tid];
    const float val = !(Lam <= 0.f) ? t / Lam : 0.f;
    if constexpr (OUT == kF32)
      static_cast<float*>(a.out)[(int64_t)row * D + tid] = val;
    else
      static_cast<uint16_t*>(a.out)[(int64_t)row * D + tid] = f32_to_bf16_rne(val);
  }
  if (tid == 0 && a.lse) a.lse[row] = !(Ex <= 0.f) ? (M + __builtin_amdgcn_logf(Ex)) * kLn2 : -INFINITY;
}

// Without partition cuts, the segments of a (sequence, kv head) pair are
// its pieces in the ranges r_lo .. r_hi it touches, the piece of range r in
// slot k0 + r.  With folding, a piece starting at a range that is not first
// in its pass-1 workgroup was merged in pass 1 and holds nothing; without
// folding (some range is empty) only non-empty ranges own a piece.  So the
// slots follow from the range indices alone and no list is built: one wave
// per (sequence, query head) row, four rows per workgroup, reductions inside
// the wave and no barrier.  Each lane carries one piece's factors; the rows
// are then summed four at a time, lane = D/64 output dimensions.
constexpr int kMergeRowsPerGroup = 4;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) v = fmaxf(v, __shfl_xor(v, k));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) v += __shfl_xor(v, k);
  return v;
}

template <int OUT, int D>
__global__ __launch_bounds__(64 * kMergeRowsPerGroup) void decode_merge_rows_kernel(DecodeArgs a) {
  constexpr int V = D / 64;
  const int lane = threadIdx.x & 63;
  const int S = a.num_seqs, H = a.num_kv_heads, R = a.num_ranges, Hq = a.num_q_heads;
  const int row = blockIdx.x * kMergeRowsPerGroup + (int)(threadIdx.x >> 6);  // s * Hq + h
  if (row >= S * Hq) return;
  const int s = row / Hq, h = row % Hq;
  const int G = a.group;
  const int g = h / G, hh = h % G;
  const cptr<int32_t> cb = as_const(a.cum);
  const cptr<int32_t> cp = as_const(a.cum_parts);
  const int T = cb[S], PT = cp[S];
  const int c0 = cb[s];
  const int nblk = cb[s + 1] - c0;
  if (nblk == 0) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      if constexpr (OUT == kF32)
        static_cast<float*>(a.out)[(int64_t)row * D + lane * V + v] = 0.f;
      else
        static_cast<uint16_t*>(a.out)[(int64_t)row * D + lane * V + v] = 0;
    }
    if (lane == 0 && a.lse) a.lse[row] = -INFINITY;
    return;
  }
  const int64_t total = (int64_t)T * H;
  const int64_t ps = (int64_t)g * T + c0;
  const int r_lo = range_of(ps, total, R);
  const int r_hi = range_of(ps + nblk - 1, total, R);
  const bool fold = total >= R;
  // finished in pass 1
  if (fold ? r_lo / kWavesPerGroup == r_hi / kWavesPerGroup : r_lo == r_hi) return;
  const int k0 = g * PT + cp[s];
  auto owns = [&](int r) {
    return r == r_lo || (fold ? r % kWavesPerGroup == 0
                              : range_start(r + 1, total, R) > range_start(r, total, R));
  };
  const int nr = r_hi - r_lo + 1;
  // The lane's piece among the first 64 ranges keeps its m, l and e from this
  // pass (issued together), so the common case of a row with at most 64
  // pieces reads them once.
  float mx = -INFINITY, m0 = -INFINITY, l0 = 0.f, e0 = 0.f;
  for (int i = lane; i < nr; i += 64)
    if (owns(r_lo + i)) {
      const int64_t pr = (int64_t)(k0 + r_lo + i) * G + hh;
      const float m = a.ws_m[pr];
      if (i < 64) {
        m0 = m;
        l0 = a.ws_l[pr];
        e0 = a.ws_e[pr];
      }
      mx = fmaxf(mx, m);
    }
  const float M = wave_max(mx);
  float lam = 0.f, ex = 0.f;
  float acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = 0.f;
  for (int i0 = 0; i0 < nr; i0 += 64) {
    const int r = r_lo + i0 + lane;
    const bool mine = i0 + lane < nr && owns(r);
    const int slot = k0 + r;
    float coef = 0.f;
    if (mine) {
      float m = m0, l = l0, e = e0;
      if (i0 > 0) {
        const int64_t pr = (int64_t)slot * G + hh;
        m = a.ws_m[pr];
        l = a.ws_l[pr];
        e = a.ws_e[pr];
      }
      const float c = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M);
      const float cl = c * l;
      lam += cl;
      ex += c * e;
      coef = OUT == kF32 ? c : cl;  // bf16 rows are normalised by l
    }
    uint64_t left = __ballot(mine);
    while (left) {
      int js[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        js[u] = left ? __builtin_ctzll(left) : -1;
        left &= left - 1;
      }
      float x[4][V], cs[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (js[u] >= 0) {
          cs[u] = __shfl(coef, js[u]);
          load_partial<OUT, D>(a, (int64_t)__shfl(slot, js[u]) * G + hh, lane, x[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (js[u] >= 0)
#pragma unroll
          for (int v = 0; v < V; ++v) acc[v] += cs[u] != 0.f ? cs[u] * x[u][v] : 0.f;
    }
  }
  const float Lam = wave_sum(lam);
  const float Ex = wave_sum(ex);
  if constexpr (OUT == kF32) {
#pragma unroll
    for (int v = 0; v < V; ++v)
      static_cast<float*>(a.out)[(int64_t)row * D + lane * V + v] = !(Lam <= 0.f) ? acc[v] / Lam : 0.f;
  } else {
#pragma unroll
    for (int v = 0; v < V; ++v)
      static_cast<uint16_t*>(a.out)[(int64_t)row * D + lane * V + v] =
          f32_to_bf16_rne(!(Lam <= 0.f) ? acc[v] / Lam : 0.f);
  }
  if (lane == 0 && a.lse) a.lse[row] = !(Ex <= 0.f) ? (M + __builtin_amdgcn_logf(Ex)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_decode_merge(const DecodeArgs& a, int out, int D, hipStream_t stream,
                               bool* supported) {
  *supported = true;
  if (a.num_seqs == 0) return hipSuccess;
  const int64_t rows = (int64_t)a.num_seqs * a.num_q_heads;
  // Without partition cuts a row has few segments: one wave per row.  With
  // them (hundreds of partitions per row) four waves share a row.
  const bool by_rows = a.part_blocks == 0;
  dim3 grid(by_rows ? (rows + kMergeRowsPerGroup - 1) / kMergeRowsPerGroup : rows);
  dim3 block(by_rows ? 64 * kMergeRowsPerGroup : kMergeThreads);
#define PKV_P2(O_, D_)                                                                      \
  if (out == O_ && D == D_) {                                                               \
    if (by_rows)                                                                            \
      hipLaunchKernelGGL((decode_merge_rows_kernel<O_, D_>), grid, block, 0, stream, a);    \
    else                                                                                    \
      hipLaunchKernelGGL((decode_merge_kernel<O_, D_>), grid, block, 0, stream, a);         \
    return hipGetLastError();                                                               \
  }
  PKV_P2(kF32, 64) PKV_P2(kF32, 128) PKV_P2(kBF16, 64) PKV_P2(kBF16, 128)
#undef PKV_P2
  *supported = false;
  return hipSuccess;
}

}  // namespace pkv
