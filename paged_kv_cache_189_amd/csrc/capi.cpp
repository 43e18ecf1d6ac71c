// C ABI of libpkv: argument validation, kernel dispatch, workspace sizing and
// error reporting for the device operations declared in include/pkv.h.
// Every check runs on the host before anything is enqueued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>
#include <string>

#include "../../include/pkv.h"
#include "pkv_internal.h"
#include "pkv_launch.h"

namespace {

thread_local std::string g_last_error;

constexpr int32_t kTile = 16;  // tokens per pass-1 tile; blocks hold 1 or 2 tiles
bool block_size_ok(int32_t bs) { return bs == 16 || bs == 32; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int elem_bytes(int32_t dt) {
  return dt == PKV_F32 ? 4 : dt == PKV_BF16 ? 2 : dt == PKV_FP8_E4M3 ? 1 : 0;
}

struct Layout {
  int32_t part_blocks = 0;   // partition cut every part_blocks blocks (0: none)
  int64_t max_segments = 0;  // bound on pass-1 segment slots
  size_t o_off = 0, m_off = 0, l_off = 0, e_off = 0;
  size_t cum_off = 0, parts_off = 0, rpair_off = 0, bytes = 0;
};

// Workspace: the partial states of at most max_segments segment slots (rows
// of D elements: fp32 for fp32 outputs, bf16 otherwise; m, l, e in fp32),
// then the plan arrays.  Slots are below (partitions of all pairs) + ranges;
// a pair has at most ceil(blocks / part_blocks) partitions (1 without
// partition cuts).  `ranges` bounds the pass-1 range count: kMaxRanges for a
// caller's workspace, whose size must not depend on the device; the
// device's own count where the library sizes the memory itself.
Layout layout_of(const pkv_decode_params& p, int64_t ranges = pkv::kMaxRanges) {
  Layout L;
  L.part_blocks = p.partition_size > 0 ? p.partition_size / kTile : 0;
  const int64_t max_blocks = ((int64_t)(p.max_context_len > 0 ? p.max_context_len : 0) + kTile - 1) / kTile;
  const int64_t pieces = L.part_blocks > 0 ? (max_blocks + L.part_blocks - 1) / L.part_blocks : 1;
  const int64_t pairs = (int64_t)p.num_seqs * p.num_kv_heads;
  const int64_t group = p.num_kv_heads > 0 ? p.num_q_heads / p.num_kv_heads : 1;
  L.max_segments = pairs * (pieces > 1 ? pieces : 1) + ranges;
  const size_t rows = (size_t)L.max_segments * (size_t)group;
  const size_t o_elem = p.out_dtype == PKV_F32 ? 4 : 2;
  L.o_off = 0;
  L.m_off = round_up(rows * (size_t)p.head_dim * o_elem, 256);
  L.l_off = L.m_off + round_up(rows * sizeof(float), 256);
  L.e_off = L.l_off + round_up(rows * sizeof(float), 256);
  L.cum_off = L.e_off + round_up(rows * sizeof(float), 256);
  L.parts_off = L.cum_off + round_up(((size_t)p.num_seqs + 1) * sizeof(int32_t), 256);
  L.rpair_off = L.parts_off + round_up(((size_t)p.num_seqs + 1) * sizeof(int32_t), 256);
  L.bytes = L.rpair_off + round_up((size_t)ranges * sizeof(int32_t), 256);
  return L;
}

pkv_status check_decode(const pkv_decode_params* p) {
  if (!p) return pkv_fail(PKV_ERR_INVALID_ARG, "decode: params is NULL");
  if (p->num_seqs < 0) return pkv_fail(PKV_ERR_INVALID_ARG, "decode: num_seqs < 0");
  if (p->num_q_heads <= 0 || p->num_kv_heads <= 0 || p->num_q_heads % p->num_kv_heads)
    return pkv_fail(PKV_ERR_INVALID_ARG, "decode: num_q_heads must be a positive multiple of num_kv_heads");
  const int32_t G = p->num_q_heads / p->num_kv_heads;
  if (G > 16) return pkv_fail(PKV_ERR_UNSUPPORTED, "decode: query heads per kv head must be <= 16");
  if (p->head_dim != 64 && p->head_dim != 128)
    return pkv_fail(PKV_ERR_UNSUPPORTED, "decode: head_dim must be 64 or 128");
  if (!block_size_ok(p->block_size)) return pkv_fail(PKV_ERR_UNSUPPORTED, "decode: block_size must be 16 or 32");
  if (p->max_blocks_per_seq <= 0) return pkv_fail(PKV_ERR_INVALID_ARG, "decode: max_blocks_per_seq must be > 0");
  if (p->max_context_len < 0 || (int64_t)p->max_context_len > (int64_t)p->max_blocks_per_seq * p->block_size)
    return pkv_fail(PKV_ERR_INVALID_ARG, "decode: max_context_len must be in [0, max_blocks_per_seq * block_size]");
  if (p->partition_size < 0 || p->partition_size % p->block_size)
    return pkv_fail(PKV_ERR_INVALID_ARG, "decode: partition_size must be 0 or a positive multiple of block_size");
  if (p->num_blocks <= 0) return pkv_fail(PKV_ERR_INVALID_ARG, "decode: num_blocks must be > 0");
  if (!std::isfinite(p->scale) || !std::isfinite(p->k_scale) || !std::isfinite(p->v_scale) || p->k_scale <= 0.f ||
      p->v_scale <= 0.f)
    return pkv_fail(PKV_ERR_INVALID_ARG, "decode: scale must be finite, k_scale and v_scale finite and > 0");
  const bool combo = (p->q_dtype == PKV_F32 && p->cache_dtype == PKV_F32 && p->out_dtype == PKV_F32) ||
                     (p->q_dtype == PKV_BF16 && p->cache_dtype == PKV_BF16 && p->out_dtype == PKV_BF16) ||
                     (p->q_dtype == PKV_BF16 && p->cache_dtype == PKV_FP8_E4M3 && p->out_dtype == PKV_BF16);
  if (!combo)
    return pkv_fail(PKV_ERR_UNSUPPORTED,
                    "decode: (q, cache, out) dtypes must be (f32,f32,f32), (bf16,bf16,bf16) or (bf16,fp8,bf16)");
  const Layout L = layout_of(*p);
  const int64_t max_blocks = ((int64_t)p->max_context_len + kTile - 1) / kTile;
  if ((int64_t)p->num_seqs * p->num_q_heads > INT32_MAX || L.max_segments * 3 > INT32_MAX ||
      (int64_t)p->num_seqs * max_blocks * p->num_kv_heads > INT32_MAX)
    return pkv_fail(PKV_ERR_UNSUPPORTED, "decode: sequences * heads * blocks too large");
  return PKV_OK;
}

pkv_status check_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return PKV_OK;
  return pkv_fail(PKV_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// ---------------------------------------------------------------- scratch
// Device memory of the allocation-free decode call: a file-scope device
// array, one copy per GPU, held until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is a stand-in, not a
// device address): the address comes from hipGetSymbolAddress, looked up
// once per device with that device current, and kept per device.
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // per device; null until the first call there

// The scratch array's address on the current device (looked up on the
// first call there).
pkv_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return check_hip(e, "decode_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return pkv_fail(PKV_ERR_UNSUPPORTED, "decode_noalloc: device index >= 64");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return check_hip(e, "decode_noalloc: hipGetSymbolAddress(scratch)");
    if (ptr == nullptr) return pkv_fail(PKV_ERR_HIP, "decode_noalloc: no device address for the scratch array");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

// Validates the call and fills the kernel arguments.  The partial states and
// the plan live in the caller's workspace, or (own_scratch) in the library's
// scratch array of the current device, laid out for that device's range
// count.
pkv_status build_args(const pkv_decode_params* p, void* out, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                      const void* workspace, size_t workspace_bytes, float* lse_out, bool need_q_cache,
                      bool own_scratch, pkv::DecodeArgs* a) {
  pkv_status st = check_decode(p);
  if (st != PKV_OK) return st;
  Layout L = layout_of(*p);
  if (p->num_seqs > 0) {
    if (!out || !context_lens) return pkv_fail(PKV_ERR_INVALID_ARG, "decode: out and context_lens are required");
    if (need_q_cache && (!q || !k_cache || !v_cache || !block_tables))
      return pkv_fail(PKV_ERR_INVALID_ARG, "decode: q, k_cache, v_cache and block_tables are required");
    if (!aligned(out, (uintptr_t)elem_bytes(p->out_dtype)) || !aligned(context_lens, 4) ||
        (need_q_cache && (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
                          !aligned(block_tables, 4))) ||
        (lse_out && !aligned(lse_out, 4)))
      return pkv_fail(PKV_ERR_INVALID_ARG, "decode: q and the caches must be 16-byte aligned, other arrays element aligned");
    if (!own_scratch) {
      if (!workspace || workspace_bytes < L.bytes)
        return pkv_fail(PKV_ERR_INVALID_ARG, "decode: workspace missing or smaller than pkv_decode_workspace_bytes()");
      if (!aligned(workspace, 256)) return pkv_fail(PKV_ERR_INVALID_ARG, "decode: workspace must be 256-byte aligned");
    }
  }
  pkv::DecodeArgs& d = *a;
  d.num_ranges = 0;
  d.block_shift = p->block_size == 32 ? 1 : 0;
  // ranges of pass 1 (one per resident wave); pass 2 derives the same slots
  if (p->num_seqs > 0) {
    hipError_t e = hipSuccess;
    d.num_ranges = pkv::decode_ranges(p->cache_dtype, p->head_dim, p->num_seqs, d.block_shift,
                                      (int64_t)p->num_seqs * p->num_kv_heads * ((int64_t)p->max_context_len + kTile - 1) / kTile,
                                      &e);
    if (e != hipSuccess) return check_hip(e, "decode: querying the device");
  }
  if (own_scratch && p->num_seqs > 0) {
    L = layout_of(*p, d.num_ranges);
    if (L.bytes > (size_t)PKV_NOALLOC_SCRATCH_BYTES)
      return pkv_fail(PKV_ERR_UNSUPPORTED,
                      "decode_noalloc: these params need " + std::to_string(L.bytes) +
                          " bytes of partial states and plan; the library's scratch holds " +
                          std::to_string((size_t)PKV_NOALLOC_SCRATCH_BYTES) + " per device");
    void* ptr = nullptr;
    st = scratch_of_current_device(&ptr);
    if (st != PKV_OK) return st;
    workspace = ptr;
  }
  d.out = out;
  d.q = q;
  d.k_cache = k_cache;
  d.v_cache = v_cache;
  d.block_tables = block_tables;
  d.context_lens = context_lens;
  char* ws = static_cast<char*>(const_cast<void*>(workspace));
  d.ws_o = reinterpret_cast<float*>(ws + L.o_off);
  d.ws_m = reinterpret_cast<float*>(ws + L.m_off);
  d.ws_l = reinterpret_cast<float*>(ws + L.l_off);
  d.ws_e = reinterpret_cast<float*>(ws + L.e_off);
  d.cum = reinterpret_cast<int32_t*>(ws + L.cum_off);
  d.cum_parts = reinterpret_cast<int32_t*>(ws + L.parts_off);
  d.range_pair = reinterpret_cast<int32_t*>(ws + L.rpair_off);
  d.lse = lse_out;
  d.num_blocks = p->num_blocks;
  d.num_seqs = p->num_seqs;
  d.num_q_heads = p->num_q_heads;
  d.num_kv_heads = p->num_kv_heads;
  d.group = p->num_q_heads / p->num_kv_heads;
  d.max_blocks = p->max_blocks_per_seq;
  d.max_context_len = p->max_context_len;
  d.part_blocks = L.part_blocks;
  d.score_scale_log2 = (float)((double)p->scale * (double)p->k_scale * 1.4426950408889634);
  d.v_scale = p->v_scale;
  return PKV_OK;
}

}  // namespace

pkv_status pkv_fail(pkv_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

extern "C" {

const char* pkv_status_string(pkv_status s) {
  switch (s) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_OUT_OF_BLOCKS: return "out of blocks (KV cache full)";
    case PKV_ERR_UNKNOWN_SEQ: return "unknown sequence";
    case PKV_ERR_SEQ_EXISTS: return "sequence exists";
    case PKV_ERR_SHARED_TAIL: return "append into a shared, partially filled block";
    case PKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKV_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* pkv_last_error(void) { return g_last_error.c_str(); }

const char* pkv_version(void) { return "pkv 0.1 (gfx950)"; }

// Shared checks and launch of the cache write; tables / lens / max_blocks
// only for the decode append.
static pkv_status cache_write(const char* what, const void* k_new, const void* v_new,
                              pkv_dtype src_dtype, void* k_cache, void* v_cache,
                              pkv_dtype cache_dtype, const int64_t* slot_mapping,
                              const int32_t* context_lens, int32_t* block_tables,
                              int32_t max_blocks, int32_t num_tokens, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int64_t num_blocks,
                              float k_scale, float v_scale, void* stream) {
  auto fail = [&](pkv_status st, const char* why) { return pkv_fail(st, std::string(what) + ": " + why); };
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0) return fail(PKV_ERR_INVALID_ARG, "bad sizes");
  if (head_dim != 64 && head_dim != 128) return fail(PKV_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (!block_size_ok(block_size)) return fail(PKV_ERR_UNSUPPORTED, "block_size must be 16 or 32");
  const bool combo = (src_dtype == PKV_F32 && (cache_dtype == PKV_F32 || cache_dtype == PKV_BF16 ||
                                               cache_dtype == PKV_FP8_E4M3)) ||
                     (src_dtype == PKV_BF16 && (cache_dtype == PKV_BF16 || cache_dtype == PKV_FP8_E4M3));
  if (!combo) return fail(PKV_ERR_UNSUPPORTED, "unsupported (src, cache) dtypes");
  if (cache_dtype == PKV_FP8_E4M3 &&
      (!std::isfinite(k_scale) || !std::isfinite(v_scale) || k_scale <= 0.f || v_scale <= 0.f))
    return fail(PKV_ERR_INVALID_ARG, "fp8 scales must be finite and > 0");
  if (block_tables != nullptr && max_blocks <= 0) return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq must be > 0");
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping) return fail(PKV_ERR_INVALID_ARG, "NULL pointer");
  if (block_tables != nullptr && context_lens == nullptr) return fail(PKV_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(slot_mapping, 8) || !aligned(block_tables, 4) || !aligned(context_lens, 4))
    return fail(PKV_ERR_INVALID_ARG, "K/V arrays must be 16-byte aligned, slots 8, tables and lengths 4");
  pkv::CacheWriteArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.slot_mapping = slot_mapping;
  a.context_lens = context_lens;
  a.block_tables = block_tables;
  a.num_blocks = num_blocks;
  a.num_tokens = num_tokens;
  a.num_kv_heads = num_kv_heads;
  a.block_size = block_size;
  a.max_blocks = max_blocks;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  bool ok = false;
  hipError_t e = pkv::launch_cache_write(a, src_dtype, cache_dtype, head_dim, (hipStream_t)stream, &ok);
  if (!ok) return fail(PKV_ERR_UNSUPPORTED, "no kernel variant");
  return check_hip(e, (std::string(what) + " launch").c_str());
}

pkv_status pkv_reshape_and_cache(const void* k_new, const void* v_new, pkv_dtype src_dtype, void* k_cache,
                                 void* v_cache, pkv_dtype cache_dtype, const int64_t* slot_mapping,
                                 int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int64_t num_blocks, float k_scale, float v_scale, void* stream) {
  return cache_write("reshape_and_cache", k_new, v_new, src_dtype, k_cache, v_cache, cache_dtype,
                     slot_mapping, nullptr, nullptr, 0, num_tokens, num_kv_heads, head_dim,
                     block_size, num_blocks, k_scale, v_scale, stream);
}

pkv_status pkv_append_decode_tokens(const void* k_new, const void* v_new, pkv_dtype src_dtype,
                                    void* k_cache, void* v_cache, pkv_dtype cache_dtype,
                                    const int64_t* slot_mapping, const int32_t* context_lens,
                                    int32_t* block_tables, int32_t max_blocks_per_seq,
                                    int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int64_t num_blocks, float k_scale,
                                    float v_scale, void* stream) {
  if (num_seqs > 0 && (block_tables == nullptr || context_lens == nullptr))
    return pkv_fail(PKV_ERR_INVALID_ARG, "append_decode_tokens: NULL pointer");
  return cache_write("append_decode_tokens", k_new, v_new, src_dtype, k_cache, v_cache, cache_dtype,
                     slot_mapping, context_lens, block_tables, max_blocks_per_seq, num_seqs,
                     num_kv_heads, head_dim, block_size, num_blocks, k_scale, v_scale, stream);
}

pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, pkv_dtype cache_dtype, const int32_t* src,
                           const int32_t* dst, int32_t n, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int64_t num_blocks, void* stream) {
  if (n < 0 || num_kv_heads <= 0 || num_blocks <= 0)
    return pkv_fail(PKV_ERR_INVALID_ARG, "copy_blocks: bad sizes");
  if (head_dim != 64 && head_dim != 128)
    return pkv_fail(PKV_ERR_UNSUPPORTED, "copy_blocks: head_dim must be 64 or 128");
  if (!block_size_ok(block_size)) return pkv_fail(PKV_ERR_UNSUPPORTED, "copy_blocks: block_size must be 16 or 32");
  const int es = elem_bytes(cache_dtype);
  if (es == 0) return pkv_fail(PKV_ERR_INVALID_ARG, "copy_blocks: unknown cache dtype");
  if (n == 0) return PKV_OK;
  if (!k_cache || !v_cache || !src || !dst) return pkv_fail(PKV_ERR_INVALID_ARG, "copy_blocks: NULL pointer");
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(src, 4) || !aligned(dst, 4))
    return pkv_fail(PKV_ERR_INVALID_ARG, "copy_blocks: misaligned pointer");
  pkv::CopyBlocksArgs a;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.src = src;
  a.dst = dst;
  a.num_blocks = num_blocks;
  a.block_bytes = (int64_t)num_kv_heads * head_dim * block_size * es;
  a.n = n;
  return check_hip(pkv::launch_copy_blocks(a, (hipStream_t)stream), "copy_blocks launch");
}

size_t pkv_decode_workspace_bytes(const pkv_decode_params* p) {
  if (check_decode(p) != PKV_OK) return 0;
  return layout_of(*p).bytes;
}

int32_t pkv_decode_partition_size(const pkv_decode_params* p) {
  if (check_decode(p) != PKV_OK) return -1;
  return layout_of(*p).part_blocks * kTile;
}

int32_t pkv_decode_num_ranges(const pkv_decode_params* p) {
  if (check_decode(p) != PKV_OK) return -1;
  if (p->num_seqs == 0) return 0;
  hipError_t e = hipSuccess;
  const int r = pkv::decode_ranges(p->cache_dtype, p->head_dim, p->num_seqs, p->block_size == 32 ? 1 : 0,
                                   (int64_t)p->num_seqs * p->num_kv_heads * ((int64_t)p->max_context_len + kTile - 1) / kTile,
                                   &e);
  if (e != hipSuccess) {
    check_hip(e, "decode_num_ranges: querying the device");
    return -1;
  }
  return r;
}

pkv_status pkv_prefill_attention(const pkv_prefill_params* p, void* out, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                                 const int32_t* query_start, float* lse_out, void* stream) {
  if (!p) return pkv_fail(PKV_ERR_INVALID_ARG, "prefill: params is NULL");
  // the shared checks of the decode parameters, then the prefill ones
  pkv_decode_params d{};
  d.num_seqs = p->num_seqs;
  d.num_q_heads = p->num_q_heads;
  d.num_kv_heads = p->num_kv_heads;
  d.head_dim = p->head_dim;
  d.block_size = p->block_size;
  d.max_blocks_per_seq = p->max_blocks_per_seq;
  d.max_context_len = p->max_context_len;
  d.partition_size = 0;
  d.num_blocks = p->num_blocks;
  d.scale = p->scale;
  d.k_scale = p->k_scale;
  d.v_scale = p->v_scale;
  d.q_dtype = p->q_dtype;
  d.cache_dtype = p->cache_dtype;
  d.out_dtype = p->out_dtype;
  pkv_status st = check_decode(&d);
  if (st != PKV_OK) return st;
  if (p->num_query_tokens < 0) return pkv_fail(PKV_ERR_INVALID_ARG, "prefill: num_query_tokens < 0");
  if (p->num_seqs > pkv::kPrefillMaxSeqs)
    return pkv_fail(PKV_ERR_UNSUPPORTED, "prefill: at most 1024 sequences per call");
  if ((int64_t)p->num_query_tokens * p->num_q_heads > INT32_MAX)
    return pkv_fail(PKV_ERR_UNSUPPORTED, "prefill: query tokens * heads too large");
  if (p->num_seqs == 0 || p->num_query_tokens == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
    return pkv_fail(PKV_ERR_INVALID_ARG, "prefill: NULL pointer");
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(query_start, 4) ||
      (lse_out && !aligned(lse_out, 4)))
    return pkv_fail(PKV_ERR_INVALID_ARG, "prefill: misaligned pointer");
  pkv::PrefillArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.lse = lse_out;
  a.num_blocks = p->num_blocks;
  a.num_seqs = p->num_seqs;
  a.num_q_heads = p->num_q_heads;
  a.num_kv_heads = p->num_kv_heads;
  a.group = p->num_q_heads / p->num_kv_heads;
  a.max_blocks = p->max_blocks_per_seq;
  a.max_context_len = p->max_context_len;
  a.tokens_per_tile = 16 / a.group;
  a.block_shift = p->block_size == 32 ? 1 : 0;
  a.score_scale_log2 = (float)((double)p->scale * (double)p->k_scale * 1.4426950408889634);
  a.v_scale = p->v_scale;
  bool ok = false;
  hipError_t e = pkv::launch_prefill(a, p->cache_dtype, p->head_dim, p->num_query_tokens, (hipStream_t)stream, &ok);
  if (!ok)
    return pkv_fail(PKV_ERR_UNSUPPORTED,
                    "prefill: no kernel for this shape (dtype / head_dim / block_size, more than 2^31 "
                    "workgroups, or a physical block of all kv heads of 4 GiB or more)");
  return check_hip(e, "prefill launch");
}

pkv_status pkv_decode_attention_partitions(const pkv_decode_params* p, void* out, const void* q, const void* k_cache,
                                           const void* v_cache, const int32_t* block_tables,
                                           const int32_t* context_lens, void* workspace, size_t workspace_bytes,
                                           float* lse_out, void* stream) {
  pkv::DecodeArgs a;
  pkv_status st = build_args(p, out, q, k_cache, v_cache, block_tables, context_lens, workspace, workspace_bytes,
                             lse_out, true, false, &a);
  if (st != PKV_OK) return st;
  bool ok = false;
  hipError_t e = pkv::launch_decode_partitions(a, p->cache_dtype, p->head_dim, (hipStream_t)stream, &ok);
  if (!ok) return pkv_fail(PKV_ERR_UNSUPPORTED, "decode: no kernel variant");
  return check_hip(e, "decode partitions launch");
}

pkv_status pkv_decode_attention_merge(const pkv_decode_params* p, void* out, const int32_t* context_lens,
                                      const void* workspace, size_t workspace_bytes, float* lse_out, void* stream) {
  pkv::DecodeArgs a;
  pkv_status st = build_args(p, out, nullptr, nullptr, nullptr, nullptr, context_lens, workspace, workspace_bytes,
                             lse_out, false, false, &a);
  if (st != PKV_OK) return st;
  bool ok = false;
  hipError_t e = pkv::launch_decode_merge(a, p->out_dtype, p->head_dim, (hipStream_t)stream, &ok);
  if (!ok) return pkv_fail(PKV_ERR_UNSUPPORTED, "decode: no merge kernel variant");
  return check_hip(e, "decode merge launch");
}

pkv_status pkv_decode_attention(const pkv_decode_params* p, void* out, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                                void* workspace, size_t workspace_bytes, float* lse_out, void* stream) {
  pkv::DecodeArgs a;
  pkv_status st = build_args(p, out, q, k_cache, v_cache, block_tables, context_lens, workspace, workspace_bytes,
                             lse_out, true, false, &a);
  if (st != PKV_OK) return st;
  bool ok = false;
  hipError_t e = pkv::launch_decode_partitions(a, p->cache_dtype, p->head_dim, (hipStream_t)stream, &ok);
  if (!ok) return pkv_fail(PKV_ERR_UNSUPPORTED, "decode: no kernel variant");
  st = check_hip(e, "decode partitions launch");
  if (st != PKV_OK) return st;
  e = pkv::launch_decode_merge(a, p->out_dtype, p->head_dim, (hipStream_t)stream, &ok);
  if (!ok) return pkv_fail(PKV_ERR_UNSUPPORTED, "decode: no merge kernel variant");
  return check_hip(e, "decode merge launch");
}

pkv_status pkv_decode_attention_noalloc(const pkv_decode_params* p, void* out, const void* q,
                                        const void* k_cache, const void* v_cache,
                                        const int32_t* block_tables, const int32_t* context_lens,
                                        float* lse_out, void* stream) {
  pkv::DecodeArgs a;
  pkv_status st = build_args(p, out, q, k_cache, v_cache, block_tables, context_lens, nullptr, 0, lse_out,
                             true, true, &a);
  if (st != PKV_OK) return st;
  bool ok = false;
  hipError_t e = pkv::launch_decode_partitions(a, p->cache_dtype, p->head_dim, (hipStream_t)stream, &ok);
  if (!ok) return pkv_fail(PKV_ERR_UNSUPPORTED, "decode_noalloc: no kernel variant");
  st = check_hip(e, "decode_noalloc partitions launch");
  if (st != PKV_OK) return st;
  e = pkv::launch_decode_merge(a, p->out_dtype, p->head_dim, (hipStream_t)stream, &ok);
  if (!ok) return pkv_fail(PKV_ERR_UNSUPPORTED, "decode_noalloc: no merge kernel variant");
  return check_hip(e, "decode_noalloc merge launch");
}

pkv_status pkv_read_probe(const void* buf, int64_t bytes, int32_t mode, const int32_t* order,
                          int64_t tile_bytes, int64_t tiles, uint32_t* sink, int32_t grid, void* stream) {
  if (!buf || !sink || !aligned(buf, 16) || !aligned(sink, 4))
    return pkv_fail(PKV_ERR_INVALID_ARG, "read_probe: buf (16-byte aligned) and sink are required");
  if (bytes <= 0 || bytes % 16 || grid <= 0 || grid > (1 << 20) || mode < 0 || mode > 2)
    return pkv_fail(PKV_ERR_INVALID_ARG, "read_probe: bytes a positive multiple of 16, grid in [1, 2^20], mode 0..2");
  if (mode == 2 && (!order || !aligned(order, 4) || tile_bytes <= 0 || tile_bytes % 1024 || tile_bytes > bytes ||
                    tiles < 0))
    return pkv_fail(PKV_ERR_INVALID_ARG, "read_probe: tiles need an order array and a tile size that is a multiple of 1 KiB");
  return check_hip(pkv::launch_read_probe(buf, bytes, mode, order, tile_bytes, tiles, sink, grid, (hipStream_t)stream),
                   "read_probe launch");
}

}  // extern "C"
