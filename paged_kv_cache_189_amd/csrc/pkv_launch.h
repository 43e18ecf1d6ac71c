// Kernel argument blocks and launchers of libpkv (internal).
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstddef>
#include <cstdint>

namespace pkv {


// Arguments of the attention kernels (passed by value).
struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_o;   // [segments][G][D]  partial sum_t e^{s_t - m} v_t (v_scale applied)
  float* ws_m;   // [segments][G]     segment max, log2 units
  float* ws_l;   // [segments][G]     sum of the weights as multiplied into V
  float* ws_e;   // [segments][G]     sum of the fp32 weights (for lse)
  float* lse;    // [S][Hq] or null
  int32_t* cum;         // [S + 1]  plan: prefix sums of blocks per sequence
  int32_t* cum_parts;   // [S + 1]  plan: prefix sums of partitions per sequence
  int32_t* range_pair;  // [R]      plan: first (kv head, sequence) pair of each range
  int64_t num_blocks;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t max_blocks;
  int32_t max_context_len;
  int32_t part_blocks;  // 16-token tiles per partition (0: cut only at range starts)
  int32_t block_shift;  // log2(block_size / 16): tiles per physical block = 1 << block_shift
  int32_t num_ranges;   // pass-1 waves, one range each (a multiple of 8 * waves per group)
  float score_scale_log2;  // scale * k_scale * log2(e)
  float v_scale;
};

// Chunked prefill: the query rows of sequence s are
// [query_start[s], query_start[s+1]), the last tokens of its context.
struct PrefillArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start;  // [S + 1]
  float* lse;                  // [rows][Hq] or null
  int64_t num_blocks;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t max_blocks;
  int32_t max_context_len;
  int32_t tokens_per_tile;  // query tokens sharing one 16-row MFMA tile: 16 / group
  int32_t block_shift;
  float score_scale_log2;
  float v_scale;
};

// Largest batch the prefill kernel plans in LDS.
constexpr int kPrefillMaxSeqs = 1024;

hipError_t launch_prefill(const PrefillArgs& a, int cache_dtype, int head_dim, int64_t num_rows,
                          hipStream_t stream, bool* supported);

struct CacheWriteArgs {
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  const int64_t* slot_mapping;
  // Decode append (optional): token t is sequence t's newest token, at
  // position context_lens[t] - 1; its table entry is set to its block.
  const int32_t* context_lens;
  int32_t* block_tables;  // [num_tokens][max_blocks] or null
  int64_t num_blocks;
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t block_size;  // tokens per physical block (16 or 32)
  int32_t max_blocks;
  float k_scale;
  float v_scale;
};

struct CopyBlocksArgs {
  void* k_cache;
  void* v_cache;
  const int32_t* src;
  const int32_t* dst;
  int64_t num_blocks;
  int64_t block_bytes;  // bytes of one physical block of one cache (K or V)
  int32_t n;
};

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream);

// Kernel variants are chosen by these codes (pkv_dtype values).
hipError_t launch_cache_write(const CacheWriteArgs& a, int src_dtype, int cache_dtype,
                              int head_dim, hipStream_t stream, bool* supported);
hipError_t launch_decode_partitions(const DecodeArgs& a, int cache_dtype, int head_dim,
                                    hipStream_t stream, bool* supported);
hipError_t launch_decode_merge(const DecodeArgs& a, int out_dtype, int head_dim,
                               hipStream_t stream, bool* supported);

// Read-bandwidth probe (read_probe.hip): mode 0 contiguous sweep, 1 the same
// non-temporal, 2 whole tiles in the order `order` (non-temporal); `grid`
// workgroups of 256 threads; sink holds grid * 256 words.
hipError_t launch_read_probe(const void* buf, int64_t bytes, int mode, const int32_t* order,
                             int64_t tile_bytes, int64_t tiles, uint32_t* sink, int grid,
                             hipStream_t stream);

// Waves per workgroup of the partition kernel.
constexpr int kWavesPerGroup = 4;
// Upper bound of pass-1 workgroups (ranges); sizes the workspace.
constexpr int kMaxRanges = 16384;

// Pass-1 ranges (one per resident wave) for a cache dtype / head dim / batch
// size / block shift on the current device, capped by the number of 16-token
// tiles that can exist.
int decode_ranges(int cache_dtype, int head_dim, int num_seqs, int block_shift,
                  int64_t max_blocks_total, hipError_t* err);

}  // namespace pkv
