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
  float* ws_o;   // [S][Hq][max_parts][D]  partial sum_t e^{s_t - m} v_t (v_scale applied)
  float* ws_m;   // [S][Hq][max_parts]     partition max, log2 units
  float* ws_l;   // [S][Hq][max_parts]     partition sum of the weights as multiplied into V
  float* ws_e;   // [S][Hq][max_parts]     partition sum of the fp32 weights (for lse)
  float* lse;    // [S][Hq] or null
  int64_t num_blocks;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t max_blocks;
  int32_t max_context_len;
  int32_t part_blocks;  // blocks per partition
  int32_t max_parts;    // partitions of the longest allowed sequence
  float score_scale_log2;  // scale * k_scale * log2(e)
  float v_scale;
};

struct CacheWriteArgs {
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  const int64_t* slot_mapping;
  int64_t num_blocks;
  int32_t num_tokens;
  int32_t num_kv_heads;
  float k_scale;
  float v_scale;
};

// Kernel variants are chosen by these codes (pkv_dtype values).
hipError_t launch_cache_write(const CacheWriteArgs& a, int src_dtype, int cache_dtype,
                              int head_dim, hipStream_t stream, bool* supported);
hipError_t launch_decode_partitions(const DecodeArgs& a, int cache_dtype, int head_dim,
                                    hipStream_t stream, bool* supported);
hipError_t launch_decode_merge(const DecodeArgs& a, int out_dtype, int head_dim,
                               hipStream_t stream, bool* supported);

// Waves per workgroup of the partition kernel.
constexpr int kWavesPerGroup = 4;

}  // namespace pkv
