/*
 * pkv.h -- C ABI of a paged KV-cache decode-attention library for AMD MI355X
 * (gfx950).
 *
 * The calls follow how the pages state the problem.  Page titles, cited by
 * section below:
 *  [P1] "Optimizing Llama 3.1 405B Inference with vLLM PagedAttention"
 *  [P2] "Optimizing vLLM Throughput with PagedAttention and Continuous
 *       Batching for Llama 3"
 *  [P3] "vLLM PagedAttention Optimization: Complete Step-by-Step Tuning Guide
 *       for Low-Latency Inference"
 *  [P4] "vLLM PagedAttention: Memory Optimization & High-Throughput LLM
 *       Inference Tuning"
 *
 * What the calls cover:
 *  - a pool of fixed-size physical blocks of 16 tokens ([P1] "Why Standard
 *    Attention Fails at Scale"; [P4] §2);
 *  - a block table per sequence, mapping logical to physical blocks ([P1]
 *    "PagedAttention Mechanics"; [P3] "How PagedAttention Solves the KV Cache
 *    Bottleneck"; [P4] §2);
 *  - appending a token, which takes a physical block only when the sequence
 *    needs a new one ([P1] "PagedAttention Mechanics");
 *  - sharing of physical blocks between sequences with a common prefix ([P1]
 *    "PagedAttention Mechanics"; [P4] §2);
 *  - freeing a finished request's blocks ([P4] §4);
 *  - the cache write of each new token's K and V, and decode attention that
 *    walks the block table ([P4] §2).
 *
 * Conventions shared by every call:
 *  - No call throws.  Each returns a pkv_status; pkv_last_error() gives
 *    the text of the calling thread's last failure.
 *  - Host pointers are read or written only during the call.
 *  - Device pointers are caller-owned device memory.  The library never
 *    allocates or frees device memory; its one device array of its own is
 *    the fixed scratch of pkv_decode_attention_noalloc (below), which the
 *    HIP loader places once per GPU.  Device operations are enqueued on
 *    `stream` (a hipStream_t; NULL = the null stream), never synchronise,
 *    and their buffers must outlive the enqueued work.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    rejected call enqueues nothing.
 *  - dtype codes: PKV_F32 (IEEE binary32), PKV_BF16 (bfloat16 bit
 *    patterns), PKV_FP8_E4M3 (OCP E4M3FN codes: bias 7, no infinities,
 *    S.1111.111 = NaN, largest finite 448; [P1] "Quantization Without
 *    Quality Loss" and [P3] Step 3 name E4M3).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1,
  PKV_ERR_OUT_OF_BLOCKS = -2, /* the pool has too few free blocks ("KV cache full", [P2]) */
  PKV_ERR_UNKNOWN_SEQ = -3,
  PKV_ERR_SEQ_EXISTS = -4,
  PKV_ERR_SHARED_TAIL = -5,   /* append into a partially filled block another sequence shares */
  PKV_ERR_UNSUPPORTED = -6,   /* valid request outside the compiled kernel variants */
  PKV_ERR_HIP = -7            /* the HIP runtime reported an error (text in pkv_last_error) */
} pkv_status;

typedef enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_FP8_E4M3 = 2 } pkv_dtype;

/* ======================================================================== */
/* Host block manager                                                        */
/* ======================================================================== */
/* Owns host memory only.  Not thread-safe: one scheduler thread drives it.
 *
 * Allocation policy (the pages leave it open): free blocks form a FIFO queue
 * seeded with `free_order`; a token at position p of a sequence takes the
 * block at the head of the queue when p % block_size == 0 ([P1] "PagedAttention
 * Mechanics": a page is taken only when needed); its slot is
 * table[p / block_size] * block_size + p % block_size.  Reference counts track
 * sharing; a block whose count reaches 0 is appended to the queue tail, in
 * the order the freed sequence's table held it. */
typedef struct pkv_block_manager pkv_block_manager;

/* num_blocks > 0 physical blocks of block_size tokens; each table holds
 * max_blocks_per_seq entries.  free_order: NULL for 0..num_blocks-1, else a
 * permutation of 0..num_blocks-1 (copied).  *out receives the handle. */
pkv_status pkv_bm_create(int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                         const int32_t* free_order, pkv_block_manager** out);
void pkv_bm_destroy(pkv_block_manager* bm);

/* A new, empty sequence.  SEQ_EXISTS if the id is live. */
pkv_status pkv_bm_add_seq(pkv_block_manager* bm, int64_t seq_id);

/* A new sequence `child` holding the same tokens as `parent`: its table
 * points at the parent's physical blocks, whose reference counts grow by one
 * (prefix sharing, [P1] "PagedAttention Mechanics"; [P4] §2). */
pkv_status pkv_bm_fork_seq(pkv_block_manager* bm, int64_t parent, int64_t child);

/* Appends one token to each listed sequence, in list order (an id may
 * appear several times: one token each), writing each token's slot to
 * slot_mapping_out[i] (n entries, host memory).  All or nothing: on any
 * error no state changes.  Errors: UNKNOWN_SEQ, INVALID_ARG (a table would
 * outgrow max_blocks_per_seq), SHARED_TAIL, OUT_OF_BLOCKS. */
pkv_status pkv_bm_append_slots(pkv_block_manager* bm, const int64_t* seq_ids, int32_t n,
                               int64_t* slot_mapping_out);

/* pkv_bm_append_slots with copy-on-write.  When a listed sequence's next
 * token falls into a partially filled block that another sequence shares
 * (after a fork inside a block), that sequence first takes a fresh block
 * from the queue, the shared block loses one reference, and the pair is
 * reported: copy_src_out[k] (old block), copy_dst_out[k] (new block),
 * k < *num_copies_out, in list order.  The caller must copy those blocks on
 * the device (pkv_copy_blocks) before writing the batch's tokens.  Sharing
 * of physical blocks is on the pages ([P1] "PagedAttention Mechanics"; [P4]
 * §2); resolving a write into a shared block by copying it is this library's
 * reading.  copy_src_out / copy_dst_out hold at least n entries (host).  All
 * or nothing; errors as pkv_bm_append_slots except that SHARED_TAIL does
 * not occur. */
pkv_status pkv_bm_append_slots_cow(pkv_block_manager* bm, const int64_t* seq_ids, int32_t n,
                                   int64_t* slot_mapping_out, int32_t* copy_src_out,
                                   int32_t* copy_dst_out, int32_t* num_copies_out);

/* ---- Automatic prefix caching ------------------------------------------
 * ([P1] and [P3] turn it on with an engine flag and credit it for the
 * highest of the pages' throughput figures; they describe no scheme, so the
 * following is this library's reading.)  A full block of a sequence whose
 * token ids are known is registered under its content: its block_size ids
 * and its parent, the registered block of the previous logical block.  A new
 * prompt walks its full blocks from the start and reuses each registered
 * block whose whole token prefix equals the prompt's, so its K and V need
 * not be computed again.  A registered block whose reference count drops to
 * 0 stays cached: allocation takes the free queue first, then evicts the
 * least recently released cached block, which also drops its cached
 * descendants (they join the free queue after it, depth first).
 * pkv_bm_num_free_blocks counts cached unreferenced blocks as free. */

/* Adds sequence seq_id with the n prompt tokens token_ids (host).  Reuses
 * cached blocks for the longest matching prefix of full blocks, at most
 * (n - 1) / block_size of them (the last prompt token is always computed),
 * takes fresh blocks for the rest, and writes the slots of all n tokens to
 * slot_mapping_out (host, n entries).  *num_cached_out = tokens at the start
 * of the prompt whose K and V are already in the cache (a multiple of
 * block_size); the caller writes K and V only for the tokens after them.
 * Full blocks the prompt fills are registered.  Errors: SEQ_EXISTS,
 * INVALID_ARG (outgrows max_blocks_per_seq), OUT_OF_BLOCKS (nothing
 * changes). */
pkv_status pkv_bm_add_seq_prompt(pkv_block_manager* bm, int64_t seq_id, const int32_t* token_ids,
                                 int32_t n, int64_t* slot_mapping_out, int32_t* num_cached_out);

/* pkv_bm_append_slots with the appended tokens' ids (token_ids, host, n
 * entries): a block of a sequence added by pkv_bm_add_seq_prompt (or forked
 * from one) that becomes full is registered.  A sequence that receives a
 * token through an id-less call stops being registered from then on. */
pkv_status pkv_bm_append_tokens(pkv_block_manager* bm, const int64_t* seq_ids,
                                const int32_t* token_ids, int32_t n, int64_t* slot_mapping_out);

/* Registered blocks (referenced or waiting in the LRU list). */
int32_t pkv_bm_num_cached_blocks(const pkv_block_manager* bm);

/* Drops the sequence; each of its blocks loses one reference ([P4] §4). */
pkv_status pkv_bm_free_seq(pkv_block_manager* bm, int64_t seq_id);

/* Writes, for the n listed sequences, their tables into block_tables_out
 * (n x max_blocks_per_seq int32, row-major; entries past the last used block
 * are -1) and their token counts into context_lens_out (n int32). */
pkv_status pkv_bm_export(const pkv_block_manager* bm, const int64_t* seq_ids, int32_t n,
                         int32_t* block_tables_out, int32_t* context_lens_out);

int32_t pkv_bm_num_free_blocks(const pkv_block_manager* bm);
/* Reference count of a physical block (-1 if out of range). */
int32_t pkv_bm_refcount(const pkv_block_manager* bm, int32_t block);

/* ======================================================================== */
/* Device memory layout                                                      */
/* ======================================================================== */
/* The pages fix no layout; this library's is:
 *   q, out        [num_seqs][num_q_heads][head_dim]
 *   k_new, v_new  [num_tokens][num_kv_heads][head_dim]
 *   k_cache       [num_blocks][num_kv_heads][head_dim / X][block_size][X],
 *                 X = 16 bytes / element size (f32 4, bf16 8, fp8 16)
 *   v_cache       [num_blocks][num_kv_heads][head_dim][block_size]
 *   block_tables  [num_seqs][max_blocks_per_seq] int32
 *   context_lens  [num_seqs] int32
 *   slot_mapping  [num_tokens] int64, slot = block * block_size + offset
 * One (block, kv head) K tile keeps 16 bytes of one token's K contiguous,
 * tokens next; the V tile keeps one dimension's block_size token values
 * contiguous.  The kernels take block_size 16 or 32.
 * Query head h reads KV head h / (num_q_heads / num_kv_heads). */

/* ======================================================================== */
/* Cache write                                                               */
/* ======================================================================== */
/* Writes each new token's K and V into the slot slot_mapping[i] names ([P1]
 * "PagedAttention Mechanics": a new token is appended to its sequence).
 *   src_dtype  : PKV_F32 or PKV_BF16 (k_new, v_new)
 *   cache_dtype: PKV_F32 (src f32 only), PKV_BF16, PKV_FP8_E4M3
 * Values are copied bit for bit when the dtypes match, rounded to nearest
 * even for f32 -> bf16, and for fp8 stored as the satfinite round-to-nearest-
 * even E4M3 code of the fp32 quotient x / scale (k_scale for K, v_scale for
 * V; both > 0).  A slot < 0, or >= num_blocks * block_size, is skipped.
 * Two tokens with one slot race (the block manager never issues that).
 * head_dim in {64, 128}, block_size 16 or 32 (the pool layout's). */
pkv_status pkv_reshape_and_cache(const void* k_new, const void* v_new, pkv_dtype src_dtype,
                                 void* k_cache, void* v_cache, pkv_dtype cache_dtype,
                                 const int64_t* slot_mapping, int32_t num_tokens,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int64_t num_blocks, float k_scale, float v_scale, void* stream);

/* Decode-step append on the device: the cache write above for one new token
 * per sequence, which also keeps a device copy of the block tables in step
 * with the host block manager ([P1] "PagedAttention Mechanics": appending a
 * token takes a fresh page only at a page boundary; [P4] section 2: the
 * kernel finds a token's page through the block table).  Token i is sequence
 * i's newest token, at position p = context_lens[i] - 1 (context_lens already
 * counts it); besides writing its K and V into slot_mapping[i] as
 * pkv_reshape_and_cache does, it sets
 *   block_tables[i * max_blocks_per_seq + p / block_size] = slot_mapping[i] / block_size,
 * which is the entry the block manager exports (a new block at a block
 * boundary, or the copy a copy-on-write gave the sequence).  A token with a
 * skipped slot, or with p < 0 or p / block_size >= max_blocks_per_seq,
 * leaves its table row alone.  k_new, v_new: [num_seqs][num_kv_heads][head_dim];
 * context_lens [num_seqs] int32 and block_tables [num_seqs][max_blocks_per_seq]
 * int32 are device memory (block_tables is written).  Errors as
 * pkv_reshape_and_cache, plus PKV_ERR_INVALID_ARG for NULL tables or lengths
 * or max_blocks_per_seq <= 0. */
pkv_status pkv_append_decode_tokens(const void* k_new, const void* v_new, pkv_dtype src_dtype,
                                    void* k_cache, void* v_cache, pkv_dtype cache_dtype,
                                    const int64_t* slot_mapping, const int32_t* context_lens,
                                    int32_t* block_tables, int32_t max_blocks_per_seq,
                                    int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int64_t num_blocks, float k_scale,
                                    float v_scale, void* stream);

/* Copies whole physical blocks (K and V, every kv head, all block_size
 * slots, bit for bit): block dst[i] <- block src[i] for i < n, e.g. the
 * copy-on-write pairs of pkv_bm_append_slots_cow.  src, dst: device int32
 * arrays of n entries, each in [0, num_blocks); a pair with an entry out of
 * range is skipped; a dst that is also some src, or two equal dst, race.
 * cache_dtype: any pkv_dtype; head_dim in {64, 128}; block_size 16 or 32. */
pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, pkv_dtype cache_dtype,
                           const int32_t* src, const int32_t* dst, int32_t n,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int64_t num_blocks, void* stream);

/* ======================================================================== */
/* Decode attention over the paged cache                                     */
/* ======================================================================== */
/* For each sequence s and query head h (g = h / G, G = Hq / Hkv), over the
 * L_s = context_lens[s] tokens whose K and V the table reaches ([P4] §1: the
 * next token attends to every earlier token; [P4] §2: the kernel fetches
 * K and V by walking the block table):
 *   sc_t = scale * k_scale * q[s][h] . K_t
 *   out[s][h] = sum_t softmax(sc)_t * v_scale * V_t,  lse[s][h] = ln sum_t e^{sc_t}
 * The softmax is evaluated with a running maximum.  The work is cut into
 * pieces attended independently and merged by log-sum-exp (split-KV): the
 * (kv head, sequence, block) positions of the batch are divided into equal
 * ranges, one per resident pass-1 wave, so a long context spans many
 * ranges; partition_size > 0 adds a cut every partition_size tokens of each
 * sequence.  The pieces change only the rounding order.  L_s == 0 yields a
 * zero row and lse = -inf.
 *
 * Supported (q, cache, out) dtypes: (F32, F32, F32), (BF16, BF16, BF16),
 * (BF16, FP8_E4M3, BF16).  head_dim in {64, 128}; block_size 16 or 32
 * ([P1] "Why Standard Attention Fails at Scale" gives 16 as the default;
 * [P2] "Key Tuning Insights" tried 32 as the alternative);
 * 1 <= Hq / Hkv <= 16; partition_size = 0 (no partition cuts) or a
 * positive multiple of block_size.  context_lens must lie in [0, max_context_len] and
 * max_context_len <= max_blocks_per_seq * block_size; table entries of the
 * first ceil(L_s / block_size) columns must be < num_blocks.  Other entries and slots
 * past L_s are never read (they may hold anything, NaN included).  Out-of-
 * range lengths are clamped and out-of-range block ids are clamped into the
 * pool, so a bad input never reads outside the buffers; its output is then
 * unspecified. */
typedef struct {
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t max_blocks_per_seq;
  int32_t max_context_len;
  int32_t partition_size; /* tokens per split-KV partition; 0 = no partition cuts */
  int64_t num_blocks;
  float scale;            /* usually 1/sqrt(head_dim) */
  float k_scale;          /* dequant scale of the K cache (1 unless fp8) */
  float v_scale;
  int32_t q_dtype;        /* pkv_dtype */
  int32_t cache_dtype;
  int32_t out_dtype;
} pkv_decode_params;

/* Bytes of device workspace pkv_decode_attention needs for these params
 * (0 only for invalid params).  The workspace holds the plan built on the
 * device from context_lens (block prefix sums) and the partial states
 * (o, m, l, e) of split pieces -- m, l, e in fp32; o in fp32 for fp32
 * outputs, otherwise bf16 and divided by its own l.  Its size depends on
 * the params, not on context_lens.  It need not be initialised; it must be
 * 256-byte aligned.
 * Calls that share a workspace must be ordered on one stream. */
size_t pkv_decode_workspace_bytes(const pkv_decode_params* p);

/* The partition size (tokens) the call will use for these params (0: no
 * partition cuts; -1: invalid params). */
int32_t pkv_decode_partition_size(const pkv_decode_params* p);

/* The number R of pass-1 ranges (one per resident pass-1 wave) a call with
 * these params divides the batch into on the calling thread's current
 * device: 0 for an empty batch, -1 for invalid params or a failed device
 * query (text in pkv_last_error).  It depends on the device and the kernel
 * variant, not on context_lens; the partial-state slots of a call are below
 * (split-KV partitions of all (sequence, kv head) pairs) + R. */
int32_t pkv_decode_num_ranges(const pkv_decode_params* p);

/* Both passes: per-partition attention, then the log-sum-exp merge.
 * out: [S][Hq][D] of out_dtype.  lse_out: NULL or [S][Hq] fp32.
 * workspace: device memory of at least pkv_decode_workspace_bytes(p). */
pkv_status pkv_decode_attention(const pkv_decode_params* p, void* out, const void* q,
                                const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, const int32_t* context_lens,
                                void* workspace, size_t workspace_bytes, float* lse_out,
                                void* stream);

/* Pass 1 alone: one kernel whose resident waves each attend to an equal
 * range of the batch's blocks.  A (sequence, kv head) whose pieces all fall
 * to one workgroup (and, with partition cuts, to one partition) gets its
 * final out / lse here; the others leave partial states in the
 * workspace for pass 2 (and empty sequences are left to pass 2).  Up to
 * 1024 sequences the plan is built inside the kernel; larger batches add a
 * one-workgroup planning kernel before it. */
pkv_status pkv_decode_attention_partitions(const pkv_decode_params* p, void* out, const void* q,
                                           const void* k_cache, const void* v_cache,
                                           const int32_t* block_tables,
                                           const int32_t* context_lens, void* workspace,
                                           size_t workspace_bytes, float* lse_out, void* stream);

/* Pass 2 alone: merges the partial states pass 1 left: M = max_p m_p,
 * Lambda = sum_p l_p e^{m_p - M}, out = sum_p e^{m_p - M} o_p / Lambda
 * (o_p = l_p times the stored row where rows are stored normalised),
 * lse = M + ln Lambda; also writes the zero rows of empty sequences.  Must
 * follow pass 1 of the same params, inputs and workspace on the same stream,
 * on the same device (the range count depends on the device). */
pkv_status pkv_decode_attention_merge(const pkv_decode_params* p, void* out,
                                      const int32_t* context_lens, const void* workspace,
                                      size_t workspace_bytes, float* lse_out, void* stream);

/* Decode attention that allocates nothing, for callers that cannot call
 * hipMalloc or take a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments, kernels and
 * results (bit for bit) as pkv_decode_attention, without the workspace: the
 * partial states and the plan live in a static device array of the library,
 * PKV_NOALLOC_SCRATCH_BYTES (64 MiB) on each GPU it runs on, held until the
 * process ends.  The call uses the copy of the calling thread's current
 * device (`stream` must belong to it); the array's address on that device is
 * looked up on the first call there.  Calls whose partial states and plan
 * need more (the bound of pkv_decode_workspace_bytes, with the device's own
 * range count, pkv_decode_num_ranges, in place of the 16384 it assumes)
 * return PKV_ERR_UNSUPPORTED with the size in pkv_last_error and enqueue
 * nothing -- e.g. 8 sequences of 128 query heads over 131072 tokens with
 * 512-token partitions need ~76 MB, the same without partition cuts ~9 MB.
 * Nothing in the array needs to start at zero.  Every call on a GPU shares
 * that GPU's array and leaves its contents there: two calls that overlap on
 * one GPU (other streams, other threads) race and give wrong results, so
 * order them on one stream. */
#define PKV_NOALLOC_SCRATCH_BYTES (64u << 20)
pkv_status pkv_decode_attention_noalloc(const pkv_decode_params* p, void* out, const void* q,
                                        const void* k_cache, const void* v_cache,
                                        const int32_t* block_tables,
                                        const int32_t* context_lens, float* lse_out,
                                        void* stream);

/* ======================================================================== */
/* Chunked prefill attention over the paged cache                            */
/* ======================================================================== */
/* Attention for a chunk of new tokens per sequence (chunked prefill, named
 * as an engine setting in [P2] and [P3] Step 2; the pages give no formula).
 * Sequence s holds L_s = context_lens[s] tokens in the cache, the last
 * C_s = query_start[s+1] - query_start[s] of which are its chunk (their K
 * and V already written, e.g. by pkv_reshape_and_cache of all C_s tokens).
 * Query row i = query_start[s] + j (0 <= j < C_s) is the token at position
 * p = L_s - C_s + j and attends causally to tokens 0..p:
 *   sc_t = scale * k_scale * q[i][h] . K_t (t <= p)
 *   out[i][h] = sum_t softmax(sc)_t * v_scale * V_t,  lse[i][h] = ln sum_t e^{sc_t}
 * With C_s = 1 this is decode.  A row with p < 0 (C_s > L_s) gets a zero row
 * and lse = -inf.  q, out: [num_query_tokens][Hq][D] (rows packed by
 * sequence); lse_out: NULL or [num_query_tokens][Hq] fp32.
 * query_start: device int32 [num_seqs + 1], non-decreasing, query_start[0]
 * = 0 and query_start[num_seqs] = num_query_tokens (not checked: it lives
 * on the device).  Other fields, dtypes and limits as pkv_decode_params;
 * num_seqs <= 1024; scale may be any finite number (negative and zero
 * included).  PKV_ERR_UNSUPPORTED also when a physical block of all kv heads
 * (num_kv_heads * block_size * head_dim * element bytes) reaches 4 GiB.  No
 * workspace: a workgroup takes a (kv head, sequence, run of query tokens) and
 * walks the table up to its last row's position.
 * Rounding: bf16 and fp8 caches multiply bf16-rounded weights into V and
 * normalise the output by the sum of those rounded weights (lse: by their
 * fp32 sum). */
typedef struct {
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t max_blocks_per_seq;
  int32_t max_context_len;
  int32_t num_query_tokens;
  int64_t num_blocks;
  float scale;
  float k_scale;
  float v_scale;
  int32_t q_dtype;
  int32_t cache_dtype;
  int32_t out_dtype;
} pkv_prefill_params;

pkv_status pkv_prefill_attention(const pkv_prefill_params* p, void* out, const void* q,
                                 const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 const int32_t* query_start, float* lse_out, void* stream);

/* ======================================================================== */
/* Continuous-batching simulation (host only)                                */
/* ======================================================================== */
/* Runs a request trace through a scheduler over the block manager and
 * reports concurrency and KV-memory use, comparing paging with a static
 * per-request reservation of max_model_len ([P2] on continuous batching and
 * max-num-seqs; [P4] §2 on the waste of static reservation).  Scheduler
 * (this library's reading), per iteration:
 *  1. admission in queue order while fewer than max_num_seqs run: PAGED adds
 *     the request's tokens so far as one prompt (through the prefix cache
 *     when prefix_cache != 0), STATIC reserves ceil(max_model_len /
 *     block_size) blocks; the first request that does not fit stops it;
 *  2. every running request, in admission order, appends one token; when the
 *     pool is full the most recently admitted running request is preempted
 *     (blocks freed, back to the front of the queue, its tokens recomputed on
 *     re-admission) and the append is retried; a request reaching its output
 *     length is freed at once;
 *  3. statistics after the step.
 * Generated token t of request r has id (r * 7919 + t) % 32000. */
enum { PKV_SIM_PAGED = 0, PKV_SIM_STATIC = 1 };

typedef struct {
  int32_t num_blocks;
  int32_t block_size;
  int32_t max_model_len;  /* prompt + output of every request must fit */
  int32_t max_num_seqs;
  int32_t policy;         /* PKV_SIM_PAGED or PKV_SIM_STATIC */
  int32_t prefix_cache;   /* PAGED only: admit prompts through the prefix cache */
} pkv_sim_config;

typedef struct {
  int64_t iterations;         /* decode steps until every request finished */
  int64_t generated_tokens;   /* tokens appended (recomputed ones excluded) */
  int64_t preemptions;
  int64_t peak_running;
  double mean_running;        /* running requests per iteration */
  double mean_kv_utilization; /* tokens held (per sequence) / slots of the blocks in use;
                                 above 1 when sequences share blocks */
  int64_t admitted_tokens;    /* tokens added at admissions (prompts, recomputations) */
  int64_t cached_tokens;      /* of those, found in the prefix cache */
} pkv_sim_result;

/* prompt_lens, output_lens: num_requests entries (host), each > 0 and
 * prompt + output <= max_model_len and fitting the pool.  prompt_ids: NULL
 * or the prompts' token ids concatenated (required with prefix_cache).
 * running_per_iter: NULL or max_iters entries receiving the running count
 * after each iteration.  INVALID_ARG when a request cannot fit or max_iters
 * is reached. */
pkv_status pkv_sim_run(const pkv_sim_config* cfg, const int32_t* prompt_lens,
                       const int32_t* output_lens, const int32_t* prompt_ids,
                       int32_t num_requests, pkv_sim_result* out, int32_t* running_per_iter,
                       int64_t max_iters);

/* ======================================================================== */
/* Diagnostics                                                               */
/* ======================================================================== */
const char* pkv_status_string(pkv_status s);
/* Text of the calling thread's last failed call ("" if none). */
const char* pkv_last_error(void);
/* Library version string. */
const char* pkv_version(void);

/* Read-bandwidth probe, the measured ceiling beside the HBM peak: reads
 * `bytes` (a positive multiple of 16) of device memory at buf (16-byte
 * aligned).  mode 0: one contiguous sweep with the default cache policy;
 * mode 1: the same with non-temporal loads; mode 2: `tiles` whole tiles of
 * tile_bytes (a multiple of 1 KiB) in the order of the device int32 array
 * `order` (tile ids, clamped into the buffer), non-temporal -- the access of
 * a block-table walk over randomly placed blocks.  grid: workgroups of 256
 * threads.  sink: device memory of grid * 256 uint32 (written only where a
 * thread's folded data hits one fixed bit pattern by chance).  The caller
 * times the launch. */
pkv_status pkv_read_probe(const void* buf, int64_t bytes, int32_t mode, const int32_t* order,
                          int64_t tile_bytes, int64_t tiles, uint32_t* sink, int32_t grid,
                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
