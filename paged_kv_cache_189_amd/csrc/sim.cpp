// Continuous-batching simulation over the host block manager.
//
// "Optimizing vLLM Throughput with PagedAttention and Continuous Batching for
// Llama 3" (continuous batching admits a new request as soon as another
// finishes; max-num-seqs caps concurrency) and "vLLM PagedAttention: Memory
// Optimization & High-Throughput LLM Inference Tuning" §2 (static per-request
// reservation of the maximum length wastes memory; paging allocates blocks on
// demand) describe the two policies this compares; the scheduler details are
// this library's reading.
//
// Each iteration: (1) admission, in queue order, while fewer than
// max_num_seqs run: paged -- the request's tokens so far (prompt plus any
// tokens generated before a preemption) are added as one prompt, stopping at
// the first request that does not fit; static -- the request reserves
// ceil(max_model_len / block_size) blocks, stopping likewise.  (2) decode:
// every running request, in admission order, appends one token; when the pool
// is full the most recently admitted running request is preempted (its
// blocks freed, it returns to the front of the queue and later recomputes
// its tokens), and the append is retried.  A request that reaches its output
// length is freed at once.  Token ids (for prefix caching): prompts carry
// theirs; generated token t of request r has id (r * 7919 + t) % 32000.
#include <cstdint>
#include <deque>
#include <string>
#include <vector>

#include "../../include/pkv.h"
#include "pkv_internal.h"

namespace {

struct Req {
  int32_t prompt_len = 0, output_len = 0, generated = 0;
  const int32_t* prompt_ids = nullptr;
  bool running = false;
};

int32_t gen_id(int32_t r, int32_t t) { return (int32_t)(((int64_t)r * 7919 + t) % 32000); }

}  // namespace

extern "C" {

pkv_status pkv_sim_run(const pkv_sim_config* cfg, const int32_t* prompt_lens,
                       const int32_t* output_lens, const int32_t* prompt_ids,
                       int32_t num_requests, pkv_sim_result* out, int32_t* running_per_iter,
                       int64_t max_iters) {
  if (!cfg || !out || num_requests < 0 || (num_requests > 0 && (!prompt_lens || !output_lens)))
    return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_sim_run: bad arguments");
  const int32_t BS = cfg->block_size, NB = cfg->num_blocks;
  if (BS <= 0 || NB <= 0 || cfg->max_model_len <= 0 || cfg->max_num_seqs <= 0 || max_iters <= 0 ||
      (cfg->policy != PKV_SIM_PAGED && cfg->policy != PKV_SIM_STATIC))
    return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_sim_run: bad config");
  const bool paged = cfg->policy == PKV_SIM_PAGED;
  const bool cache = paged && cfg->prefix_cache != 0;
  if (cache && !prompt_ids) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_sim_run: prefix cache needs prompt ids");
  const int32_t max_blocks = (cfg->max_model_len + BS - 1) / BS;
  if (!paged && max_blocks > NB)
    return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_sim_run: one static reservation does not fit the pool");
  std::vector<Req> reqs(num_requests);
  int64_t off = 0;
  for (int32_t r = 0; r < num_requests; ++r) {
    Req& q = reqs[r];
    q.prompt_len = prompt_lens[r];
    q.output_len = output_lens[r];
    if (q.prompt_len <= 0 || q.output_len <= 0 || q.prompt_len + q.output_len > cfg->max_model_len ||
        (int64_t)(q.prompt_len + q.output_len + BS - 1) / BS > NB)
      return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_sim_run: a request does not fit the model length or the pool");
    if (prompt_ids) q.prompt_ids = prompt_ids + off;
    off += q.prompt_len;
  }
  pkv_block_manager* bm = nullptr;
  pkv_status st = pkv_bm_create(NB, BS, max_blocks, nullptr, &bm);
  if (st != PKV_OK) return st;
  std::deque<int32_t> waiting;
  for (int32_t r = 0; r < num_requests; ++r) waiting.push_back(r);
  std::vector<int32_t> running;  // admission order
  int32_t reserved_blocks = 0;   // static policy
  int64_t it = 0, done = 0, generated = 0, preemptions = 0, peak = 0;
  int64_t cached_tokens = 0, admitted_tokens = 0;
  double sum_running = 0.0, sum_util = 0.0;
  std::vector<int32_t> ids;
  std::vector<int64_t> slots;
  auto tokens_of = [&](int32_t r) { return reqs[r].prompt_len + reqs[r].generated; };
  auto preempt = [&](int32_t victim) {
    if (paged) pkv_bm_free_seq(bm, victim);
    else reserved_blocks -= max_blocks;
    reqs[victim].running = false;
    waiting.push_front(victim);
    ++preemptions;
  };
  while (done < num_requests) {
    if (it >= max_iters) {
      pkv_bm_destroy(bm);
      return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_sim_run: max_iters reached");
    }
    // (1) admission
    while (!waiting.empty() && (int32_t)running.size() < cfg->max_num_seqs) {
      const int32_t r = waiting.front();
      const int32_t n = tokens_of(r);
      if (paged) {
        ids.resize(n);
        for (int32_t t = 0; t < n; ++t)
          ids[t] = t < reqs[r].prompt_len ? (reqs[r].prompt_ids ? reqs[r].prompt_ids[t] : 0)
                                          : gen_id(r, t - reqs[r].prompt_len);
        slots.resize(n > 0 ? n : 1);
        int32_t ncached = 0;
        pkv_status s;
        if (cache) {
          s = pkv_bm_add_seq_prompt(bm, r, ids.data(), n, slots.data(), &ncached);
        } else {
          s = pkv_bm_add_seq(bm, r);
          if (s == PKV_OK) {
            std::vector<int64_t> rid(n, r);
            s = pkv_bm_append_slots(bm, rid.data(), n, slots.data());
            if (s != PKV_OK) pkv_bm_free_seq(bm, r);
          }
        }
        if (s == PKV_ERR_OUT_OF_BLOCKS) break;
        if (s != PKV_OK) {
          pkv_bm_destroy(bm);
          return s;
        }
        cached_tokens += ncached;
        admitted_tokens += n;
      } else {
        if (reserved_blocks + max_blocks > NB) break;
        reserved_blocks += max_blocks;
        admitted_tokens += n;
      }
      waiting.pop_front();
      reqs[r].running = true;
      running.push_back(r);
    }
    // (2) one decode step
    std::vector<int32_t> next;
    for (size_t k = 0; k < running.size(); ++k) {
      const int32_t r = running[k];
      if (!reqs[r].running) continue;  // preempted earlier in this step
      bool ok = !paged;
      while (paged) {
        const int64_t rid = r;
        const int32_t tid = gen_id(r, reqs[r].generated);
        int64_t slot;
        pkv_status s = cache ? pkv_bm_append_tokens(bm, &rid, &tid, 1, &slot)
                             : pkv_bm_append_slots(bm, &rid, 1, &slot);
        if (s == PKV_OK) {
          ok = true;
          break;
        }
        if (s != PKV_ERR_OUT_OF_BLOCKS) {
          pkv_bm_destroy(bm);
          return s;
        }
        // preempt the most recently admitted request still running
        int32_t victim = -1;
        for (size_t j = running.size(); j-- > 0;)
          if (reqs[running[j]].running) {
            victim = running[j];
            break;
          }
        preempt(victim);
        if (victim == r) break;
      }
      if (!ok) continue;
      reqs[r].generated += 1;
      ++generated;
      if (reqs[r].generated == reqs[r].output_len) {
        if (paged) pkv_bm_free_seq(bm, r);
        else reserved_blocks -= max_blocks;
        reqs[r].running = false;
        ++done;
      } else {
        next.push_back(r);
      }
    }
    running.swap(next);
    // (3) statistics after the step
    int64_t held = 0;
    for (int32_t r : running) held += tokens_of(r);
    const int64_t used = paged ? (int64_t)NB - pkv_bm_num_free_blocks(bm) : reserved_blocks;
    if (running_per_iter) running_per_iter[it] = (int32_t)running.size();
    sum_running += (double)running.size();
    sum_util += used > 0 ? (double)held / ((double)used * BS) : 0.0;
    if ((int64_t)running.size() > peak) peak = (int64_t)running.size();
    ++it;
  }
  pkv_bm_destroy(bm);
  out->iterations = it;
  out->generated_tokens = generated;
  out->preemptions = preemptions;
  out->peak_running = peak;
  out->mean_running = it ? sum_running / (double)it : 0.0;
  out->mean_kv_utilization = it ? sum_util / (double)it : 0.0;
  out->admitted_tokens = admitted_tokens;
  out->cached_tokens = cached_tokens;
  return PKV_OK;
}

}  // extern "C"
