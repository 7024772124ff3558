// Continuous-batching scheduler over the host block pool.  Pure C++17, no
// GPU runtime: it plans each step (which chunks of which requests run, their
// KV slots) through the pool's own C ABI, and the caller runs the kernels.
//
// Follows (page title and section):
//   - techfeed.io ngrok summary, scheduler section: every forward pass takes
//     the batch's tokens within a token budget, running (decoding) requests
//     first and waiting requests' prefill with what is left; very long
//     prompts are split into chunks over several passes; when KV blocks run
//     out, the most recently added request is preempted: its blocks are
//     freed, it returns to the head of the waiting queue and is computed
//     again from its prompt later.
//   - ta-paperlens "LLM serving from scratch", scheduler skeleton: admit from
//     the waiting queue while the head can be allocated, step all running
//     requests, remove finished ones and free their blocks, and while out of
//     blocks preempt running[-1] -- moved to CPU memory or dropped for
//     recomputation.  Swap mode takes the first: a preempted request keeps
//     its progress, its blocks are moved out (the caller copies them to host
//     memory) and it resumes, ahead of new admissions, in fresh blocks.
#include <algorithm>
#include <cstdint>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"

namespace {

constexpr int32_t kBS = PA_BLOCK_SIZE;

struct Req {
  int32_t prompt = 0;
  int32_t out = 0;
  int32_t computed = 0;   // input tokens whose K/V are in the cache
  int32_t generated = 0;  // output tokens produced
  int32_t preemptions = 0;
  int32_t total() const { return prompt + generated; }  // input length
  // exactly the newest token is left and it follows the prompt: a decode step
  bool decoding() const { return total() - computed == 1 && computed >= prompt; }
};

inline int32_t blocks_for(int64_t tokens) { return static_cast<int32_t>((tokens + kBS - 1) / kBS); }

struct SwapOp {
  int64_t req;
  int32_t kind;  // 0: out, 1: in
  int32_t len;
  std::vector<int32_t> blocks;
};

}  // namespace

struct pa_sched {
  pa_pool* pool = nullptr;
  int32_t budget = 0;
  int32_t max_running = 0;
  std::unordered_map<int64_t, Req> reqs;
  std::deque<int64_t> waiting;
  std::vector<int64_t> running;  // admission order
  // the planned step, consumed by pa_sched_commit
  std::vector<pa_sched_item> planned;
  bool has_plan = false;
  bool swap = false;
  std::deque<int64_t> swapped;   // swapped-out requests, next to resume first
  std::vector<SwapOp> swap_ops;  // the planned step's: outs, then ins
  int64_t steps = 0, preemptions = 0, finished = 0;
};

extern "C" {

pa_status pa_sched_create(pa_pool* pool, int32_t token_budget, int32_t max_running,
                          pa_sched** out) {
  if (pool == nullptr || out == nullptr || token_budget < 1 || max_running < 1)
    return PA_ERR_INVALID;
  pa_sched* s = new (std::nothrow) pa_sched();
  if (s == nullptr) return PA_ERR_INTERNAL;
  s->pool = pool;
  s->budget = token_budget;
  s->max_running = max_running;
  *out = s;
  return PA_OK;
}

void pa_sched_destroy(pa_sched* s) { delete s; }

pa_status pa_sched_add_request(pa_sched* s, int64_t req_id, int32_t prompt_len,
                               int32_t output_len) {
  if (s == nullptr || prompt_len < 1 || output_len < 1) return PA_ERR_INVALID;
  if (s->reqs.count(req_id)) return PA_ERR_EXISTS;
  pa_pool_stats st;
  if (pa_pool_get_stats(s->pool, &st) != PA_OK) return PA_ERR_INVALID;
  // the prompt and all but the last output token must fit the pool alone
  if (static_cast<int64_t>(prompt_len) + output_len - 1 > INT32_MAX - kBS ||
      blocks_for(static_cast<int64_t>(prompt_len) + output_len - 1) > st.num_blocks)
    return PA_ERR_INVALID;
  Req r;
  r.prompt = prompt_len;
  r.out = output_len;
  s->reqs.emplace(req_id, r);
  s->waiting.push_back(req_id);
  return PA_OK;
}

pa_status pa_sched_schedule(pa_sched* s, pa_sched_item* items, int32_t item_cap,
                            int32_t* n_items, int32_t* slot_mapping, int64_t slot_cap,
                            pa_copy* copies, int32_t copy_cap, int32_t* n_copies,
                            int64_t* preempted, int32_t preempt_cap, int32_t* n_preempted) {
  if (s == nullptr || n_items == nullptr || n_copies == nullptr || n_preempted == nullptr)
    return PA_ERR_INVALID;
  if (s->has_plan) return PA_ERR_INVALID;  // commit the previous step first
  // every buffer is sized for the worst case before anything changes
  if (item_cap < s->max_running || slot_cap < s->budget || copy_cap < s->max_running ||
      preempt_cap < s->max_running || items == nullptr || slot_mapping == nullptr ||
      copies == nullptr || preempted == nullptr)
    return PA_ERR_CAPACITY;

  // swap mode: resume swapped requests first, while the pool holds their
  // blocks plus one block per running request
  std::vector<SwapOp> ins, outs;
  while (!s->swapped.empty() && static_cast<int32_t>(s->running.size()) < s->max_running) {
    const int64_t id = s->swapped.front();
    const Req& r = s->reqs[id];
    const int32_t nb = blocks_for(r.computed);
    if (nb + static_cast<int32_t>(s->running.size()) > pa_num_free_blocks(s->pool)) break;
    SwapOp op{id, 1, r.computed, std::vector<int32_t>(static_cast<size_t>(nb))};
    int32_t got = 0;
    const pa_status st = pa_seq_swap_in(s->pool, id, r.computed, op.blocks.data(), nb, &got);
    if (st != PA_OK) return st;
    s->swapped.pop_front();
    s->running.push_back(id);
    ins.push_back(std::move(op));
  }

  int32_t budget = s->budget;
  std::vector<int64_t> ids;
  std::vector<int32_t> ns;
  for (int64_t id : s->running) {  // decode first
    const Req& r = s->reqs[id];
    if (r.decoding() && budget > 0) {
      ids.push_back(id);
      ns.push_back(1);
      budget -= 1;
    }
  }
  for (int64_t id : s->running) {  // then running prefill chunks
    const Req& r = s->reqs[id];
    if (!r.decoding() && budget > 0) {
      const int32_t n = std::min(r.total() - r.computed, budget);
      ids.push_back(id);
      ns.push_back(n);
      budget -= n;
    }
  }
  int32_t need = 0;
  if (!ids.empty()) {
    const pa_status st = pa_can_append(s->pool, static_cast<int32_t>(ids.size()), ids.data(),
                                       ns.data(), &need);
    if (st != PA_OK) return st;
  }
  int32_t spare = pa_num_free_blocks(s->pool) - need;
  while (!s->waiting.empty() && budget > 0 &&
         static_cast<int32_t>(s->running.size()) < s->max_running) {
    const int64_t id = s->waiting.front();
    const Req& r = s->reqs[id];
    const int32_t n = std::min(r.total() - r.computed, budget);
    const int32_t blocks = blocks_for(n);
    if (blocks > spare) break;
    s->waiting.pop_front();
    const pa_status st = pa_seq_add(s->pool, id);
    if (st != PA_OK) return st;
    s->running.push_back(id);
    ids.push_back(id);
    ns.push_back(n);
    budget -= n;
    spare -= blocks;
  }
  int32_t n_pre = 0;
  int32_t ncopy = 0;
  for (;;) {
    const pa_status st = pa_append_slots(s->pool, static_cast<int32_t>(ids.size()), ids.data(),
                                         ns.data(), slot_mapping, slot_cap, copies, copy_cap,
                                         &ncopy);
    if (st == PA_OK) break;
    if (st != PA_ERR_OUT_OF_BLOCKS || s->running.empty()) return st;
    const int64_t victim = s->running.back();  // the request added last
    s->running.pop_back();
    Req& v = s->reqs[victim];
    auto resumed = std::find_if(ins.begin(), ins.end(),
                                [victim](const SwapOp& o) { return o.req == victim; });
    if (s->swap && resumed != ins.end()) {
      // resumed in this very step: back to the swapped queue, its saved copy
      // is still the current one and nothing moves
      const pa_status fs = pa_seq_free(s->pool, victim);
      if (fs != PA_OK) return fs;
      ins.erase(resumed);
      s->swapped.push_front(victim);
    } else if (s->swap && v.computed > 0) {
      SwapOp op{victim, 0, 0, std::vector<int32_t>(static_cast<size_t>(blocks_for(v.computed)))};
      int32_t nb = 0;
      const pa_status fs = pa_seq_swap_out(s->pool, victim, op.blocks.data(),
                                           static_cast<int32_t>(op.blocks.size()), &nb, &op.len);
      if (fs != PA_OK) return fs;
      op.blocks.resize(static_cast<size_t>(nb));
      outs.push_back(std::move(op));
      s->swapped.push_front(victim);
    } else {
      const pa_status fs = pa_seq_free(s->pool, victim);
      if (fs != PA_OK) return fs;
      v.computed = 0;
      s->waiting.push_front(victim);
    }
    ++v.preemptions;
    ++s->preemptions;
    preempted[n_pre++] = victim;
    for (size_t i = 0; i < ids.size(); ++i) {
      if (ids[i] == victim) {
        ids.erase(ids.begin() + static_cast<std::ptrdiff_t>(i));
        ns.erase(ns.begin() + static_cast<std::ptrdiff_t>(i));
        break;
      }
    }
  }
  s->planned.clear();
  for (size_t i = 0; i < ids.size(); ++i) {
    const Req& r = s->reqs[ids[i]];
    pa_sched_item it;
    it.req_id = ids[i];
    it.start = r.computed;
    it.n_tokens = ns[i];
    it.decode = (ns[i] == 1 && r.computed >= r.prompt) ? 1 : 0;
    it.reserved = 0;
    items[i] = it;
    s->planned.push_back(it);
  }
  s->swap_ops = std::move(outs);
  for (SwapOp& op : ins) s->swap_ops.push_back(std::move(op));
  *n_items = static_cast<int32_t>(ids.size());
  *n_copies = ncopy;
  *n_preempted = n_pre;
  s->has_plan = true;
  ++s->steps;
  return PA_OK;
}

pa_status pa_sched_commit(pa_sched* s, int64_t* finished, int32_t cap, int32_t* n_finished) {
  if (s == nullptr || n_finished == nullptr) return PA_ERR_INVALID;
  if (!s->has_plan) return PA_ERR_INVALID;
  if (cap < static_cast<int32_t>(s->planned.size()) ||
      (!s->planned.empty() && finished == nullptr))
    return PA_ERR_CAPACITY;
  int32_t nf = 0;
  for (const pa_sched_item& it : s->planned) {
    Req& r = s->reqs[it.req_id];
    r.computed = it.start + it.n_tokens;
    if (r.computed == r.total()) {
      ++r.generated;
      if (r.generated == r.out) finished[nf++] = it.req_id;
    }
  }
  for (int32_t i = 0; i < nf; ++i) {
    const int64_t id = finished[i];
    s->running.erase(std::find(s->running.begin(), s->running.end(), id));
    const pa_status st = pa_seq_free(s->pool, id);
    if (st != PA_OK) return st;
    ++s->finished;
  }
  s->planned.clear();
  s->swap_ops.clear();
  s->has_plan = false;
  *n_finished = nf;
  return PA_OK;
}

pa_status pa_sched_set_swap(pa_sched* s, int32_t enable) {
  if (s == nullptr || s->has_plan) return PA_ERR_INVALID;
  if (!enable && !s->swapped.empty()) return PA_ERR_INVALID;  // they could never resume
  s->swap = enable != 0;
  return PA_OK;
}

pa_status pa_sched_swaps(const pa_sched* s, pa_sched_swap* ops, int32_t cap, int32_t* n_ops,
                         int32_t* blocks, int64_t blocks_cap, int64_t* n_blocks) {
  if (s == nullptr || n_ops == nullptr || n_blocks == nullptr || !s->has_plan)
    return PA_ERR_INVALID;
  int64_t total = 0;
  for (const SwapOp& op : s->swap_ops) total += static_cast<int64_t>(op.blocks.size());
  const int32_t n = static_cast<int32_t>(s->swap_ops.size());
  *n_ops = n;
  *n_blocks = total;
  if (n > cap || total > blocks_cap) return PA_ERR_CAPACITY;
  if ((n > 0 && ops == nullptr) || (total > 0 && blocks == nullptr)) return PA_ERR_INVALID;
  int64_t off = 0;
  for (int32_t i = 0; i < n; ++i) {
    const SwapOp& op = s->swap_ops[static_cast<size_t>(i)];
    ops[i] = pa_sched_swap{op.req, op.kind, op.len, off,
                           static_cast<int32_t>(op.blocks.size()), 0};
    for (int32_t b : op.blocks) blocks[off++] = b;
  }
  return PA_OK;
}

pa_status pa_sched_get_stats(const pa_sched* s, pa_sched_stats* st) {
  if (s == nullptr || st == nullptr) return PA_ERR_INVALID;
  st->n_waiting = static_cast<int32_t>(s->waiting.size());
  st->n_swapped = static_cast<int32_t>(s->swapped.size());
  st->reserved = 0;
  st->n_running = static_cast<int32_t>(s->running.size());
  st->steps = s->steps;
  st->preemptions = s->preemptions;
  st->finished = s->finished;
  return PA_OK;
}

pa_status pa_sched_request(const pa_sched* s, int64_t req_id, int32_t* computed,
                           int32_t* generated, int32_t* preemptions) {
  if (s == nullptr || computed == nullptr || generated == nullptr || preemptions == nullptr)
    return PA_ERR_INVALID;
  auto it = s->reqs.find(req_id);
  if (it == s->reqs.end()) return PA_ERR_UNKNOWN_SEQ;
  *computed = it->second.computed;
  *generated = it->second.generated;
  *preemptions = it->second.preemptions;
  return PA_OK;
}

}  // extern "C"
