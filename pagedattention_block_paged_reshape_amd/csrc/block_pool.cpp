// Host block manager: physical block pool metadata, per-request block tables,
// reference counts and copy-on-write planning.  Pure C++17, no GPU runtime.
//
// Follows (page title and section):
//   - youngju.dev "vLLM inference optimization", PagedAttention section: the
//     free list holds every block id at start, allocation takes the last
//     entry, an empty list is an error, freeing appends; a request gets a new
//     block when its token count reaches a multiple of the block size.
//   - techfeed.io ngrok summary, "PagedAttention": no up-front reservation,
//     a new block only when the last one is full, blocks anywhere, a table
//     per request.
//   - media.tcdigital.jp, "memory sharing for parallel sampling": shared
//     blocks are referenced, and a new block is taken only when outputs
//     diverge (copy-on-write).
//   - techfeed.io ngrok summary, "prefix caching": requests starting with
//     the same tokens share the KV blocks of that prefix; a block is
//     identified by a hash of the previous block's hash and its own tokens,
//     so one differing token ends the sharing from its block on.
#include <algorithm>
#include <array>
#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"

namespace {

constexpr int32_t kBS = PA_BLOCK_SIZE;

struct Seq {
  std::vector<int32_t> table;
  int32_t len = 0;
};

inline int32_t ceil_div(int64_t a, int64_t b) { return static_cast<int32_t>((a + b - 1) / b); }

}  // namespace

struct pa_pool {
  int32_t num_blocks = 0;
  std::vector<int32_t> free_stack;  // bottom -> top; pop from the back
  std::vector<int32_t> ref;
  // Prefix cache (sized on first use).  A cached block is a full block whose
  // key is the hash chain of the token prefix it ends; it keeps the parent
  // hash and its tokens so that a hash hit is confirmed exactly.  A cached
  // block whose last reference goes away becomes evictable (kept, oldest
  // first in an intrusive list) instead of free.
  std::vector<uint64_t> hash_of;    // 0 = not cached
  std::vector<uint64_t> parent_of;
  std::vector<std::array<int32_t, PA_BLOCK_SIZE>> tokens_of;
  std::unordered_map<uint64_t, int32_t> cache;
  std::vector<int32_t> ev_prev, ev_next;
  int32_t ev_head = -1, ev_tail = -1, n_evictable = 0;
  std::unordered_map<int64_t, Seq> seqs;
  int64_t allocs = 0, frees = 0, cows = 0;
  int32_t shared = 0;  // blocks with ref > 1

  void ref_up(int32_t b) {
    if (++ref[b] == 2) ++shared;
  }
  // Drops one reference; true when the block became free.
  bool ref_down(int32_t b) {
    const int32_t r = --ref[b];
    if (r == 1) --shared;
    return r == 0;
  }

  bool cached(int32_t b) const { return !hash_of.empty() && hash_of[b] != 0; }
  int32_t available() const { return static_cast<int32_t>(free_stack.size()) + n_evictable; }

  void ensure_cache() {
    if (hash_of.empty()) {
      hash_of.assign(num_blocks, 0);
      parent_of.assign(num_blocks, 0);
      tokens_of.resize(num_blocks);
      ev_prev.assign(num_blocks, -1);
      ev_next.assign(num_blocks, -1);
    }
  }
  void ev_push_back(int32_t b) {
    ev_prev[b] = ev_tail;
    ev_next[b] = -1;
    if (ev_tail >= 0) ev_next[ev_tail] = b; else ev_head = b;
    ev_tail = b;
    ++n_evictable;
  }
  void ev_remove(int32_t b) {
    if (ev_prev[b] >= 0) ev_next[ev_prev[b]] = ev_next[b]; else ev_head = ev_next[b];
    if (ev_next[b] >= 0) ev_prev[ev_next[b]] = ev_prev[b]; else ev_tail = ev_prev[b];
    ev_prev[b] = ev_next[b] = -1;
    --n_evictable;
  }

  // A free block: the top of the free stack, or, when the stack is empty,
  // the block that became evictable longest ago (its cache entry dropped).
  int32_t pop() {
    int32_t b;
    if (!free_stack.empty()) {
      b = free_stack.back();
      free_stack.pop_back();
    } else {
      b = ev_head;
      ev_remove(b);
      cache.erase(hash_of[b]);
      hash_of[b] = 0;
    }
    ref[b] = 1;
    ++allocs;
    return b;
  }
  // Drops one reference (a sequence freed); a block left unreferenced goes
  // back to the free stack, or to the evictable list if it is cached.
  void release(int32_t b) {
    if (ref_down(b)) {
      if (cached(b)) ev_push_back(b); else free_stack.push_back(b);
      ++frees;
    }
  }
};

namespace {

// Hash of a full block given its parent's hash (0 for the first block):
// splitmix64 finaliser steps over the parent and each token with its slot.
inline uint64_t mix64(uint64_t x) {
  x ^= x >> 30;
  x *= 0xbf58476d1ce4e5b9ULL;
  x ^= x >> 27;
  x *= 0x94d049bb133111ebULL;
  x ^= x >> 31;
  return x;
}

uint64_t block_hash(uint64_t parent, const int32_t* t) {
  uint64_t h = mix64(parent ^ 0x9e3779b97f4a7c15ULL);
  for (int i = 0; i < PA_BLOCK_SIZE; ++i)
    h = mix64(h ^ static_cast<uint32_t>(t[i]) ^ (static_cast<uint64_t>(i + 1) << 32));
  return h == 0 ? 1 : h;
}

// Cached block holding exactly (parent, tokens), or -1.
int32_t cache_find(const pa_pool* p, uint64_t h, uint64_t parent, const int32_t* t) {
  auto it = p->cache.find(h);
  if (it == p->cache.end()) return -1;
  const int32_t b = it->second;
  if (p->parent_of[b] != parent) return -1;
  for (int i = 0; i < PA_BLOCK_SIZE; ++i)
    if (p->tokens_of[b][i] != t[i]) return -1;
  return b;
}

}  // namespace

namespace {

// Blocks an append would take, simulated without side effects.  Returns
// PA_OK and fills *need / *copies / *tokens, or an error with no effect.
pa_status plan_append(const pa_pool* p, int32_t n, const int64_t* ids, const int32_t* n_new,
                      int32_t* need, int32_t* n_copies, int64_t* n_tokens) {
  if (n < 0 || (n > 0 && (ids == nullptr || n_new == nullptr))) return PA_ERR_INVALID;
  std::unordered_map<int32_t, int32_t> sim_ref;
  std::unordered_map<int64_t, char> seen;
  seen.reserve(static_cast<size_t>(n) * 2);
  int64_t blocks = 0, copies = 0, tokens = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (n_new[i] < 0) return PA_ERR_INVALID;
    if (!seen.emplace(ids[i], 1).second) return PA_ERR_INVALID;  // duplicate id
    auto it = p->seqs.find(ids[i]);
    if (it == p->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
    const Seq& s = it->second;
    const int64_t len = s.len, add = n_new[i];
    if (len + add > static_cast<int64_t>(INT32_MAX) - kBS) return PA_ERR_INVALID;
    tokens += add;
    if (add == 0) continue;
    const int32_t off = static_cast<int32_t>(len % kBS);
    if (off != 0) {
      const int32_t blk = s.table[len / kBS];
      auto r = sim_ref.find(blk);
      int32_t cur = (r == sim_ref.end()) ? p->ref[blk] : r->second;
      if (cur > 1) {
        ++blocks;
        ++copies;
        sim_ref[blk] = cur - 1;
      }
    }
    const int64_t first_new = off == 0 ? len : len + (kBS - off);
    const int64_t end = len + add;
    if (end > first_new) blocks += (end - first_new + kBS - 1) / kBS;
  }
  if (blocks > INT32_MAX || copies > INT32_MAX) return PA_ERR_INVALID;
  *need = static_cast<int32_t>(blocks);
  *n_copies = static_cast<int32_t>(copies);
  *n_tokens = tokens;
  return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID: return "invalid argument";
    case PA_ERR_OUT_OF_BLOCKS: return "out of blocks";
    case PA_ERR_UNKNOWN_SEQ: return "unknown sequence";
    case PA_ERR_EXISTS: return "sequence exists";
    case PA_ERR_CAPACITY: return "output buffer too small";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_INTERNAL: return "internal invariant violated";
  }
  return "unknown status";
}

pa_status pa_pool_create(const pa_pool_desc* desc, pa_pool** out) {
  if (desc == nullptr || out == nullptr) return PA_ERR_INVALID;
  if (desc->block_size != kBS) return PA_ERR_INVALID;
  if (desc->num_blocks < 1 || static_cast<int64_t>(desc->num_blocks) * kBS >= (1LL << 31))
    return PA_ERR_INVALID;
  pa_pool* p = new (std::nothrow) pa_pool();
  if (p == nullptr) return PA_ERR_INTERNAL;
  const int32_t N = desc->num_blocks;
  p->num_blocks = N;
  p->ref.assign(N, 0);
  p->free_stack.resize(N);
  if (desc->free_order == nullptr) {
    for (int32_t i = 0; i < N; ++i) p->free_stack[i] = i;
  } else {
    std::vector<char> seen(N, 0);
    for (int32_t i = 0; i < N; ++i) {
      const int32_t b = desc->free_order[i];
      if (b < 0 || b >= N || seen[b]) {
        delete p;
        return PA_ERR_INVALID;
      }
      seen[b] = 1;
      p->free_stack[i] = b;
    }
  }
  *out = p;
  return PA_OK;
}

void pa_pool_destroy(pa_pool* pool) { delete pool; }

pa_status pa_seq_add(pa_pool* pool, int64_t seq_id) {
  if (pool == nullptr) return PA_ERR_INVALID;
  if (pool->seqs.count(seq_id)) return PA_ERR_EXISTS;
  pool->seqs.emplace(seq_id, Seq{});
  return PA_OK;
}

pa_status pa_seq_fork(pa_pool* pool, int64_t parent, int64_t child) {
  if (pool == nullptr) return PA_ERR_INVALID;
  auto it = pool->seqs.find(parent);
  if (it == pool->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
  if (pool->seqs.count(child)) return PA_ERR_EXISTS;
  Seq c = it->second;
  for (int32_t b : c.table) pool->ref_up(b);
  pool->seqs.emplace(child, std::move(c));
  return PA_OK;
}

pa_status pa_seq_free(pa_pool* pool, int64_t seq_id) {
  if (pool == nullptr) return PA_ERR_INVALID;
  auto it = pool->seqs.find(seq_id);
  if (it == pool->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
  for (int32_t b : it->second.table) pool->release(b);
  pool->seqs.erase(it);
  return PA_OK;
}

pa_status pa_seq_swap_out(pa_pool* pool, int64_t seq_id, int32_t* blocks, int32_t cap,
                          int32_t* n_blocks, int32_t* seq_len) {
  if (pool == nullptr || n_blocks == nullptr || seq_len == nullptr) return PA_ERR_INVALID;
  auto it = pool->seqs.find(seq_id);
  if (it == pool->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
  const Seq& s = it->second;
  const int32_t n = static_cast<int32_t>(s.table.size());
  if (n > cap) return PA_ERR_CAPACITY;
  if (n > 0 && blocks == nullptr) return PA_ERR_INVALID;
  for (int32_t i = 0; i < n; ++i) blocks[i] = s.table[i];
  *n_blocks = n;
  *seq_len = s.len;
  for (int32_t b : s.table) pool->release(b);
  pool->seqs.erase(it);
  return PA_OK;
}

pa_status pa_seq_swap_in(pa_pool* pool, int64_t seq_id, int32_t seq_len, int32_t* blocks,
                         int32_t cap, int32_t* n_blocks) {
  if (pool == nullptr || n_blocks == nullptr || seq_len < 0) return PA_ERR_INVALID;
  if (pool->seqs.count(seq_id)) return PA_ERR_EXISTS;
  const int32_t n = ceil_div(seq_len, kBS);
  if (n > cap) return PA_ERR_CAPACITY;
  if (n > 0 && blocks == nullptr) return PA_ERR_INVALID;
  if (n > pool->available()) return PA_ERR_OUT_OF_BLOCKS;
  Seq s;
  s.len = seq_len;
  s.table.reserve(n);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = pool->pop();
    s.table.push_back(b);
    blocks[i] = b;
  }
  pool->seqs.emplace(seq_id, std::move(s));
  *n_blocks = n;
  return PA_OK;
}

pa_status pa_can_append(const pa_pool* pool, int32_t n, const int64_t* seq_ids,
                        const int32_t* n_new, int32_t* blocks_needed) {
  if (pool == nullptr || blocks_needed == nullptr) return PA_ERR_INVALID;
  int32_t need = 0, copies = 0;
  int64_t tokens = 0;
  pa_status st = plan_append(pool, n, seq_ids, n_new, &need, &copies, &tokens);
  if (st != PA_OK) return st;
  *blocks_needed = need;
  return PA_OK;
}

pa_status pa_append_slots(pa_pool* pool, int32_t n, const int64_t* seq_ids,
                          const int32_t* n_new, int32_t* slot_mapping, int64_t slot_cap,
                          pa_copy* copies, int32_t copy_cap, int32_t* n_copies) {
  if (pool == nullptr || n_copies == nullptr) return PA_ERR_INVALID;
  int32_t need = 0, ncopy = 0;
  int64_t tokens = 0;
  pa_status st = plan_append(pool, n, seq_ids, n_new, &need, &ncopy, &tokens);
  if (st != PA_OK) return st;
  if (tokens > 0 && slot_mapping == nullptr) return PA_ERR_INVALID;
  if (tokens > slot_cap || ncopy > copy_cap) return PA_ERR_CAPACITY;
  if (ncopy > 0 && copies == nullptr) return PA_ERR_INVALID;
  if (need > pool->available()) return PA_ERR_OUT_OF_BLOCKS;

  int64_t t = 0;
  int32_t c = 0;
  for (int32_t i = 0; i < n; ++i) {
    Seq& s = pool->seqs.find(seq_ids[i])->second;
    for (int32_t k = 0; k < n_new[i]; ++k) {
      const int32_t pos = s.len;
      const int32_t off = pos % kBS;
      const int32_t logical = pos / kBS;
      int32_t blk;
      if (off == 0) {
        blk = pool->pop();
        s.table.push_back(blk);
      } else {
        blk = s.table[logical];
        if (pool->ref[blk] > 1) {
          const int32_t fresh = pool->pop();
          pool->ref_down(blk);
          copies[c++] = pa_copy{blk, fresh, off};
          ++pool->cows;
          s.table[logical] = fresh;
          blk = fresh;
        }
      }
      slot_mapping[t++] = blk * kBS + off;
      s.len = pos + 1;
    }
  }
  *n_copies = c;
  return (c == ncopy && t == tokens) ? PA_OK : PA_ERR_INTERNAL;
}

pa_status pa_block_tables(const pa_pool* pool, int32_t n, const int64_t* seq_ids,
                          int32_t max_blocks, int32_t* tables, int32_t* seq_lens) {
  if (pool == nullptr || n < 0 || max_blocks < 0) return PA_ERR_INVALID;
  if (n > 0 && (seq_ids == nullptr || seq_lens == nullptr)) return PA_ERR_INVALID;
  if (n > 0 && max_blocks > 0 && tables == nullptr) return PA_ERR_INVALID;
  for (int32_t i = 0; i < n; ++i) {
    auto it = pool->seqs.find(seq_ids[i]);
    if (it == pool->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
    if (static_cast<int64_t>(it->second.table.size()) > max_blocks) return PA_ERR_CAPACITY;
  }
  for (int32_t i = 0; i < n; ++i) {
    const Seq& s = pool->seqs.find(seq_ids[i])->second;
    int32_t* row = tables + static_cast<int64_t>(i) * max_blocks;
    const int32_t nb = static_cast<int32_t>(s.table.size());
    if (nb > 0) std::memcpy(row, s.table.data(), sizeof(int32_t) * nb);
    for (int32_t j = nb; j < max_blocks; ++j) row[j] = -1;
    seq_lens[i] = s.len;
  }
  return PA_OK;
}

pa_status pa_seq_table(const pa_pool* pool, int64_t seq_id, int32_t* table, int32_t cap,
                       int32_t* n_blocks, int32_t* seq_len) {
  if (pool == nullptr || n_blocks == nullptr || seq_len == nullptr) return PA_ERR_INVALID;
  auto it = pool->seqs.find(seq_id);
  if (it == pool->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
  const int32_t nb = static_cast<int32_t>(it->second.table.size());
  *n_blocks = nb;
  *seq_len = it->second.len;
  if (nb > cap) return PA_ERR_CAPACITY;
  if (nb > 0) {
    if (table == nullptr) return PA_ERR_INVALID;
    std::memcpy(table, it->second.table.data(), sizeof(int32_t) * nb);
  }
  return PA_OK;
}

int32_t pa_num_free_blocks(const pa_pool* pool) {
  return pool == nullptr ? -1 : pool->available();
}

pa_status pa_seq_add_cached(pa_pool* pool, int64_t seq_id, const int32_t* tokens,
                            int32_t n_tokens, int32_t* n_cached) {
  if (pool == nullptr || n_cached == nullptr || n_tokens < 0 ||
      (n_tokens > 0 && tokens == nullptr))
    return PA_ERR_INVALID;
  if (pool->seqs.count(seq_id)) return PA_ERR_EXISTS;
  Seq s;
  if (!pool->cache.empty()) {
    uint64_t parent = 0;
    for (int32_t i = 0; i + kBS <= n_tokens; i += kBS) {
      const uint64_t h = block_hash(parent, tokens + i);
      const int32_t b = cache_find(pool, h, parent, tokens + i);
      if (b < 0) break;
      if (pool->ref[b] == 0) pool->ev_remove(b);
      pool->ref_up(b);
      s.table.push_back(b);
      parent = h;
    }
  }
  s.len = kBS * static_cast<int32_t>(s.table.size());
  *n_cached = s.len;
  pool->seqs.emplace(seq_id, std::move(s));
  return PA_OK;
}

pa_status pa_seq_register(pa_pool* pool, int64_t seq_id, const int32_t* tokens,
                          int32_t n_tokens, int32_t* n_registered) {
  if (pool == nullptr || n_registered == nullptr || n_tokens < 0 ||
      (n_tokens > 0 && tokens == nullptr))
    return PA_ERR_INVALID;
  auto it = pool->seqs.find(seq_id);
  if (it == pool->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
  const Seq& s = it->second;
  if (n_tokens > s.len) return PA_ERR_INVALID;
  pool->ensure_cache();
  int32_t added = 0;
  uint64_t parent = 0;
  for (int32_t i = 0; i + kBS <= n_tokens; i += kBS) {
    const uint64_t h = block_hash(parent, tokens + i);
    const int32_t b = s.table[i / kBS];
    // a block keeps the key it has; a key stays with the block that has it
    if (!pool->cached(b) && pool->cache.find(h) == pool->cache.end()) {
      pool->cache.emplace(h, b);
      pool->hash_of[b] = h;
      pool->parent_of[b] = parent;
      std::copy(tokens + i, tokens + i + kBS, pool->tokens_of[b].begin());
      ++added;
    }
    parent = h;
  }
  *n_registered = added;
  return PA_OK;
}

pa_status pa_evictable_list(const pa_pool* pool, int32_t* out, int32_t cap, int32_t* n) {
  if (pool == nullptr || n == nullptr) return PA_ERR_INVALID;
  *n = pool->n_evictable;
  if (pool->n_evictable > cap) return PA_ERR_CAPACITY;
  if (pool->n_evictable > 0 && out == nullptr) return PA_ERR_INVALID;
  int32_t k = 0;
  for (int32_t b = pool->ev_head; b >= 0; b = pool->ev_next[b]) out[k++] = b;
  return PA_OK;
}

pa_status pa_ref_count(const pa_pool* pool, int32_t block, int32_t* ref) {
  if (pool == nullptr || ref == nullptr || block < 0 || block >= pool->num_blocks)
    return PA_ERR_INVALID;
  *ref = pool->ref[block];
  return PA_OK;
}

pa_status pa_pool_get_stats(const pa_pool* pool, pa_pool_stats* stats) {
  if (pool == nullptr || stats == nullptr) return PA_ERR_INVALID;
  stats->num_blocks = pool->num_blocks;
  stats->num_free = static_cast<int32_t>(pool->free_stack.size());
  stats->num_seqs = static_cast<int32_t>(pool->seqs.size());
  stats->num_shared = pool->shared;
  stats->num_evictable = pool->n_evictable;
  stats->num_cached = static_cast<int32_t>(pool->cache.size());
  stats->allocs = pool->allocs;
  stats->frees = pool->frees;
  stats->cows = pool->cows;
  return PA_OK;
}

pa_status pa_free_list(const pa_pool* pool, int32_t* out, int32_t cap, int32_t* n) {
  if (pool == nullptr || n == nullptr) return PA_ERR_INVALID;
  const int32_t nf = static_cast<int32_t>(pool->free_stack.size());
  *n = nf;
  if (nf > cap) return PA_ERR_CAPACITY;
  if (nf > 0) {
    if (out == nullptr) return PA_ERR_INVALID;
    std::memcpy(out, pool->free_stack.data(), sizeof(int32_t) * nf);
  }
  return PA_OK;
}

pa_status pa_pool_check(const pa_pool* pool) {
  if (pool == nullptr) return PA_ERR_INVALID;
  const int32_t N = pool->num_blocks;
  std::vector<int64_t> held(N, 0);
  for (const auto& kv : pool->seqs) {
    const Seq& s = kv.second;
    if (static_cast<int32_t>(s.table.size()) != ceil_div(s.len, kBS)) return PA_ERR_INTERNAL;
    for (int32_t b : s.table) {
      if (b < 0 || b >= N) return PA_ERR_INTERNAL;
      ++held[b];
    }
  }
  int64_t referenced = 0, shared = 0;
  for (int32_t b = 0; b < N; ++b) {
    if (held[b] != pool->ref[b]) return PA_ERR_INTERNAL;
    if (pool->ref[b] > 0) ++referenced;
    if (pool->ref[b] > 1) ++shared;
  }
  if (shared != pool->shared) return PA_ERR_INTERNAL;
  std::vector<char> in_free(N, 0);
  for (int32_t b : pool->free_stack) {
    if (b < 0 || b >= N || in_free[b] || pool->ref[b] != 0 || pool->cached(b))
      return PA_ERR_INTERNAL;
    in_free[b] = 1;
  }
  // evictable: unreferenced cached blocks, each once, links consistent
  int64_t evictable = 0;
  for (int32_t b = pool->ev_head, prev = -1; b >= 0; prev = b, b = pool->ev_next[b]) {
    if (b >= N || in_free[b] || pool->ref[b] != 0 || !pool->cached(b) || pool->ev_prev[b] != prev)
      return PA_ERR_INTERNAL;
    in_free[b] = 1;
    if (++evictable > N) return PA_ERR_INTERNAL;
    if (pool->ev_next[b] < 0 && pool->ev_tail != b) return PA_ERR_INTERNAL;
  }
  if (evictable != pool->n_evictable) return PA_ERR_INTERNAL;
  if (static_cast<int64_t>(pool->free_stack.size()) + evictable + referenced != N)
    return PA_ERR_INTERNAL;
  // the cache map and the per-block keys agree
  int64_t keyed = 0;
  for (int32_t b = 0; b < N; ++b) {
    if (!pool->cached(b)) continue;
    ++keyed;
    auto it = pool->cache.find(pool->hash_of[b]);
    if (it == pool->cache.end() || it->second != b) return PA_ERR_INTERNAL;
  }
  if (keyed != static_cast<int64_t>(pool->cache.size())) return PA_ERR_INTERNAL;
  return PA_OK;
}

uint64_t pa_kv_bytes_per_token(int32_t layers, int32_t num_kv_heads, int32_t head_dim,
                               int32_t dtype_bytes) {
  if (layers < 0 || num_kv_heads < 0 || head_dim < 0 || dtype_bytes < 0) return 0;
  return 2ull * static_cast<uint64_t>(layers) * static_cast<uint64_t>(num_kv_heads) *
         static_cast<uint64_t>(head_dim) * static_cast<uint64_t>(dtype_bytes);
}

}  // extern "C"
