// Host block pool: free list, per-sequence block tables, reference counts,
// fork and copy-on-write.
//
// The rules follow the pages ("vLLM PagedAttention：大模型推理的显存管理革命"
// (horeb.top), 分配策略 and 内存共享：写时复制; "vllm-pagedattention"
// (chenyuan1125.github.io), 页表真正解开的… and 一块内存，如何安全地属于多条序列;
// "vllm-paged-attention-engine" (aiqz.cc), 分页存储设计 and the allocator of
// Python 演示):
//   * n tokens occupy ceil(n / B) blocks;
//   * blocks leave from the front of the free list and come back at its end;
//   * a full last block makes growth take one more block;
//   * fork shares blocks by reference count; a write into a still-shared
//     last block copies it first; full blocks stay shared;
//   * refused requests change nothing.
// The free list is an intrusive doubly linked list over the block ids (prev /
// next arrays): push at the back, pop at the front and removal from the
// middle (a prefix-cache hit on a free block) are all O(1) without
// allocation.
//
// Optional prefix cache (automatic prefix caching: a full block is identified
// by its parent block, its tokens and extra keys such as a cache salt, so a
// new request can find and reuse the blocks of a prefix already in the cache
// and skip their prefill -- "vllm-pagedattention" (chenyuan1125.github.io),
// the passage after 一块内存，如何安全地属于多条序列 on automatic prefix caching;
// a salt keeps tenants' prefixes apart, same page, closing remarks):
//   * key of a full block = (physical id of its parent block, salt, its B
//     token ids); a lookup walks a prompt's full blocks from the first and
//     stops at the first miss;
//   * a newly full block is registered when its parent is registered (or it
//     is the first block) and no block holds its key yet;
//   * a registered block whose count reaches 0 stays cached on the free list;
//     taking it from the front evicts it (least recently released first); a
//     hit takes it back off the list;
//   * with the cache on, a sequence releases its blocks last to first, so a
//     cached block's cached descendants always sit ahead of it on the free
//     list and are evicted first: a registered key never names a parent that
//     has been evicted and reused.
#include <cstdint>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"
#include "status.h"

using pkv::fail;
using pkv::ok;

namespace {

struct Sequence {
  std::vector<int32_t> table;  // physical block ids, logical order
  int64_t len = 0;             // tokens held
  // prefix cache: the sequence's token ids are known (admitted with them and
  // grown token by token); partial holds those of its partly filled last block
  bool tracked = false;
  uint64_t salt = 0;
  std::vector<int32_t> partial;
  // swapped out: the contents live in host memory, the sequence holds no block
  bool swapped = false;
};

struct BlockKey {
  int32_t parent = -1;  // physical id of the parent block, -1 for a first block
  uint64_t salt = 0;
  std::vector<int32_t> tokens;
  bool operator==(const BlockKey& o) const {
    return parent == o.parent && salt == o.salt && tokens == o.tokens;
  }
};

struct BlockKeyHash {
  size_t operator()(const BlockKey& k) const {
    // FNV-1a over the parent id, the salt and the tokens (64-bit)
    uint64_t h = 1469598103934665603ull;
    auto mix = [&h](uint64_t x) {
      for (int i = 0; i < 8; ++i) {
        h ^= (x >> (8 * i)) & 0xffu;
        h *= 1099511628211ull;
      }
    };
    mix(uint64_t(uint32_t(k.parent)));
    mix(k.salt);
    for (int32_t t : k.tokens) mix(uint64_t(uint32_t(t)));
    return size_t(h);
  }
};

}  // namespace

struct pa_pool {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> prev, next;  // free list links, -1 at the ends
  int32_t front = -1, back = -1;
  int64_t count = 0;                // entries on the free list
  std::vector<int32_t> refcount;
  std::unordered_map<int64_t, Sequence> seqs;

  // prefix cache
  bool caching = false;
  std::unordered_map<BlockKey, int32_t, BlockKeyHash> cache;
  std::vector<BlockKey> key_of;     // key of each registered block
  std::vector<char> cached;         // block is registered
  int64_t lookups = 0, hit_blocks = 0, registered = 0, evictions = 0;

  void unlink(int32_t b) {
    const int32_t p = prev[b], n = next[b];
    if (p >= 0) next[p] = n; else front = n;
    if (n >= 0) prev[n] = p; else back = p;
    prev[b] = next[b] = -1;
    --count;
  }
  int32_t pop_front() {
    const int32_t b = front;
    unlink(b);
    if (cached[b]) {  // a cached block leaving the free list is evicted
      cache.erase(key_of[b]);
      key_of[b] = BlockKey();
      cached[b] = 0;
      ++evictions;
    }
    return b;
  }
  void push_back(int32_t b) {
    prev[b] = back;
    next[b] = -1;
    if (back >= 0) next[back] = b; else front = b;
    back = b;
    ++count;
  }
  void release(int32_t b) {
    if (--refcount[b] == 0) push_back(b);
  }
  // Gives back a sequence's blocks: in table order, or last to first with the
  // prefix cache on (descendants then reach the free list first).
  void release_table(const std::vector<int32_t>& t) {
    if (caching) {
      for (size_t i = t.size(); i-- > 0;) release(t[i]);
    } else {
      for (int32_t b : t) release(b);
    }
  }
  // Registers block b of a sequence under (parent, salt, tokens) when its
  // parent is registered (or it is a first block) and the key is new.
  void try_register(int32_t b, int32_t parent, uint64_t salt, const int32_t* tokens) {
    if (parent >= 0 && !cached[parent]) return;
    BlockKey k;
    k.parent = parent;
    k.salt = salt;
    k.tokens.assign(tokens, tokens + block_size);
    if (cache.count(k)) return;
    key_of[b] = k;
    cache.emplace(std::move(k), b);
    cached[b] = 1;
    ++registered;
  }
  int64_t slot_of(const Sequence& s, int64_t pos) const {
    return int64_t(s.table[pos / block_size]) * block_size + pos % block_size;
  }
  int64_t blocks_for(int64_t n) const { return (n + block_size - 1) / block_size; }
};

extern "C" {

pa_status pa_pool_create(int32_t num_blocks, int32_t block_size,
                         const int32_t* initial_free_order, pa_pool** out) {
  if (!out) return fail(PA_E_INVAL, "out is null");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0)
    return fail(PA_E_INVAL, "num_blocks and block_size must be positive");
  if (int64_t(num_blocks) * block_size > INT32_MAX)
    return fail(PA_E_INVAL, "num_blocks * block_size must stay below 2^31");
  pa_pool* p = new (std::nothrow) pa_pool;
  if (!p) return fail(PA_E_INVAL, "out of host memory");
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->prev.assign(num_blocks, -1);
  p->next.assign(num_blocks, -1);
  p->refcount.assign(num_blocks, 0);
  p->key_of.resize(num_blocks);
  p->cached.assign(num_blocks, 0);
  if (initial_free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = initial_free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete p;
        return fail(PA_E_INVAL, "initial_free_order is not a permutation of 0..num_blocks-1");
      }
      seen[b] = 1;
      p->push_back(b);
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) p->push_back(i);
  }
  *out = p;
  return ok();
}

void pa_pool_destroy(pa_pool* pool) { delete pool; }

pa_status pa_seq_alloc(pa_pool* pool, int64_t seq, int32_t n_tokens, int64_t* slots_out) {
  if (!pool) return fail(PA_E_INVAL, "pool is null");
  if (n_tokens < 0) return fail(PA_E_INVAL, "n_tokens must be >= 0");
  if (pool->seqs.count(seq)) return fail(PA_E_EXISTS, "sequence " + std::to_string(seq));
  const int64_t want = pool->blocks_for(n_tokens);
  if (want > pool->count)
    return fail(PA_E_NOBLOCKS, "need " + std::to_string(want) + " blocks, " +
                                   std::to_string(pool->count) + " free");
  Sequence s;
  s.table.reserve(want);
  for (int64_t i = 0; i < want; ++i) {
    int32_t b = pool->pop_front();
    pool->refcount[b] = 1;
    s.table.push_back(b);
  }
  s.len = n_tokens;
  if (slots_out)
    for (int64_t i = 0; i < n_tokens; ++i) slots_out[i] = pool->slot_of(s, i);
  pool->seqs.emplace(seq, std::move(s));
  return ok();
}

pa_status pa_seq_extend(pa_pool* pool, int64_t seq, int32_t n, int64_t* slots_out,
                        int32_t* cow_src, int32_t* cow_dst) {
  if (cow_src) *cow_src = -1;
  if (cow_dst) *cow_dst = -1;
  if (!pool) return fail(PA_E_INVAL, "pool is null");
  if (n < 0) return fail(PA_E_INVAL, "n must be >= 0");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return fail(PA_E_NOSEQ, "sequence " + std::to_string(seq));
  Sequence& s = it->second;
  if (s.swapped) return fail(PA_E_INVAL, "sequence " + std::to_string(seq) + " is swapped out");
  if (n == 0) return ok();
  const int32_t B = pool->block_size;
  // Blocks this request takes: one copy if the first token lands in a shared,
  // partly filled last block, plus the new blocks growth needs.
  const bool copy = (s.len % B != 0) && pool->refcount[s.table.back()] > 1;
  const int64_t grow = pool->blocks_for(s.len + n) - int64_t(s.table.size());
  if (grow + (copy ? 1 : 0) > pool->count)
    return fail(PA_E_NOBLOCKS, "need " + std::to_string(grow + (copy ? 1 : 0)) + " blocks, " +
                                   std::to_string(pool->count) + " free");
  s.tracked = false;  // token ids unknown from here on: no block of s is registered any more
  s.partial.clear();
  if (copy) {
    int32_t src = s.table.back();
    int32_t dst = pool->pop_front();
    pool->refcount[src] -= 1;
    pool->refcount[dst] = 1;
    s.table.back() = dst;
    if (cow_src) *cow_src = src;
    if (cow_dst) *cow_dst = dst;
  }
  for (int32_t i = 0; i < n; ++i) {
    const int64_t pos = s.len;
    if (pos % B == 0) {
      int32_t b = pool->pop_front();
      pool->refcount[b] = 1;
      s.table.push_back(b);
    }
    if (slots_out) slots_out[i] = pool->slot_of(s, pos);
    s.len = pos + 1;
  }
  return ok();
}

pa_status pa_seq_append(pa_pool* pool, int64_t seq, int64_t* slot_out, int32_t* cow_src,
                        int32_t* cow_dst) {
  int64_t slot = -1;
  pa_status st = pa_seq_extend(pool, seq, 1, &slot, cow_src, cow_dst);
  if (st == PA_OK && slot_out) *slot_out = slot;
  return st;
}

pa_status pa_seq_append_token(pa_pool* pool, int64_t seq, int32_t token, int64_t* slot_out,
                              int32_t* cow_src, int32_t* cow_dst) {
  if (!pool) return fail(PA_E_INVAL, "pool is null");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return fail(PA_E_NOSEQ, "sequence " + std::to_string(seq));
  if (it->second.swapped) return fail(PA_E_INVAL, "sequence " + std::to_string(seq) + " is swapped out");
  const bool tracked = it->second.tracked;
  std::vector<int32_t> partial = std::move(it->second.partial);
  int64_t slot = -1;
  pa_status st = pa_seq_extend(pool, seq, 1, &slot, cow_src, cow_dst);  // untracks s
  Sequence& s = pool->seqs.find(seq)->second;
  if (st != PA_OK) {
    s.tracked = tracked;
    s.partial = std::move(partial);
    return st;
  }
  if (slot_out) *slot_out = slot;
  if (tracked) {
    s.tracked = true;
    partial.push_back(token);
    if (s.len % pool->block_size == 0) {  // the last block just filled up
      const size_t nb = s.table.size();
      pool->try_register(s.table[nb - 1], nb >= 2 ? s.table[nb - 2] : -1, s.salt, partial.data());
      partial.clear();
    }
    s.partial = std::move(partial);
  }
  return ok();
}

pa_status pa_seq_fork(pa_pool* pool, int64_t parent, int64_t child) {
  if (!pool) return fail(PA_E_INVAL, "pool is null");
  auto it = pool->seqs.find(parent);
  if (it == pool->seqs.end()) return fail(PA_E_NOSEQ, "parent " + std::to_string(parent));
  if (pool->seqs.count(child)) return fail(PA_E_EXISTS, "child " + std::to_string(child));
  if (it->second.swapped) return fail(PA_E_INVAL, "parent " + std::to_string(parent) + " is swapped out");
  Sequence c = it->second;  // copy of table and length
  for (int32_t b : c.table) pool->refcount[b] += 1;
  pool->seqs.emplace(child, std::move(c));
  return ok();
}

pa_status pa_seq_free(pa_pool* pool, int64_t seq) {
  if (!pool) return fail(PA_E_INVAL, "pool is null");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return fail(PA_E_NOSEQ, "sequence " + std::to_string(seq));
  pool->release_table(it->second.table);  // empty when swapped out
  pool->seqs.erase(it);
  return ok();
}

pa_status pa_seq_swap_out(pa_pool* pool, int64_t seq, int32_t* blocks_out, int32_t cap, int32_t* n_out) {
  if (!pool || !n_out) return fail(PA_E_INVAL, "null argument");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return fail(PA_E_NOSEQ, "sequence " + std::to_string(seq));
  Sequence& s = it->second;
  if (s.swapped) return fail(PA_E_INVAL, "sequence " + std::to_string(seq) + " is already swapped out");
  const int64_t nb = int64_t(s.table.size());
  if (nb > cap || (nb > 0 && !blocks_out)) return fail(PA_E_INVAL, "blocks_out holds fewer entries than the table");
  for (int64_t i = 0; i < nb; ++i) blocks_out[i] = s.table[i];
  *n_out = int32_t(nb);
  pool->release_table(s.table);
  s.table.clear();
  s.swapped = true;
  s.tracked = false;  // blocks restored by swap-in are not registered
  s.partial.clear();
  return ok();
}

pa_status pa_seq_swap_in(pa_pool* pool, int64_t seq, int32_t* blocks_out, int32_t cap, int32_t* n_out) {
  if (!pool || !n_out) return fail(PA_E_INVAL, "null argument");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return fail(PA_E_NOSEQ, "sequence " + std::to_string(seq));
  Sequence& s = it->second;
  if (!s.swapped) return fail(PA_E_INVAL, "sequence " + std::to_string(seq) + " is not swapped out");
  const int64_t want = pool->blocks_for(s.len);
  if (want > cap || (want > 0 && !blocks_out)) return fail(PA_E_INVAL, "blocks_out holds fewer entries than the table");
  if (want > pool->count)
    return fail(PA_E_NOBLOCKS, "need " + std::to_string(want) + " blocks, " + std::to_string(pool->count) + " free");
  for (int64_t i = 0; i < want; ++i) {
    const int32_t b = pool->pop_front();
    pool->refcount[b] = 1;
    s.table.push_back(b);
    blocks_out[i] = b;
  }
  *n_out = int32_t(want);
  s.swapped = false;
  return ok();
}

pa_status pa_pool_enable_prefix_cache(pa_pool* pool) {
  if (!pool) return fail(PA_E_INVAL, "pool is null");
  if (!pool->seqs.empty()) return fail(PA_E_INVAL, "enable the prefix cache before admitting sequences");
  pool->caching = true;
  return ok();
}

pa_status pa_seq_alloc_prefix(pa_pool* pool, int64_t seq, const int32_t* tokens, int32_t n_tokens,
                              uint64_t salt, int32_t* cached_tokens_out, int64_t* slots_out) {
  if (!pool) return fail(PA_E_INVAL, "pool is null");
  if (!pool->caching) return fail(PA_E_INVAL, "the prefix cache is not enabled on this pool");
  if (n_tokens < 0 || (n_tokens > 0 && !tokens)) return fail(PA_E_INVAL, "n_tokens >= 0 and tokens required");
  if (pool->seqs.count(seq)) return fail(PA_E_EXISTS, "sequence " + std::to_string(seq));
  const int32_t B = pool->block_size;
  const int64_t nfull = n_tokens / B;
  // Longest cached prefix of whole blocks.
  std::vector<int32_t> hits;
  int64_t revive = 0;  // hits that sit on the free list
  {
    BlockKey k;
    k.salt = salt;
    for (int64_t i = 0; i < nfull; ++i) {
      k.tokens.assign(tokens + i * B, tokens + (i + 1) * B);
      ++pool->lookups;
      auto f = pool->cache.find(k);
      if (f == pool->cache.end()) break;
      hits.push_back(f->second);
      revive += pool->refcount[f->second] == 0;
      k.parent = f->second;
    }
  }
  const int64_t want = pool->blocks_for(n_tokens) - int64_t(hits.size());
  if (want > pool->count - revive)
    return fail(PA_E_NOBLOCKS, "need " + std::to_string(want) + " blocks, " +
                                   std::to_string(pool->count - revive) + " free");
  Sequence s;
  s.table.reserve(pool->blocks_for(n_tokens));
  for (int32_t b : hits) {
    if (pool->refcount[b] == 0) pool->unlink(b);
    pool->refcount[b] += 1;
    s.table.push_back(b);
  }
  for (int64_t i = 0; i < want; ++i) {
    const int32_t b = pool->pop_front();
    pool->refcount[b] = 1;
    s.table.push_back(b);
  }
  for (int64_t i = int64_t(hits.size()); i < nfull; ++i)
    pool->try_register(s.table[i], i > 0 ? s.table[i - 1] : -1, salt, tokens + i * B);
  pool->hit_blocks += int64_t(hits.size());
  s.len = n_tokens;
  s.tracked = true;
  s.salt = salt;
  s.partial.assign(tokens + nfull * B, tokens + n_tokens);
  if (slots_out)
    for (int64_t i = 0; i < n_tokens; ++i) slots_out[i] = pool->slot_of(s, i);
  if (cached_tokens_out) *cached_tokens_out = int32_t(hits.size()) * B;
  pool->seqs.emplace(seq, std::move(s));
  return ok();
}

pa_status pa_prefix_cache_stats(const pa_pool* pool, pa_prefix_stats_t* out) {
  if (!pool || !out) return fail(PA_E_INVAL, "null argument");
  pa_prefix_stats_t st{};
  st.lookups = pool->lookups;
  st.hit_blocks = pool->hit_blocks;
  st.registered = pool->registered;
  st.evictions = pool->evictions;
  st.cached_blocks = int32_t(pool->cache.size());
  *out = st;
  return ok();
}

int32_t pa_pool_block_cached(const pa_pool* pool, int32_t block) {
  if (!pool || block < 0 || block >= pool->num_blocks) return -1;
  return pool->cached[block] ? 1 : 0;
}

pa_status pa_seq_len(const pa_pool* pool, int64_t seq, int32_t* len_out) {
  if (!pool || !len_out) return fail(PA_E_INVAL, "null argument");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return fail(PA_E_NOSEQ, "sequence " + std::to_string(seq));
  if (it->second.len > INT32_MAX) return fail(PA_E_INVAL, "length exceeds int32");
  *len_out = int32_t(it->second.len);
  return ok();
}

pa_status pa_pool_block_tables(const pa_pool* pool, const int64_t* seqs, int32_t n,
                               int32_t max_blocks, int32_t* tables_out, int32_t* ctx_out) {
  if (!pool || (n > 0 && (!seqs || !tables_out))) return fail(PA_E_INVAL, "null argument");
  if (n < 0 || max_blocks <= 0) return fail(PA_E_INVAL, "n >= 0 and max_blocks > 0 required");
  for (int32_t i = 0; i < n; ++i) {
    auto it = pool->seqs.find(seqs[i]);
    if (it == pool->seqs.end()) return fail(PA_E_NOSEQ, "sequence " + std::to_string(seqs[i]));
    const Sequence& s = it->second;
    if (s.swapped) return fail(PA_E_INVAL, "sequence " + std::to_string(seqs[i]) + " is swapped out");
    if (int64_t(s.table.size()) > max_blocks)
      return fail(PA_E_INVAL, "sequence " + std::to_string(seqs[i]) + " holds " +
                                  std::to_string(s.table.size()) + " blocks > max_blocks");
    if (s.len > INT32_MAX) return fail(PA_E_INVAL, "length exceeds int32");
    int32_t* row = tables_out + int64_t(i) * max_blocks;
    for (int32_t j = 0; j < max_blocks; ++j)
      row[j] = j < int32_t(s.table.size()) ? s.table[j] : -1;
    if (ctx_out) ctx_out[i] = int32_t(s.len);
  }
  return ok();
}

pa_status pa_pool_stats(const pa_pool* pool, pa_pool_stats_t* out) {
  if (!pool || !out) return fail(PA_E_INVAL, "null argument");
  pa_pool_stats_t st{};
  st.num_blocks = pool->num_blocks;
  st.block_size = pool->block_size;
  st.free_blocks = int32_t(pool->count);
  for (int32_t c : pool->refcount) {
    st.used_blocks += c > 0;
    st.shared_blocks += c > 1;
  }
  for (const auto& kv : pool->seqs) {  // resident sequences (swapped ones hold no block)
    if (kv.second.swapped) continue;
    st.num_seqs += 1;
    st.tokens += kv.second.len;
    st.waste_tokens += int64_t(kv.second.table.size()) * pool->block_size - kv.second.len;
  }
  *out = st;
  return ok();
}

int32_t pa_pool_refcount(const pa_pool* pool, int32_t block) {
  if (!pool || block < 0 || block >= pool->num_blocks) return -1;
  return pool->refcount[block];
}

pa_status pa_pool_free_list(const pa_pool* pool, int32_t* out, int32_t cap, int32_t* n_out) {
  if (!pool || !n_out || (cap > 0 && !out) || cap < 0) return fail(PA_E_INVAL, "bad argument");
  int64_t i = 0;
  for (int32_t b = pool->front; b >= 0 && i < cap; b = pool->next[b]) out[i++] = b;
  *n_out = int32_t(pool->count);
  return ok();
}

}  // extern "C"
