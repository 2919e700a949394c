// Host block pool, block-table builder and slot-mapping builder, with
// copy-on-write forks and a block-granular prefix cache.
//
// Block lifecycle follows §3.5 of the page "Understanding KV Cache: Attention,
// P/D Disaggregation and vLLM's Paged Memory Management" (steinslab.io):
// blocks are taken from a free pool when a sequence grows, used through its
// block table, and returned when the sequence finishes. Any free block may go
// to any sequence (§3.1), so the free list is a plain FIFO of ids, optionally
// shuffled once by a seeded Fisher-Yates pass.
//
// Sharing ("KV Cache and Inference Optimization", sections "PagedAttention"
// and "APC"): a block held by several sequences carries a reference count.
// A sequence about to write into a shared block gets a private copy first
// (copy-on-write on divergence); the pool hands the (source, destination)
// pairs to the caller, whose device copy runs before the write. Full blocks
// can be registered in a prefix cache under a key chained over the whole
// token prefix; a new request reuses cached blocks from its first block on
// and stops at the first block that misses, and only full blocks are ever
// reused. A cached block whose last holder leaves stays cached (evictable)
// until the pool runs out of never-cached free blocks; then the least
// recently released one is evicted.
//
// Pure host C++: no HIP call, usable without a GPU.
#include <pkv.h>

#include <algorithm>
#include <cstdint>
#include <deque>
#include <list>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

struct pkv_pool {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::deque<int32_t> free_list;                 // never-cached free blocks, FIFO
  std::vector<int32_t> refcount;                 // per physical block
  std::vector<std::vector<int32_t>> seq_blocks;  // per sequence, logical order
  std::vector<int32_t> seq_len;

  // prefix cache, per physical block
  std::vector<uint64_t> gen;             // bumped whenever the block is handed out fresh
  std::vector<uint8_t> cached;
  std::vector<uint64_t> key;             // chained lookup key
  std::vector<int32_t> parent_id;        // previous block of the prefix, -1 for a first block
  std::vector<uint64_t> parent_tag;      // parent's generation, or the namespace for a first block
  std::vector<std::vector<int32_t>> tokens;
  std::unordered_map<uint64_t, int32_t> index;  // key -> cached block
  std::list<int32_t> evictable;                 // cached, refcount 0, least recently released first
  std::vector<std::list<int32_t>::iterator> evict_pos;
  pkv_prefix_stats pstats{};
};

namespace {

// xorshift64* (Vigna, "An experimental exploration of Marsaglia's xorshift
// generators, scrambled", 2016): state ^= state >> 12, << 25, >> 27, output
// state * 2685821657736338717.
struct XorShift64Star {
  uint64_t s;
  explicit XorShift64Star(uint64_t seed) : s(seed ? seed : 0x9E3779B97F4A7C15ull) {}
  uint64_t next() {
    s ^= s >> 12;
    s ^= s << 25;
    s ^= s >> 27;
    return s * 2685821657736338717ull;
  }
  // uniform in [0, n) by rejection (no modulo bias)
  uint64_t below(uint64_t n) {
    const uint64_t limit = UINT64_MAX - UINT64_MAX % n;
    uint64_t x;
    do {
      x = next();
    } while (x >= limit);
    return x % n;
  }
};

bool valid_seq(const pkv_pool* p, int32_t seq) {
  return p && seq >= 0 && static_cast<size_t>(seq) < p->seq_blocks.size();
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// splitmix64 finaliser (Steele, Lea and Flood, "Fast splittable pseudorandom
// number generators", 2014): a bijective 64-bit mixer.
uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Lookup key of a full block: chained over the previous block's key, so the
// key of block i depends on every token before it. Only a hint: a hit is
// accepted after comparing the tokens and the parent exactly.
uint64_t chain_key(uint64_t prev, const int32_t* toks, int32_t n) {
  uint64_t h = mix64(prev ^ 0x6A09E667F3BCC909ull);
  for (int32_t t = 0; t < n; ++t) {
    const uint64_t tok = static_cast<uint32_t>(toks[t]);
    h = mix64(h ^ (tok + 0x9E3779B97F4A7C15ull));
  }
  return h;
}
uint64_t root_key(uint64_t ns) { return mix64(ns + 0x3C6EF372FE94F82Bull); }

size_t available(const pkv_pool* p) { return p->free_list.size() + p->evictable.size(); }

// Drop a block from the prefix cache; a block nobody holds then becomes plain free.
void uncache(pkv_pool* p, int32_t id) {
  if (!p->cached[id]) return;
  auto it = p->index.find(p->key[id]);
  if (it != p->index.end() && it->second == id) p->index.erase(it);
  p->cached[id] = 0;
  p->tokens[id].clear();
  p->tokens[id].shrink_to_fit();
  if (p->refcount[id] == 0) {
    p->evictable.erase(p->evict_pos[id]);
    p->free_list.push_back(id);
  }
}

// A fresh block for a writer: a never-cached free block if there is one, else
// the least recently released cached block (evicted). Caller checks available().
int32_t take_block(pkv_pool* p) {
  int32_t id;
  if (!p->free_list.empty()) {
    id = p->free_list.front();
    p->free_list.pop_front();
  } else {
    id = p->evictable.front();
    uncache(p, id);  // moves it to the free list
    p->free_list.pop_back();
    p->pstats.evictions += 1;
  }
  p->refcount[id] = 1;
  p->gen[id] += 1;
  return id;
}

void release(pkv_pool* p, int32_t id) {
  if (--p->refcount[id] > 0) return;
  if (p->cached[id]) {
    p->evictable.push_back(id);
    p->evict_pos[id] = std::prev(p->evictable.end());
  } else {
    p->free_list.push_back(id);
  }
}

void hold(pkv_pool* p, int32_t id) {
  if (p->refcount[id] == 0 && p->cached[id]) p->evictable.erase(p->evict_pos[id]);
  p->refcount[id] += 1;
}

// Is cached block `id` the block with these tokens after `parent` (-1: first
// block, tagged with namespace `ns`)?
bool same_block(const pkv_pool* p, int32_t id, int32_t parent, uint64_t ns, const int32_t* toks) {
  if (!p->cached[id] || p->parent_id[id] != parent) return false;
  if (p->parent_tag[id] != (parent < 0 ? ns : p->gen[parent])) return false;
  return std::equal(toks, toks + p->block_size, p->tokens[id].begin());
}

// Walk the prefix cache along `toks`; returns the leading hits (stops at the first miss).
int32_t walk_prefix(const pkv_pool* p, const int32_t* toks, int32_t n_tokens, uint64_t ns, int32_t* ids,
                    int32_t capacity) {
  const int32_t bs = p->block_size;
  uint64_t k = root_key(ns);
  int32_t parent = -1, hits = 0;
  for (int32_t i = 0; (static_cast<int64_t>(i) + 1) * bs <= n_tokens; ++i) {
    const int32_t* bt = toks + static_cast<int64_t>(i) * bs;
    k = chain_key(k, bt, bs);
    auto it = p->index.find(k);
    if (it == p->index.end() || !same_block(p, it->second, parent, ns, bt)) break;
    parent = it->second;
    if (ids && hits < capacity) ids[hits] = parent;
    ++hits;
  }
  return hits;
}

}  // namespace

extern "C" {

pkv_status pkv_pool_create(int32_t num_blocks, int32_t block_size, int32_t max_seqs, uint64_t seed,
                           pkv_pool** out) {
  if (!out || num_blocks <= 0 || block_size <= 0 || max_seqs <= 0) return PKV_EINVAL;
  *out = nullptr;
  pkv_pool* p = new (std::nothrow) pkv_pool;
  if (!p) return PKV_ENOMEM;
  try {
    p->num_blocks = num_blocks;
    p->block_size = block_size;
    std::vector<int32_t> ids(num_blocks);
    for (int32_t i = 0; i < num_blocks; ++i) ids[i] = i;
    if (seed != 0) {
      // Fisher-Yates: for i = n-1 .. 1 swap ids[i] with ids[j], j uniform in [0, i]
      XorShift64Star rng(seed);
      for (int32_t i = num_blocks - 1; i > 0; --i) {
        const int32_t j = static_cast<int32_t>(rng.below(static_cast<uint64_t>(i) + 1));
        std::swap(ids[i], ids[j]);
      }
    }
    p->free_list.assign(ids.begin(), ids.end());
    p->refcount.assign(num_blocks, 0);
    p->seq_blocks.resize(max_seqs);
    p->seq_len.assign(max_seqs, 0);
    p->gen.assign(num_blocks, 0);
    p->cached.assign(num_blocks, 0);
    p->key.assign(num_blocks, 0);
    p->parent_id.assign(num_blocks, -1);
    p->parent_tag.assign(num_blocks, 0);
    p->tokens.resize(num_blocks);
    p->evict_pos.resize(num_blocks);
  } catch (const std::bad_alloc&) {
    delete p;
    return PKV_ENOMEM;
  }
  *out = p;
  return PKV_OK;
}

void pkv_pool_destroy(pkv_pool* pool) { delete pool; }

pkv_status pkv_seq_grow(pkv_pool* pool, int32_t seq, int32_t new_len) {
  if (!valid_seq(pool, seq) || new_len < 0) return PKV_EINVAL;
  if (new_len < pool->seq_len[seq]) return PKV_ERANGE;
  auto& blocks = pool->seq_blocks[seq];
  // Growing writes new positions into the partial last block; when another
  // sequence holds it too (after a fork) or the prefix cache owns it, those
  // writes would land in shared state, so refuse (pkv_seq_append_slots is the
  // path that copies such a block first).
  const int32_t len = pool->seq_len[seq];
  if (new_len > len && len % pool->block_size != 0) {
    const int32_t last = blocks[len / pool->block_size];
    if (pool->refcount[last] > 1 || pool->cached[last]) return PKV_EBUSY;
  }
  const int64_t need = ceil_div(new_len, pool->block_size) - static_cast<int64_t>(blocks.size());
  if (need > static_cast<int64_t>(available(pool))) return PKV_ENOMEM;
  for (int64_t i = 0; i < need; ++i) blocks.push_back(take_block(pool));
  pool->seq_len[seq] = new_len;
  return PKV_OK;
}

pkv_status pkv_seq_share_prefix(pkv_pool* pool, int32_t dst, int32_t src, int32_t n_tokens) {
  if (!valid_seq(pool, dst) || !valid_seq(pool, src) || dst == src || n_tokens < 0) return PKV_EINVAL;
  if (!pool->seq_blocks[dst].empty() || pool->seq_len[dst] != 0) return PKV_EINVAL;
  if (n_tokens > pool->seq_len[src]) return PKV_ERANGE;
  const int32_t full = n_tokens / pool->block_size;
  auto& d = pool->seq_blocks[dst];
  const auto& s = pool->seq_blocks[src];
  for (int32_t i = 0; i < full; ++i) {
    d.push_back(s[i]);
    hold(pool, s[i]);
  }
  pool->seq_len[dst] = full * pool->block_size;
  return PKV_OK;
}

pkv_status pkv_seq_fork(pkv_pool* pool, int32_t dst, int32_t src) {
  if (!valid_seq(pool, dst) || !valid_seq(pool, src) || dst == src) return PKV_EINVAL;
  if (!pool->seq_blocks[dst].empty() || pool->seq_len[dst] != 0) return PKV_EINVAL;
  auto& d = pool->seq_blocks[dst];
  for (int32_t id : pool->seq_blocks[src]) {
    d.push_back(id);
    hold(pool, id);
  }
  pool->seq_len[dst] = pool->seq_len[src];
  return PKV_OK;
}

pkv_status pkv_seq_free(pkv_pool* pool, int32_t seq) {
  if (!valid_seq(pool, seq)) return PKV_EINVAL;
  auto& blocks = pool->seq_blocks[seq];
  if (blocks.empty() && pool->seq_len[seq] == 0) return PKV_EINVAL;
  for (int32_t id : blocks)
    if (pool->refcount[id] <= 0) return PKV_EINVAL;  // bookkeeping corrupted
  for (int32_t id : blocks) release(pool, id);
  blocks.clear();
  pool->seq_len[seq] = 0;
  return PKV_OK;
}

pkv_status pkv_seq_append_slots(pkv_pool* pool, const int32_t* seqs, int32_t n, int64_t* slots,
                                int32_t* copy_pairs, int32_t* n_copies) {
  if (!pool || n < 0 || !n_copies || (n > 0 && (!seqs || !slots || !copy_pairs))) return PKV_EINVAL;
  *n_copies = 0;
  const int32_t bs = pool->block_size;
  std::unordered_set<int32_t> seen;
  size_t need = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = seqs[i];
    if (!valid_seq(pool, s) || !seen.insert(s).second) return PKV_EINVAL;
    const int32_t pos = pool->seq_len[s];
    if (pos == INT32_MAX) return PKV_ERANGE;
    if (pos % bs == 0) {
      need += 1;  // a fresh block
    } else {
      const int32_t id = pool->seq_blocks[s][pos / bs];
      if (pool->cached[id]) return PKV_EBUSY;  // only full blocks are cached; a partial one never is
      need += pool->refcount[id] > 1;          // a private copy
    }
  }
  if (need > available(pool)) return PKV_ENOMEM;
  int32_t copies = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = seqs[i];
    const int32_t pos = pool->seq_len[s];
    auto& blocks = pool->seq_blocks[s];
    int32_t id;
    if (pos % bs == 0) {
      id = take_block(pool);
      blocks.push_back(id);
    } else {
      id = blocks[pos / bs];
      if (pool->refcount[id] > 1) {
        const int32_t fresh = take_block(pool);
        copy_pairs[2 * copies] = id;
        copy_pairs[2 * copies + 1] = fresh;
        ++copies;
        release(pool, id);  // stays held by the other sequences
        blocks[pos / bs] = fresh;
        id = fresh;
      }
    }
    pool->seq_len[s] = pos + 1;
    slots[i] = static_cast<int64_t>(id) * bs + pos % bs;
  }
  *n_copies = copies;
  pool->pstats.cow_copies += copies;
  return PKV_OK;
}

pkv_status pkv_prefix_register(pkv_pool* pool, int32_t seq, const int32_t* tokens, int32_t n_tokens,
                               uint64_t ns, int32_t* n_cached) {
  if (!valid_seq(pool, seq) || n_tokens < 0 || (n_tokens > 0 && !tokens)) return PKV_EINVAL;
  if (n_cached) *n_cached = 0;
  if (n_tokens > pool->seq_len[seq]) return PKV_ERANGE;
  const int32_t bs = pool->block_size;
  const auto& blocks = pool->seq_blocks[seq];
  uint64_t k = root_key(ns);
  int32_t parent = -1, done = 0;
  for (int32_t i = 0; (static_cast<int64_t>(i) + 1) * bs <= n_tokens; ++i) {
    const int32_t* bt = tokens + static_cast<int64_t>(i) * bs;
    const int32_t id = blocks[i];
    k = chain_key(k, bt, bs);
    if (pool->cached[id]) {
      if (!same_block(pool, id, parent, ns, bt)) return PKV_EINVAL;  // the block holds other tokens
    } else {
      auto it = pool->index.find(k);
      if (it != pool->index.end()) {
        const int32_t other = it->second;
        // The same content is already cached in another block: this chain
        // continues there, not through `id`, so stop registering.
        if (same_block(pool, other, parent, ns, bt)) break;
        uncache(pool, other);  // stale (its parent was evicted) or a key collision
      }
      try {
        pool->tokens[id].assign(bt, bt + bs);
        pool->index.emplace(k, id);
      } catch (const std::bad_alloc&) {
        pool->tokens[id].clear();
        return PKV_ENOMEM;
      }
      pool->cached[id] = 1;
      pool->key[id] = k;
      pool->parent_id[id] = parent;
      pool->parent_tag[id] = parent < 0 ? ns : pool->gen[parent];
    }
    parent = id;
    ++done;
  }
  if (n_cached) *n_cached = done;
  return PKV_OK;
}

pkv_status pkv_prefix_match(const pkv_pool* pool, const int32_t* tokens, int32_t n_tokens, uint64_t ns,
                            int32_t* block_ids, int32_t capacity, int32_t* n_hit) {
  if (!pool || !n_hit || n_tokens < 0 || capacity < 0 || (n_tokens > 0 && !tokens)) return PKV_EINVAL;
  *n_hit = walk_prefix(pool, tokens, n_tokens, ns, block_ids, block_ids ? capacity : 0);
  return PKV_OK;
}

pkv_status pkv_seq_adopt_prefix(pkv_pool* pool, int32_t seq, const int32_t* tokens, int32_t n_tokens, uint64_t ns,
                                int32_t* hit_tokens) {
  if (!valid_seq(pool, seq) || n_tokens < 0 || (n_tokens > 0 && !tokens)) return PKV_EINVAL;
  if (!pool->seq_blocks[seq].empty() || pool->seq_len[seq] != 0) return PKV_EINVAL;
  const int32_t bs = pool->block_size;
  std::vector<int32_t> ids(static_cast<size_t>(n_tokens / bs));
  const int32_t hits = walk_prefix(pool, tokens, n_tokens, ns, ids.data(), static_cast<int32_t>(ids.size()));
  auto& blocks = pool->seq_blocks[seq];
  for (int32_t i = 0; i < hits; ++i) {
    hold(pool, ids[i]);
    blocks.push_back(ids[i]);
  }
  pool->seq_len[seq] = hits * bs;
  pool->pstats.lookups += 1;
  pool->pstats.lookup_blocks += n_tokens / bs;
  pool->pstats.hit_blocks += hits;
  if (hit_tokens) *hit_tokens = hits * bs;
  return PKV_OK;
}

pkv_status pkv_pool_get_prefix_stats(const pkv_pool* pool, pkv_prefix_stats* out) {
  if (!pool || !out) return PKV_EINVAL;
  pkv_prefix_stats s = pool->pstats;
  s.cached_blocks = static_cast<int64_t>(pool->index.size());
  s.evictable_blocks = static_cast<int64_t>(pool->evictable.size());
  *out = s;
  return PKV_OK;
}

pkv_status pkv_seq_info(const pkv_pool* pool, int32_t seq, int32_t* length, int32_t* num_blocks,
                        int32_t* blocks, int32_t capacity) {
  if (!valid_seq(pool, seq)) return PKV_EINVAL;
  const auto& b = pool->seq_blocks[seq];
  if (length) *length = pool->seq_len[seq];
  if (num_blocks) *num_blocks = static_cast<int32_t>(b.size());
  if (blocks) {
    if (capacity < static_cast<int32_t>(b.size())) return PKV_ESMALL;
    std::copy(b.begin(), b.end(), blocks);
  }
  return PKV_OK;
}

pkv_status pkv_build_block_tables(const pkv_pool* pool, const int32_t* seqs, int32_t n, int32_t max_blocks,
                                  int32_t pad, int32_t* out) {
  if (!pool || n < 0 || max_blocks < 0 || (n > 0 && (!seqs || !out))) return PKV_EINVAL;
  for (int32_t i = 0; i < n; ++i) {
    if (!valid_seq(pool, seqs[i])) return PKV_EINVAL;
    const auto& b = pool->seq_blocks[seqs[i]];
    if (static_cast<int64_t>(b.size()) > max_blocks) return PKV_ERANGE;
    int32_t* row = out + static_cast<int64_t>(i) * max_blocks;
    std::copy(b.begin(), b.end(), row);
    std::fill(row + b.size(), row + max_blocks, pad);
  }
  return PKV_OK;
}

pkv_status pkv_build_slot_mapping(const pkv_pool* pool, const int32_t* seqs, const int32_t* positions,
                                  int32_t n, int64_t* out) {
  if (!pool || n < 0 || (n > 0 && (!seqs || !positions || !out))) return PKV_EINVAL;
  std::unordered_set<int64_t> seen;
  seen.reserve(static_cast<size_t>(n) * 2);
  const int32_t bs = pool->block_size;
  for (int32_t i = 0; i < n; ++i) {
    if (!valid_seq(pool, seqs[i])) return PKV_EINVAL;
    const int32_t pos = positions[i];
    if (pos < 0) {
      out[i] = -1;
      continue;
    }
    if (pos >= pool->seq_len[seqs[i]]) return PKV_ERANGE;
    const int32_t logical = pos / bs;
    const int32_t offset = pos % bs;
    const int32_t physical = pool->seq_blocks[seqs[i]][logical];
    if (pool->refcount[physical] > 1) return PKV_EBUSY;
    const int64_t slot = static_cast<int64_t>(physical) * bs + offset;
    if (!seen.insert(slot).second) return PKV_EBUSY;
    out[i] = slot;
  }
  return PKV_OK;
}

pkv_status pkv_slot_mapping_from_tables(const int32_t* block_tables, int32_t max_blocks, const int32_t* positions,
                                        int32_t n, int32_t block_size, int64_t* out) {
  if (n < 0 || max_blocks < 0 || block_size <= 0 || (n > 0 && (!block_tables || !positions || !out)))
    return PKV_EINVAL;
  std::unordered_set<int64_t> seen;
  seen.reserve(static_cast<size_t>(n) * 2);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t pos = positions[i];
    if (pos < 0) {
      out[i] = -1;
      continue;
    }
    const int32_t logical = pos / block_size;
    if (logical >= max_blocks) return PKV_ERANGE;
    const int32_t physical = block_tables[static_cast<int64_t>(i) * max_blocks + logical];
    if (physical < 0) return PKV_ERANGE;
    const int64_t slot = static_cast<int64_t>(physical) * block_size + pos % block_size;
    if (!seen.insert(slot).second) return PKV_EBUSY;
    out[i] = slot;
  }
  return PKV_OK;
}

pkv_status pkv_pool_get_stats(const pkv_pool* pool, pkv_pool_stats* out) {
  if (!pool || !out) return PKV_EINVAL;
  pkv_pool_stats s{};
  s.num_blocks = pool->num_blocks;
  s.free_blocks = static_cast<int64_t>(available(pool));
  for (int32_t rc : pool->refcount) {
    s.used_blocks += rc > 0;
    s.shared_blocks += rc > 1;
  }
  for (size_t i = 0; i < pool->seq_blocks.size(); ++i) {
    s.live_seqs += pool->seq_len[i] > 0;
    s.payload_tokens += pool->seq_len[i];
    s.capacity_tokens += static_cast<int64_t>(pool->seq_blocks[i].size()) * pool->block_size;
  }
  *out = s;
  return PKV_OK;
}

int64_t pkv_blocks_for(int64_t n, int32_t block_size) {
  if (n < 0 || block_size <= 0) return -1;
  return ceil_div(n, block_size);
}

int64_t pkv_empty_slots(int64_t n, int32_t block_size) {
  if (n < 0 || block_size <= 0) return -1;
  return ceil_div(n, block_size) * block_size - n;
}

pkv_status pkv_validate_tables(const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                               int32_t num_seqs, int32_t block_size, int32_t num_blocks, int32_t* bad_seq) {
  if (bad_seq) *bad_seq = -1;
  if (num_seqs < 0 || max_blocks_per_seq < 0 || block_size <= 0 || num_blocks <= 0) return PKV_EINVAL;
  if (num_seqs > 0 && (!block_tables || !context_lens)) return PKV_EINVAL;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t n = context_lens[b];
    if (n < 0 || n > static_cast<int64_t>(max_blocks_per_seq) * block_size) {
      if (bad_seq) *bad_seq = b;
      return PKV_ERANGE;
    }
    const int64_t nb = ceil_div(n, block_size);
    for (int64_t i = 0; i < nb; ++i) {
      const int32_t id = block_tables[static_cast<int64_t>(b) * max_blocks_per_seq + i];
      if (id < 0 || id >= num_blocks) {
        if (bad_seq) *bad_seq = b;
        return PKV_ERANGE;
      }
    }
  }
  return PKV_OK;
}

}  // extern "C"
