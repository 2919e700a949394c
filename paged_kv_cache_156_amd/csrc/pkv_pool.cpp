// Host block pool, block-table builder and slot-mapping builder.
//
// Block lifecycle follows §3.5 of the page "Understanding KV Cache: Attention,
// P/D Disaggregation and vLLM's Paged Memory Management" (steinslab.io):
// blocks are taken from a free pool when a sequence grows, used through its
// block table, and returned when the sequence finishes. Any free block may go
// to any sequence (§3.1), so the free list is a plain FIFO of ids, optionally
// shuffled once by a seeded Fisher-Yates pass. Shared prefix blocks carry a
// reference count; writing into one is refused (copy-on-write belongs to the
// caller, page "KV Cache and Inference Optimization", section
// "PagedAttention").
//
// Pure host C++: no HIP call, usable without a GPU.
#include <pkv.h>

#include <algorithm>
#include <cstdint>
#include <deque>
#include <new>
#include <unordered_set>
#include <vector>

struct pkv_pool {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::deque<int32_t> free_list;
  std::vector<int32_t> refcount;                // per physical block
  std::vector<std::vector<int32_t>> seq_blocks;  // per sequence, logical order
  std::vector<int32_t> seq_len;
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

}  // namespace

extern "C" {

pkv_status pkv_pool_create(int32_t num_blocks, int32_t block_size, int32_t max_seqs, uint64_t seed,
                           pkv_pool** out) {
  if (!out || num_blocks <= 0 || block_size <= 0 || max_seqs <= 0) return PKV_EINVAL;
  *out = nullptr;
  pkv_pool* p = new (std::nothrow) pkv_pool;
  if (!p) return PKV_ENOMEM;
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
  *out = p;
  return PKV_OK;
}

void pkv_pool_destroy(pkv_pool* pool) { delete pool; }

pkv_status pkv_seq_grow(pkv_pool* pool, int32_t seq, int32_t new_len) {
  if (!valid_seq(pool, seq) || new_len < 0) return PKV_EINVAL;
  if (new_len < pool->seq_len[seq]) return PKV_ERANGE;
  auto& blocks = pool->seq_blocks[seq];
  const int64_t need = ceil_div(new_len, pool->block_size) - static_cast<int64_t>(blocks.size());
  if (need > static_cast<int64_t>(pool->free_list.size())) return PKV_ENOMEM;
  for (int64_t i = 0; i < need; ++i) {
    const int32_t id = pool->free_list.front();
    pool->free_list.pop_front();
    pool->refcount[id] = 1;
    blocks.push_back(id);
  }
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
    pool->refcount[s[i]] += 1;
  }
  pool->seq_len[dst] = full * pool->block_size;
  return PKV_OK;
}

pkv_status pkv_seq_free(pkv_pool* pool, int32_t seq) {
  if (!valid_seq(pool, seq)) return PKV_EINVAL;
  auto& blocks = pool->seq_blocks[seq];
  if (blocks.empty() && pool->seq_len[seq] == 0) return PKV_EINVAL;
  for (int32_t id : blocks) {
    if (pool->refcount[id] <= 0) return PKV_EINVAL;  // bookkeeping corrupted
    if (--pool->refcount[id] == 0) pool->free_list.push_back(id);
  }
  blocks.clear();
  pool->seq_len[seq] = 0;
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
  s.free_blocks = static_cast<int64_t>(pool->free_list.size());
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
