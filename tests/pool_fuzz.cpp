// Seeded random exercise of the host block pool through its C ABI, built by
// tests/test_host_pool_sanitized.py with AddressSanitizer and UBSan (host
// code only). Every step checks the pool's own accounting against what the
// sequences report: free + used blocks == pool size, payload and capacity
// tokens == the sums over sequences, dense tables == the block lists, and
// shared blocks counted by the pool == blocks held by two or more sequences.
// Exits non-zero (and prints the step) on the first violation.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <vector>

#include "pkv.h"

namespace {

uint64_t rng_state;
uint32_t next_u32() {  // xorshift64*
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return static_cast<uint32_t>((rng_state * 0x2545F4914F6CDD1DULL) >> 32);
}
int below(int n) { return n <= 0 ? 0 : static_cast<int>(next_u32() % static_cast<uint32_t>(n)); }

int fail(int step, const char* what) {
  std::fprintf(stderr, "pool_fuzz: step %d: %s\n", step, what);
  return 1;
}

}  // namespace

int main(int argc, char** argv) {
  const uint64_t seed = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 1;
  const int steps = argc > 2 ? std::atoi(argv[2]) : 3000;
  rng_state = seed * 0x9E3779B97F4A7C15ULL + 1;
  const int kBlocks = 96, kBs = 16, kSeqs = 12, kMaxBlocks = 64;
  pkv_pool* pool = nullptr;
  if (pkv_pool_create(kBlocks, kBs, kSeqs, seed, &pool) != PKV_OK) return fail(0, "create");
  // token streams: a small alphabet, so prefix-cache hits happen
  std::vector<std::vector<int32_t>> toks(kSeqs);
  for (int step = 1; step <= steps; ++step) {
    const int op = below(10), s = below(kSeqs), t = below(kSeqs);
    int32_t len = 0, nb = 0;
    pkv_seq_info(pool, s, &len, &nb, nullptr, 0);
    switch (op) {
      case 0:
      case 1: {  // grow
        const int32_t want = len + below(40);
        if (pkv_seq_grow(pool, s, want) == PKV_OK)
          while (static_cast<int32_t>(toks[s].size()) < want) toks[s].push_back(below(3));
        break;
      }
      case 2: {  // share a prefix / fork into an empty sequence
        int32_t tl = 0, tb = 0;
        pkv_seq_info(pool, t, &tl, &tb, nullptr, 0);
        if (len == 0 && s != t && tl > 0) {
          const bool fork = below(2) == 0;
          const int32_t n = fork ? tl : below(tl + 1);
          const pkv_status st = fork ? pkv_seq_fork(pool, s, t) : pkv_seq_share_prefix(pool, s, t, n);
          if (st == PKV_OK) {
            int32_t nl = 0, nn = 0;
            pkv_seq_info(pool, s, &nl, &nn, nullptr, 0);
            toks[s].assign(toks[t].begin(), toks[t].begin() + nl);
          }
        }
        break;
      }
      case 3:  // free
        if (len > 0) {
          if (pkv_seq_free(pool, s) != PKV_OK) return fail(step, "free of a live sequence");
          toks[s].clear();
        } else if (pkv_seq_free(pool, s) != PKV_EINVAL) {
          return fail(step, "double free accepted");
        }
        break;
      case 4:
      case 5: {  // one decode step's append for a few distinct sequences
        std::vector<int32_t> seqs;
        for (int i = 0; i < kSeqs; ++i)
          if (below(3) == 0) seqs.push_back(i);
        if (seqs.empty()) break;
        std::vector<int64_t> slots(seqs.size());
        std::vector<int32_t> pairs(2 * seqs.size());
        int32_t ncp = 0;
        if (pkv_seq_append_slots(pool, seqs.data(), static_cast<int32_t>(seqs.size()), slots.data(), pairs.data(),
                                 &ncp) == PKV_OK) {
          for (int32_t q : seqs) toks[q].push_back(below(3));
          if (ncp < 0 || ncp > static_cast<int32_t>(seqs.size())) return fail(step, "copy-pair count");
          // the new positions are writable now
          std::vector<int32_t> pos(seqs.size());
          for (size_t i = 0; i < seqs.size(); ++i) pos[i] = static_cast<int32_t>(toks[seqs[i]].size()) - 1;
          std::vector<int64_t> chk(seqs.size());
          if (pkv_build_slot_mapping(pool, seqs.data(), pos.data(), static_cast<int32_t>(seqs.size()), chk.data()) !=
              PKV_OK)
            return fail(step, "appended slots not writable");
          for (size_t i = 0; i < seqs.size(); ++i)
            if (chk[i] != slots[i]) return fail(step, "slot mapping differs from the append's slot");
        }
        break;
      }
      case 6: {  // prefix cache: register, then adopt into an empty sequence
        if (len >= kBs) pkv_prefix_register(pool, s, toks[s].data(), len, 7, nullptr);
        int32_t tl = 0, tb = 0;
        pkv_seq_info(pool, t, &tl, &tb, nullptr, 0);
        if (tl == 0 && !toks[s].empty()) {
          int32_t hit = 0;
          if (pkv_seq_adopt_prefix(pool, t, toks[s].data(), static_cast<int32_t>(toks[s].size()), 7, &hit) ==
              PKV_OK)
            toks[t].assign(toks[s].begin(), toks[s].begin() + hit);
        }
        break;
      }
      case 7: {  // slot mapping of random positions: OK, ERANGE or EBUSY, nothing else
        int32_t pos = below(len + 2) - 1;
        int64_t slot = 0;
        const pkv_status st = pkv_build_slot_mapping(pool, &s, &pos, 1, &slot);
        if (st != PKV_OK && st != PKV_ERANGE && st != PKV_EBUSY) return fail(step, "slot mapping status");
        if (st == PKV_OK && pos < 0 && slot != -1) return fail(step, "padding position not -1");
        break;
      }
      default:
        break;
    }
    // accounting checks
    pkv_pool_stats ps{};
    if (pkv_pool_get_stats(pool, &ps) != PKV_OK) return fail(step, "stats");
    if (ps.free_blocks + ps.used_blocks != kBlocks) return fail(step, "free + used != pool size");
    int64_t payload = 0, capacity = 0, live = 0;
    std::map<int32_t, int> holders;
    std::vector<int32_t> ids(kMaxBlocks * 4);
    for (int q = 0; q < kSeqs; ++q) {
      int32_t ql = 0, qn = 0;
      if (pkv_seq_info(pool, q, &ql, &qn, ids.data(), static_cast<int32_t>(ids.size())) != PKV_OK)
        return fail(step, "seq_info");
      if (ql != static_cast<int32_t>(toks[q].size())) return fail(step, "length differs from the model");
      if (qn != pkv_blocks_for(ql, kBs)) return fail(step, "block count != ceil(length / bs)");
      payload += ql;
      capacity += static_cast<int64_t>(qn) * kBs;
      live += ql > 0;
      for (int i = 0; i < qn; ++i) {
        if (ids[i] < 0 || ids[i] >= kBlocks) return fail(step, "block id out of range");
        holders[ids[i]] += 1;
      }
      if (qn <= kMaxBlocks) {
        std::vector<int32_t> row(kMaxBlocks);
        if (pkv_build_block_tables(pool, &q, 1, kMaxBlocks, -1, row.data()) != PKV_OK)
          return fail(step, "block table");
        for (int i = 0; i < kMaxBlocks; ++i)
          if (row[i] != (i < qn ? ids[i] : -1)) return fail(step, "table row differs from the block list");
        int32_t bad = -1;
        if (pkv_validate_tables(row.data(), kMaxBlocks, &ql, 1, kBs, kBlocks, &bad) != PKV_OK)
          return fail(step, "validate_tables rejects a pool-built table");
      }
    }
    int64_t shared = 0;
    for (const auto& h : holders) shared += h.second > 1;
    if (ps.payload_tokens != payload) return fail(step, "payload tokens");
    if (ps.capacity_tokens != capacity) return fail(step, "capacity tokens");
    if (ps.live_seqs != live) return fail(step, "live sequences");
    if (ps.used_blocks != static_cast<int64_t>(holders.size())) return fail(step, "used blocks");
    if (ps.shared_blocks != shared) return fail(step, "shared blocks");
  }
  pkv_pool_destroy(pool);
  std::printf("pool_fuzz: seed %llu, %d steps ok\n", static_cast<unsigned long long>(seed), steps);
  return 0;
}
