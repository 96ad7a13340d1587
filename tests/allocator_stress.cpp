// Randomised stress driver for the host block allocator, built by the CPU
// test suite with AddressSanitizer and UndefinedBehaviorSanitizer (g++, host
// code only).  It drives every allocator call through the C ABI with a
// seeded mix of operations and, after each one, checks the bookkeeping that
// the paged cache relies on:
//   - every block's reference count equals the number of resident sequences
//     whose table holds it, and free + referenced blocks = the pool;
//   - the same for the host pool (swapped-out sequences);
//   - every sequence's length and block count follow from its appends
//     (ceil(length / block_size) blocks);
//   - slots handed out by an append lie in the sequence's own blocks;
//   - calls that must fail (unknown ids, oversize requests) fail and change
//     nothing.
// Usage: allocator_stress <seed> <iterations>; exit status 0 when every
// check held.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <set>
#include <vector>

#include "pkv.h"

namespace {

int g_failures = 0;

#define CHECK(cond, ...)                                               \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "check failed at line %d: ", __LINE__);     \
      std::fprintf(stderr, __VA_ARGS__);                               \
      std::fprintf(stderr, "\n");                                      \
      if (++g_failures > 20) std::exit(1);                             \
    }                                                                  \
  } while (0)

struct Model {
  int32_t nblocks, bs, nhost;
  std::map<int64_t, int64_t> len;  // sequence -> tokens (resident or swapped)
  std::set<int64_t> swapped;
};

// Tables of the given resident sequences.
std::vector<int32_t> tables_of(pkv_allocator* a, const std::vector<int64_t>& ids, int32_t maxb) {
  std::vector<int32_t> t(ids.size() * size_t(maxb > 0 ? maxb : 1), -1);
  std::vector<int32_t> ctx(ids.size());
  if (!ids.empty()) {
    const pkv_status st = pkv_build_block_tables(a, ids.data(), int32_t(ids.size()), maxb, -1,
                                                 t.data(), ctx.data());
    CHECK(st == PKV_OK, "build_block_tables: %d (%s)", int(st), pkv_last_error());
  }
  return t;
}

void check_invariants(pkv_allocator* a, const Model& m) {
  std::vector<int64_t> resident;
  int32_t maxb = 1;
  for (const auto& kv : m.len) {
    const int64_t want_blocks = (kv.second + m.bs - 1) / m.bs;
    CHECK(pkv_seq_context_len(a, kv.first) == kv.second, "seq %lld length %lld, expected %lld",
          (long long)kv.first, (long long)pkv_seq_context_len(a, kv.first),
          (long long)kv.second);
    CHECK(pkv_seq_num_blocks(a, kv.first) == want_blocks, "seq %lld blocks %d, expected %lld",
          (long long)kv.first, pkv_seq_num_blocks(a, kv.first), (long long)want_blocks);
    const bool sw = m.swapped.count(kv.first) != 0;
    CHECK(pkv_seq_is_swapped(a, kv.first) == (sw ? 1 : 0), "seq %lld swapped flag",
          (long long)kv.first);
    if (!sw) {
      resident.push_back(kv.first);
      maxb = std::max<int32_t>(maxb, int32_t(want_blocks));
    }
  }
  std::vector<int32_t> holders(size_t(m.nblocks), 0);
  const std::vector<int32_t> t = tables_of(a, resident, maxb);
  for (size_t i = 0; i < resident.size(); ++i) {
    std::set<int32_t> own;
    for (int32_t j = 0; j < maxb; ++j) {
      const int32_t b = t[i * size_t(maxb) + size_t(j)];
      if (b < 0) continue;
      CHECK(b < m.nblocks, "block id %d outside the pool", b);
      if (b >= 0 && b < m.nblocks && own.insert(b).second) ++holders[size_t(b)];
    }
  }
  int32_t referenced = 0;
  for (int32_t b = 0; b < m.nblocks; ++b) {
    const int32_t rc = pkv_block_refcount(a, b);
    // cached prefix blocks may be shared by sequences and nothing else; a
    // free block has count 0
    CHECK(rc == holders[size_t(b)], "block %d refcount %d, held by %d sequences", b, rc,
          holders[size_t(b)]);
    if (rc > 0) ++referenced;
  }
  CHECK(pkv_num_free_blocks(a) + referenced == m.nblocks, "free %d + referenced %d != %d",
        pkv_num_free_blocks(a), referenced, m.nblocks);
  if (m.nhost > 0) {
    int32_t used = 0;
    for (int32_t h = 0; h < m.nhost; ++h) used += pkv_host_block_refcount(a, h) > 0;
    CHECK(pkv_num_free_host_blocks(a) + used == m.nhost, "host free %d + used %d != %d",
          pkv_num_free_host_blocks(a), used, m.nhost);
  }
}

}  // namespace

int main(int argc, char** argv) {
  const uint64_t seed = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 1;
  const int iters = argc > 2 ? std::atoi(argv[2]) : 2000;
  std::mt19937_64 rng(seed);
  auto rnd = [&](int64_t lo, int64_t hi) {  // inclusive
    return std::uniform_int_distribution<int64_t>(lo, hi)(rng);
  };

  Model m;
  m.nblocks = int32_t(rnd(8, 96));
  m.bs = rnd(0, 1) ? 16 : 32;
  m.nhost = int32_t(rnd(0, 64));
  std::vector<int32_t> order(size_t(m.nblocks));
  for (int32_t i = 0; i < m.nblocks; ++i) order[size_t(i)] = i;
  std::shuffle(order.begin(), order.end(), rng);
  pkv_allocator* a = nullptr;
  CHECK(pkv_allocator_create(m.nblocks, m.bs, order.data(), &a) == PKV_OK, "create");
  if (!a) return 1;
  if (m.nhost > 0) CHECK(pkv_allocator_set_host_pool(a, m.nhost, nullptr) == PKV_OK, "host pool");
  const bool prefix = rnd(0, 1) != 0;
  if (prefix) CHECK(pkv_allocator_enable_prefix_cache(a) == PKV_OK, "prefix cache");
  int64_t next_id = 1;
  // a few shared prompt stems for the prefix cache
  std::vector<std::vector<int32_t>> stems(3);
  for (auto& s : stems) {
    s.resize(size_t(rnd(1, 4 * m.bs)));
    for (auto& x : s) x = int32_t(rnd(0, 50));
  }

  auto resident_ids = [&]() {
    std::vector<int64_t> v;
    for (const auto& kv : m.len)
      if (!m.swapped.count(kv.first)) v.push_back(kv.first);
    return v;
  };
  auto pick = [&](const std::vector<int64_t>& v) { return v[size_t(rnd(0, int64_t(v.size()) - 1))]; };

  int done[12] = {};  // operations that went through, per kind
  for (int it = 0; it < iters; ++it) {
    const int op = int(rnd(0, 11));
    const std::vector<int64_t> res = resident_ids();
    if (op == 0 || m.len.empty()) {  // add
      const int64_t id = next_id++;
      CHECK(pkv_seq_add(a, id) == PKV_OK, "add");
      m.len[id] = 0;
      CHECK(pkv_seq_add(a, id) == PKV_ERR_INVALID_ARG, "re-add must fail");
      ++done[0];
    } else if (op == 1 && !res.empty()) {  // append with slots
      const int64_t id = pick(res);
      const int32_t n = int32_t(rnd(1, 3 * m.bs));
      std::vector<int64_t> slots(static_cast<size_t>(n));
      const pkv_status st = pkv_seq_append(a, id, n, slots.data());
      CHECK(st == PKV_OK || st == PKV_ERR_OUT_OF_BLOCKS || st == PKV_ERR_SHARED_WRITE,
            "append: %d", int(st));
      if (st == PKV_OK) {
        ++done[1];
        const int64_t len0 = m.len[id];
        m.len[id] += n;
        const int32_t nb = pkv_seq_num_blocks(a, id);
        std::vector<int32_t> t = tables_of(a, {id}, nb);
        for (int32_t i = 0; i < n; ++i) {
          const int64_t pos = len0 + i;
          const int64_t want = int64_t(t[size_t(pos / m.bs)]) * m.bs + pos % m.bs;
          CHECK(slots[size_t(i)] == want, "slot of position %lld: %lld, expected %lld",
                (long long)pos, (long long)slots[size_t(i)], (long long)want);
        }
      }
    } else if (op == 2 && !res.empty()) {  // batched copy-on-write append
      std::vector<int64_t> ids;
      std::vector<int32_t> counts;
      std::set<int64_t> seen;
      for (int k = 0; k < 4; ++k) {
        const int64_t id = pick(res);
        if (!seen.insert(id).second) continue;
        ids.push_back(id);
        counts.push_back(int32_t(rnd(1, m.bs)));
      }
      int64_t total = 0;
      for (int32_t c : counts) total += c;
      std::vector<int64_t> slots(static_cast<size_t>(total));
      std::vector<int64_t> pairs(2 * 8);
      int32_t npairs = -1;
      const pkv_status st = pkv_append_tokens_cow(a, ids.data(), counts.data(), int32_t(ids.size()),
                                                  slots.data(), pairs.data(), 8, &npairs);
      CHECK(st == PKV_OK || st == PKV_ERR_OUT_OF_BLOCKS || st == PKV_ERR_INVALID_ARG,
            "cow append: %d", int(st));
      if (st == PKV_OK) {
        CHECK(npairs >= 0 && npairs <= 8, "pairs %d", npairs);
        done[2] += 1 + 100 * npairs;  // appends, and copies (hundreds)
        for (size_t i = 0; i < ids.size(); ++i) m.len[ids[i]] += counts[i];
      }
    } else if (op == 3 && !res.empty()) {  // fork
      const int64_t src = pick(res);
      const int64_t dst = next_id++;
      CHECK(pkv_seq_add(a, dst) == PKV_OK, "add for fork");
      m.len[dst] = 0;
      const int64_t L = m.len[src];
      const int32_t n = rnd(0, 1) ? int32_t(L) : int32_t((L / m.bs) * m.bs);
      const pkv_status st = pkv_seq_fork_prefix(a, src, dst, n);
      CHECK(st == PKV_OK, "fork %d tokens of %lld: %d (%s)", n, (long long)L, int(st),
            pkv_last_error());
      if (st == PKV_OK) {
        m.len[dst] = n;
        ++done[3];
      }
    } else if (op == 4 && !m.len.empty()) {  // free (resident or swapped)
      auto itr = m.len.begin();
      std::advance(itr, rnd(0, int64_t(m.len.size()) - 1));
      CHECK(pkv_seq_free(a, itr->first) == PKV_OK, "free");
      m.swapped.erase(itr->first);
      m.len.erase(itr);
    } else if (op == 5 && m.nhost > 0 && !res.empty()) {  // swap out
      const int64_t id = pick(res);
      std::vector<int64_t> pairs(2 * 512);
      int32_t np = 0;
      const pkv_status st = pkv_swap_out(a, &id, 1, pairs.data(), 512, &np);
      CHECK(st == PKV_OK || st == PKV_ERR_OUT_OF_BLOCKS, "swap out: %d", int(st));
      if (st == PKV_OK) {
        m.swapped.insert(id);
        ++done[5];
      }
    } else if (op == 6 && !m.swapped.empty()) {  // swap in
      const int64_t id = *m.swapped.begin();
      std::vector<int64_t> pairs(2 * 512);
      int32_t np = 0;
      const pkv_status st = pkv_swap_in(a, &id, 1, pairs.data(), 512, &np);
      CHECK(st == PKV_OK || st == PKV_ERR_OUT_OF_BLOCKS, "swap in: %d", int(st));
      if (st == PKV_OK) {
        m.swapped.erase(id);
        ++done[6];
      }
      int64_t dummy = 0;
      if (st != PKV_OK)
        CHECK(pkv_seq_append(a, id, 1, &dummy) == PKV_ERR_SWAPPED, "append to swapped");
    } else if (op == 7) {  // prompt (prefix cache when enabled)
      const int64_t id = next_id++;
      std::vector<int32_t> toks = stems[size_t(rnd(0, 2))];
      const int64_t extra = rnd(0, 2 * m.bs);
      for (int64_t k = 0; k < extra; ++k) toks.push_back(int32_t(rnd(0, 50)));
      std::vector<int64_t> slots(toks.size());
      int32_t cached = -1;
      const pkv_status st = pkv_seq_add_prompt(a, id, toks.data(), int32_t(toks.size()),
                                               slots.data(), &cached);
      CHECK(st == PKV_OK || st == PKV_ERR_OUT_OF_BLOCKS, "add_prompt: %d", int(st));
      if (st == PKV_OK) {
        CHECK(cached >= 0 && cached < int32_t(toks.size()) && cached % m.bs == 0,
              "cached %d of %zu", cached, toks.size());
        m.len[id] = int64_t(toks.size());
        done[7] += 1 + 1000 * (cached > 0);  // prompts, and prompts with a cache hit (thousands)
      }
    } else if (op == 8 && !res.empty()) {  // decode step over all resident sequences
      std::vector<int64_t> ids = res;
      const int32_t maxb = int32_t((m.nblocks + 1) * 2);
      std::vector<int64_t> slots(ids.size());
      std::vector<int32_t> t(ids.size() * size_t(maxb)), ctx(ids.size()), ord(ids.size());
      int32_t maxc = -1;
      const pkv_status st = pkv_decode_step_prepare(a, ids.data(), int32_t(ids.size()), maxb, -1,
                                                    slots.data(), t.data(), ctx.data(), &maxc,
                                                    ord.data());
      CHECK(st == PKV_OK || st == PKV_ERR_OUT_OF_BLOCKS || st == PKV_ERR_SHARED_WRITE,
            "decode_step_prepare: %d (%s)", int(st), pkv_last_error());
      if (st == PKV_OK) {
        int32_t mc = 0;
        for (size_t i = 0; i < ids.size(); ++i) {
          m.len[ids[i]] += 1;
          CHECK(ctx[i] == m.len[ids[i]], "ctx of %lld", (long long)ids[i]);
          mc = std::max(mc, ctx[i]);
        }
        CHECK(maxc == mc, "max context %d vs %d", maxc, mc);
        ++done[8];
        for (size_t i = 1; i < ord.size(); ++i)
          CHECK(ctx[size_t(ord[i - 1])] >= ctx[size_t(ord[i])], "longest-first order");
      }
    } else if (op == 9) {  // calls that must fail and change nothing
      const int32_t free0 = pkv_num_free_blocks(a);
      int64_t s = 0;
      CHECK(pkv_seq_append(a, -12345, 1, &s) == PKV_ERR_NOT_FOUND, "append unknown");
      CHECK(pkv_seq_free(a, -12345) == PKV_ERR_NOT_FOUND, "free unknown");
      if (!res.empty()) {
        // more tokens than the pool holds: refused (into a shared last block
        // the shared-write refusal may come first)
        std::vector<int64_t> big(size_t(m.nblocks + 1) * size_t(m.bs));
        const pkv_status st = pkv_seq_append(a, res[0], int32_t(big.size()), big.data());
        CHECK(st == PKV_ERR_OUT_OF_BLOCKS || st == PKV_ERR_SHARED_WRITE, "oversize append: %d",
              int(st));
      }
      CHECK(pkv_num_free_blocks(a) == free0, "a failed call changed the pool");
    } else if (op == 10) {  // longest-first helper on random lengths
      const int n = int(rnd(0, 20));
      std::vector<int32_t> c(static_cast<size_t>(n)), o(static_cast<size_t>(n));
      for (auto& x : c) x = int32_t(rnd(0, 40));
      CHECK(pkv_longest_first_order(c.data(), n, o.data()) == PKV_OK, "order");
      std::vector<int> seen(static_cast<size_t>(n), 0);
      for (int i = 0; i < n; ++i) {
        CHECK(o[size_t(i)] >= 0 && o[size_t(i)] < n, "order entry");
        if (o[size_t(i)] >= 0 && o[size_t(i)] < n) ++seen[size_t(o[size_t(i)])];
        if (i > 0) CHECK(c[size_t(o[size_t(i - 1)])] >= c[size_t(o[size_t(i)])], "order sorted");
      }
      for (int v : seen) CHECK(v == 1, "order is a permutation");
    } else if (op == 11 && m.len.size() > 12) {  // keep the population bounded
      auto itr = m.len.begin();
      CHECK(pkv_seq_free(a, itr->first) == PKV_OK, "trim free");
      m.swapped.erase(itr->first);
      m.len.erase(itr);
    }
    check_invariants(a, m);
  }
  // free everything: the pool must be whole again (cached prefix blocks are
  // free blocks that keep their entries)
  for (const auto& kv : m.len) CHECK(pkv_seq_free(a, kv.first) == PKV_OK, "final free");
  CHECK(pkv_num_free_blocks(a) == m.nblocks, "pool not whole: %d of %d", pkv_num_free_blocks(a),
        m.nblocks);
  if (m.nhost > 0)
    CHECK(pkv_num_free_host_blocks(a) == m.nhost, "host pool not whole");
  pkv_allocator_destroy(a);
  if (g_failures) {
    std::fprintf(stderr, "seed %llu: %d failed checks\n", (unsigned long long)seed, g_failures);
    return 1;
  }
  std::printf("seed %llu: %d operations, all checks held; went through: add %d append %d "
              "cow %d fork %d swap-out %d swap-in %d prompt %d decode-step %d\n",
              (unsigned long long)seed, iters, done[0], done[1], done[2], done[3], done[5],
              done[6], done[7], done[8]);
  return 0;
}
