// Host block allocator for the paged KV cache.
//
// Fixed-size blocks are handed out one at a time as sequences grow, and each
// sequence keeps a table of its physical blocks in logical order ("vLLM in
// Production …", section "PagedAttention — Virtual Memory for the KV Cache";
// "Serving models with vLLM", section "How it works: PagedAttention").
// Sequences with a common prefix share physical blocks, tracked by reference
// counts ("What Is vLLM …", section "How does PagedAttention work?").
//
// Policy where the pages are silent: free blocks leave a FIFO queue that
// starts as the caller's free_order; a block whose count drops to zero joins
// its tail.  Every operation checks all of its preconditions before changing
// anything, so a failing call leaves the allocator as it was.
//
// Preemption by swapping ("What Is vLLM …", section "What is continuous
// batching in vLLM?", step 2) moves a group of sequences between the device
// pool and a second pool of blocks in host memory, managed the same way.
#include <algorithm>
#include <cstdint>
#include <deque>
#include <numeric>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pkv_internal.h"

namespace {

// Free list of one pool: first-in first-out, and a free block can also be
// taken out of the middle (a cached block shared again) without disturbing
// the order of the others.  Entries are (block, stamp); a block's current
// stamp is set when it is freed and cleared when it is taken, so entries
// left behind by a take are recognised as stale and skipped.
struct Pool {
  std::deque<std::pair<int32_t, uint64_t>> q;
  std::vector<uint64_t> stamp;  // 0 = held
  std::vector<int32_t> refcount;
  uint64_t next_stamp = 1;
  int64_t nfree = 0;

  void init(int32_t n, const int32_t* order) {
    stamp.assign(size_t(n), 0);
    refcount.assign(size_t(n), 0);
    for (int32_t i = 0; i < n; ++i) push(order ? order[i] : i);
  }
  int64_t size() const { return nfree; }
  bool is_free(int32_t b) const { return stamp[size_t(b)] != 0; }
  void push(int32_t b) {
    stamp[size_t(b)] = next_stamp++;
    q.emplace_back(b, stamp[size_t(b)]);
    ++nfree;
  }
  int32_t pop() {  // the head; the caller checked size() > 0
    while (q.front().second != stamp[size_t(q.front().first)]) q.pop_front();
    const int32_t b = q.front().first;
    q.pop_front();
    stamp[size_t(b)] = 0;
    --nfree;
    return b;
  }
  void take(int32_t b) {  // out of the middle
    stamp[size_t(b)] = 0;
    --nfree;
    if (q.size() > size_t(2 * nfree + 64)) {  // drop the stale entries
      std::deque<std::pair<int32_t, uint64_t>> keep;
      for (const auto& e : q)
        if (e.second == stamp[size_t(e.first)]) keep.push_back(e);
      q.swap(keep);
    }
  }
};

// Prefix-cache key of a full block: the block cached for the prefix before
// it (-1 for the first block) and the block's own tokens.  Because an
// entry is dropped together with every entry below it, a parent id always
// names the same prefix, so the key names the whole prefix exactly.
struct CacheKey {
  int32_t parent = -1;
  std::vector<int32_t> tokens;
  bool operator==(const CacheKey& o) const { return parent == o.parent && tokens == o.tokens; }
};
struct CacheKeyHash {
  size_t operator()(const CacheKey& k) const {
    uint64_t h = 0x9E3779B97F4A7C15ull ^ uint64_t(uint32_t(k.parent));
    for (int32_t t : k.tokens) {
      h ^= uint64_t(uint32_t(t)) + 0x9E3779B97F4A7C15ull + (h << 6) + (h >> 2);
      h *= 0xBF58476D1CE4E5B9ull;
    }
    return size_t(h ^ (h >> 31));
  }
};

}  // namespace

struct pkv_allocator {
  struct Seq {
    std::vector<int32_t> blocks;  // device blocks, or host blocks while swapped
    int64_t len = 0;
    bool swapped = false;
  };
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  Pool dev;   // the device cache's blocks
  Pool host;  // the host pool's blocks (empty until set)
  bool has_host = false;
  std::vector<int32_t>& refcount = dev.refcount;
  std::unordered_map<int64_t, Seq> seqs;

  // prefix cache (off until enabled)
  bool cache_on = false;
  std::unordered_map<CacheKey, int32_t, CacheKeyHash> cache;
  std::vector<CacheKey> block_key;               // valid where block_cached
  std::vector<char> block_cached;
  std::vector<std::vector<int32_t>> children;    // cached blocks keyed under this one
  int64_t lookups = 0;
  int64_t hits = 0;

  int64_t blocks_for(int64_t tokens) const {
    return (tokens + block_size - 1) / block_size;
  }
  // Whether appending n > 0 tokens to s would write into a block that another
  // sequence also holds (its last block, partly filled and shared).
  bool writes_shared(const Seq& s, int64_t n) const {
    return n > 0 && s.len % block_size != 0 && refcount[s.blocks.back()] > 1;
  }
  // Drops block b's cache entry and every entry below it.
  void evict(int32_t b) {
    std::vector<int32_t> stack{b};
    while (!stack.empty()) {
      const int32_t x = stack.back();
      stack.pop_back();
      if (!block_cached[size_t(x)]) continue;
      const int32_t parent = block_key[size_t(x)].parent;
      if (parent >= 0) {
        auto& sib = children[size_t(parent)];
        sib.erase(std::remove(sib.begin(), sib.end(), x), sib.end());
      }
      cache.erase(block_key[size_t(x)]);
      block_key[size_t(x)] = CacheKey{};
      block_cached[size_t(x)] = 0;
      for (int32_t c : children[size_t(x)]) stack.push_back(c);
      children[size_t(x)].clear();
    }
  }
  // Hands out the device free list's head; a block that still held a cached
  // prefix is about to receive other tokens and loses its entry.
  int32_t take_free() {
    const int32_t b = dev.pop();
    if (cache_on && block_cached[size_t(b)]) evict(b);
    return b;
  }
  // Appends n tokens (preconditions already checked), writing slots.
  void grow(Seq& s, int64_t n, int64_t* slots) {
    for (int64_t pos = s.len; pos < s.len + n; ++pos) {
      if (pos % block_size == 0) {
        int32_t blk = take_free();
        refcount[blk] += 1;
        s.blocks.push_back(blk);
      }
      if (slots)
        *slots++ = int64_t(s.blocks[pos / block_size]) * block_size + pos % block_size;
    }
    s.len += n;
  }
};

using pkv::fail;

extern "C" pkv_status pkv_allocator_create(int32_t num_blocks, int32_t block_size,
                                           const int32_t* free_order,
                                           pkv_allocator** out) {
  if (!out) return fail(PKV_ERR_INVALID_ARG, "allocator_create: out is NULL");
  *out = nullptr;
  if (num_blocks < 0 || block_size <= 0)
    return fail(PKV_ERR_INVALID_ARG, "allocator_create: num_blocks=%d block_size=%d",
                num_blocks, block_size);
  if (free_order) {
    std::vector<char> seen(size_t(num_blocks), 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[size_t(b)])
        return fail(PKV_ERR_INVALID_ARG,
                    "allocator_create: free_order is not a permutation (entry %d = %d)", i, b);
      seen[size_t(b)] = 1;
    }
  }
  auto* a = new (std::nothrow) pkv_allocator();
  if (!a) return fail(PKV_ERR_INVALID_ARG, "allocator_create: out of host memory");
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  a->dev.init(num_blocks, free_order);
  *out = a;
  return pkv::ok();
}

extern "C" void pkv_allocator_destroy(pkv_allocator* a) { delete a; }

extern "C" pkv_status pkv_seq_add(pkv_allocator* a, int64_t seq_id) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "seq_add: NULL allocator");
  if (a->seqs.count(seq_id)) return fail(PKV_ERR_INVALID_ARG, "seq_add: sequence %lld exists", (long long)seq_id);
  a->seqs.emplace(seq_id, pkv_allocator::Seq{});
  return pkv::ok();
}

extern "C" pkv_status pkv_seq_fork_prefix(pkv_allocator* a, int64_t src, int64_t dst,
                                          int32_t num_tokens) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "seq_fork_prefix: NULL allocator");
  auto is = a->seqs.find(src);
  auto id = a->seqs.find(dst);
  if (is == a->seqs.end() || id == a->seqs.end())
    return fail(PKV_ERR_NOT_FOUND, "seq_fork_prefix: unknown sequence (%lld -> %lld)",
                (long long)src, (long long)dst);
  if (is->second.swapped || id->second.swapped)
    return fail(PKV_ERR_SWAPPED, "seq_fork_prefix: sequence %lld is swapped out",
                (long long)(is->second.swapped ? src : dst));
  const auto& s = is->second;
  bool whole = num_tokens % a->block_size == 0 || num_tokens == s.len;
  if (src == dst || num_tokens < 0 || num_tokens > s.len || !whole || id->second.len != 0)
    return fail(PKV_ERR_INVALID_ARG,
                "seq_fork_prefix: %d tokens of %lld (length %lld) into %lld: needs whole blocks "
                "or the whole source, and an empty destination",
                num_tokens, (long long)src, (long long)s.len, (long long)dst);
  int64_t nb = a->blocks_for(num_tokens);
  auto& d = id->second;
  d.blocks.assign(s.blocks.begin(), s.blocks.begin() + nb);
  for (int32_t b : d.blocks) a->refcount[size_t(b)] += 1;
  d.len = num_tokens;
  return pkv::ok();
}

extern "C" pkv_status pkv_seq_append(pkv_allocator* a, int64_t seq_id, int32_t num_tokens,
                                     int64_t* slots_out) {
  return pkv_append_tokens(a, &seq_id, &num_tokens, 1, slots_out);
}

extern "C" pkv_status pkv_append_tokens(pkv_allocator* a, const int64_t* seq_ids,
                                        const int32_t* num_tokens, int32_t num_seqs,
                                        int64_t* slots_out) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "append: NULL allocator");
  if (num_seqs < 0 || (num_seqs > 0 && (!seq_ids || !num_tokens)))
    return fail(PKV_ERR_INVALID_ARG, "append: bad batch (num_seqs=%d)", num_seqs);
  // Check everything first.  A sequence may appear several times; later
  // entries see the growth of earlier ones.
  std::unordered_map<int64_t, int64_t> pending;  // seq -> tokens added so far in this call
  int64_t need = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end())
      return fail(PKV_ERR_NOT_FOUND, "append: unknown sequence %lld", (long long)seq_ids[i]);
    if (it->second.swapped)
      return fail(PKV_ERR_SWAPPED, "append: sequence %lld is swapped out", (long long)seq_ids[i]);
    if (num_tokens[i] < 0)
      return fail(PKV_ERR_INVALID_ARG, "append: negative token count %d", num_tokens[i]);
    const auto& s = it->second;
    int64_t& extra = pending[seq_ids[i]];
    if (extra == 0 && a->writes_shared(s, num_tokens[i]))
      return fail(PKV_ERR_SHARED_WRITE,
                  "append: last block of sequence %lld is shared (copy it first)",
                  (long long)seq_ids[i]);
    int64_t before = s.len + extra;
    need += a->blocks_for(before + num_tokens[i]) - a->blocks_for(before);
    extra += num_tokens[i];
  }
  if (need > a->dev.size())
    return fail(PKV_ERR_OUT_OF_BLOCKS, "append: need %lld blocks, %lld free", (long long)need,
                (long long)a->dev.size());
  int64_t* out = slots_out;
  for (int32_t i = 0; i < num_seqs; ++i) {
    a->grow(a->seqs[seq_ids[i]], num_tokens[i], out);
    if (out) out += num_tokens[i];
  }
  return pkv::ok();
}

extern "C" pkv_status pkv_append_tokens_cow(pkv_allocator* a, const int64_t* seq_ids,
                                            const int32_t* num_tokens, int32_t num_seqs,
                                            int64_t* slots_out, int64_t* copy_pairs_out,
                                            int32_t max_pairs, int32_t* num_pairs_out) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "append_cow: NULL allocator");
  if (num_seqs < 0 || max_pairs < 0 || (num_seqs > 0 && (!seq_ids || !num_tokens)) ||
      (max_pairs > 0 && !copy_pairs_out))
    return fail(PKV_ERR_INVALID_ARG, "append_cow: bad arguments");
  // Check everything first, simulating repeated ids in order: a sequence's
  // shared, partly filled last block is copied once, before its first write.
  struct Pending {
    int64_t extra = 0;
    bool copied = false;
  };
  std::unordered_map<int64_t, Pending> pending;
  int64_t need = 0;
  int32_t pairs = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end())
      return fail(PKV_ERR_NOT_FOUND, "append_cow: unknown sequence %lld", (long long)seq_ids[i]);
    if (it->second.swapped)
      return fail(PKV_ERR_SWAPPED, "append_cow: sequence %lld is swapped out",
                  (long long)seq_ids[i]);
    if (num_tokens[i] < 0)
      return fail(PKV_ERR_INVALID_ARG, "append_cow: negative token count %d", num_tokens[i]);
    const auto& sq = it->second;
    Pending& pd = pending[seq_ids[i]];
    if (pd.extra == 0 && !pd.copied && a->writes_shared(sq, num_tokens[i])) {
      pd.copied = true;
      ++need;
      ++pairs;
    }
    const int64_t before = sq.len + pd.extra;
    need += a->blocks_for(before + num_tokens[i]) - a->blocks_for(before);
    pd.extra += num_tokens[i];
  }
  if (pairs > max_pairs)
    return fail(PKV_ERR_INVALID_ARG, "append_cow: %d copies needed, room for %d", pairs,
                max_pairs);
  if (need > a->dev.size())
    return fail(PKV_ERR_OUT_OF_BLOCKS, "append_cow: need %lld blocks, %lld free",
                (long long)need, (long long)a->dev.size());
  int32_t np = 0;
  int64_t* out = slots_out;
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto& sq = a->seqs[seq_ids[i]];
    if (a->writes_shared(sq, num_tokens[i])) {
      const int32_t old = sq.blocks.back();
      const int32_t fresh = a->take_free();
      a->refcount[size_t(fresh)] += 1;
      a->refcount[size_t(old)] -= 1;  // still > 0: another sequence holds it
      sq.blocks.back() = fresh;
      copy_pairs_out[2 * np] = old;
      copy_pairs_out[2 * np + 1] = fresh;
      ++np;
    }
    a->grow(sq, num_tokens[i], out);
    if (out) out += num_tokens[i];
  }
  if (num_pairs_out) *num_pairs_out = np;
  return pkv::ok();
}

extern "C" pkv_status pkv_seq_free(pkv_allocator* a, int64_t seq_id) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "seq_free: NULL allocator");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end())
    return fail(PKV_ERR_NOT_FOUND, "seq_free: unknown sequence %lld", (long long)seq_id);
  auto& pool = it->second.swapped ? a->host : a->dev;
  for (int32_t b : it->second.blocks) {
    if (--pool.refcount[size_t(b)] == 0) pool.push(b);
  }
  a->seqs.erase(it);
  return pkv::ok();
}

extern "C" pkv_status pkv_build_block_tables(const pkv_allocator* a, const int64_t* seq_ids,
                                             int32_t num_seqs, int32_t max_blocks_per_seq,
                                             int32_t pad_value, int32_t* tables_out,
                                             int32_t* context_lens_out) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "build_block_tables: NULL allocator");
  if (num_seqs < 0 || max_blocks_per_seq < 0 ||
      (num_seqs > 0 && (!seq_ids || (!tables_out && max_blocks_per_seq > 0))))
    return fail(PKV_ERR_INVALID_ARG, "build_block_tables: bad arguments");
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end())
      return fail(PKV_ERR_NOT_FOUND, "build_block_tables: unknown sequence %lld",
                  (long long)seq_ids[i]);
    if (it->second.swapped)
      return fail(PKV_ERR_SWAPPED, "build_block_tables: sequence %lld is swapped out",
                  (long long)seq_ids[i]);
    if (int64_t(it->second.blocks.size()) > max_blocks_per_seq)
      return fail(PKV_ERR_INVALID_ARG, "build_block_tables: sequence %lld has %zu blocks > %d",
                  (long long)seq_ids[i], it->second.blocks.size(), max_blocks_per_seq);
    if (it->second.len > INT32_MAX)
      return fail(PKV_ERR_INVALID_ARG, "build_block_tables: sequence too long");
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const auto& s = a->seqs.at(seq_ids[i]);
    int32_t* row = tables_out + int64_t(i) * max_blocks_per_seq;
    size_t n = s.blocks.size();
    for (size_t j = 0; j < n; ++j) row[j] = s.blocks[j];
    for (int64_t j = int64_t(n); j < max_blocks_per_seq; ++j) row[j] = pad_value;
    if (context_lens_out) context_lens_out[i] = int32_t(s.len);
  }
  return pkv::ok();
}

extern "C" pkv_status pkv_allocator_set_host_pool(pkv_allocator* a, int32_t num_host_blocks,
                                                  const int32_t* host_free_order) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "set_host_pool: NULL allocator");
  if (a->has_host) return fail(PKV_ERR_INVALID_ARG, "set_host_pool: the host pool is already set");
  if (num_host_blocks < 0)
    return fail(PKV_ERR_INVALID_ARG, "set_host_pool: num_host_blocks=%d", num_host_blocks);
  if (host_free_order) {
    std::vector<char> seen(size_t(num_host_blocks), 0);
    for (int32_t i = 0; i < num_host_blocks; ++i) {
      const int32_t b = host_free_order[i];
      if (b < 0 || b >= num_host_blocks || seen[size_t(b)])
        return fail(PKV_ERR_INVALID_ARG,
                    "set_host_pool: host_free_order is not a permutation (entry %d = %d)", i, b);
      seen[size_t(b)] = 1;
    }
  }
  a->host.init(num_host_blocks, host_free_order);
  a->has_host = true;
  return pkv::ok();
}

namespace {

// Moves a group of sequences from one pool to the other (swap-out: device to
// host; swap-in: host to device).  Each distinct source block of the group
// gets one destination block, taken from the destination pool's free queue
// in visiting order (sequence by sequence, table order); every holder in the
// group moves its reference, and a source block whose count drops to zero
// rejoins its pool's free queue.  All preconditions are checked first.
pkv_status move_group(pkv_allocator* a, const int64_t* seq_ids, int32_t num_seqs,
                      int64_t* pairs_out, int32_t max_pairs, int32_t* num_pairs_out,
                      bool to_host) {
  const char* what = to_host ? "swap_out" : "swap_in";
  if (!a) return fail(PKV_ERR_INVALID_ARG, "%s: NULL allocator", what);
  if (!a->has_host) return fail(PKV_ERR_INVALID_ARG, "%s: the allocator has no host pool", what);
  if (num_seqs < 0 || max_pairs < 0 || (num_seqs > 0 && !seq_ids) ||
      (max_pairs > 0 && !pairs_out))
    return fail(PKV_ERR_INVALID_ARG, "%s: bad arguments", what);
  std::unordered_set<int64_t> seen;
  for (int32_t i = 0; i < num_seqs; ++i)
    if (!seen.insert(seq_ids[i]).second)
      return fail(PKV_ERR_INVALID_ARG, "%s: sequence %lld listed twice", what,
                  (long long)seq_ids[i]);
  std::unordered_set<int32_t> distinct;
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end())
      return fail(PKV_ERR_NOT_FOUND, "%s: unknown sequence %lld", what, (long long)seq_ids[i]);
    if (it->second.swapped == to_host)
      return fail(PKV_ERR_SWAPPED, "%s: sequence %lld is %s", what, (long long)seq_ids[i],
                  to_host ? "already swapped out" : "not swapped out");
    for (int32_t b : it->second.blocks) distinct.insert(b);
  }
  Pool& src = to_host ? a->dev : a->host;
  Pool& dst = to_host ? a->host : a->dev;
  const int64_t need = int64_t(distinct.size());
  if (need > max_pairs)
    return fail(PKV_ERR_INVALID_ARG, "%s: %lld block copies needed, room for %d", what,
                (long long)need, max_pairs);
  if (need > dst.size())
    return fail(PKV_ERR_OUT_OF_BLOCKS, "%s: need %lld %s blocks, %lld free", what,
                (long long)need, to_host ? "host" : "device", (long long)dst.size());
  std::unordered_map<int32_t, int32_t> moved;  // source block -> destination block
  moved.reserve(size_t(need) * 2);
  int32_t np = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto& sq = a->seqs[seq_ids[i]];
    for (int32_t& b : sq.blocks) {
      auto m = moved.find(b);
      int32_t to;
      if (m == moved.end()) {
        to = to_host ? dst.pop() : a->take_free();
        moved.emplace(b, to);
        pairs_out[2 * np] = b;
        pairs_out[2 * np + 1] = to;
        ++np;
      } else {
        to = m->second;
      }
      dst.refcount[size_t(to)] += 1;
      if (--src.refcount[size_t(b)] == 0) src.push(b);
      b = to;
    }
    sq.swapped = to_host;
  }
  if (num_pairs_out) *num_pairs_out = np;
  return pkv::ok();
}

}  // namespace

extern "C" pkv_status pkv_swap_out(pkv_allocator* a, const int64_t* seq_ids, int32_t num_seqs,
                                   int64_t* pairs_out, int32_t max_pairs,
                                   int32_t* num_pairs_out) {
  return move_group(a, seq_ids, num_seqs, pairs_out, max_pairs, num_pairs_out, true);
}

extern "C" pkv_status pkv_swap_in(pkv_allocator* a, const int64_t* seq_ids, int32_t num_seqs,
                                  int64_t* pairs_out, int32_t max_pairs,
                                  int32_t* num_pairs_out) {
  return move_group(a, seq_ids, num_seqs, pairs_out, max_pairs, num_pairs_out, false);
}

extern "C" int32_t pkv_seq_is_swapped(const pkv_allocator* a, int64_t seq_id) {
  if (!a) return -1;
  auto it = a->seqs.find(seq_id);
  return it == a->seqs.end() ? -1 : (it->second.swapped ? 1 : 0);
}

extern "C" int32_t pkv_num_free_host_blocks(const pkv_allocator* a) {
  return a && a->has_host ? int32_t(a->host.size()) : -1;
}

extern "C" int32_t pkv_host_block_refcount(const pkv_allocator* a, int32_t host_block_id) {
  if (!a || host_block_id < 0 || host_block_id >= int32_t(a->host.refcount.size())) return -1;
  return a->host.refcount[size_t(host_block_id)];
}

extern "C" pkv_status pkv_allocator_enable_prefix_cache(pkv_allocator* a) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "enable_prefix_cache: NULL allocator");
  if (a->cache_on) return fail(PKV_ERR_INVALID_ARG, "enable_prefix_cache: already enabled");
  a->cache_on = true;
  a->block_key.assign(size_t(a->num_blocks), CacheKey{});
  a->block_cached.assign(size_t(a->num_blocks), 0);
  a->children.assign(size_t(a->num_blocks), {});
  return pkv::ok();
}

extern "C" pkv_status pkv_seq_add_prompt(pkv_allocator* a, int64_t seq_id, const int32_t* tokens,
                                         int32_t num_tokens, int64_t* slots_out,
                                         int32_t* num_cached_out) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "seq_add_prompt: NULL allocator");
  if (num_tokens < 0 || (num_tokens > 0 && !tokens))
    return fail(PKV_ERR_INVALID_ARG, "seq_add_prompt: bad prompt (num_tokens=%d)", num_tokens);
  if (a->seqs.count(seq_id))
    return fail(PKV_ERR_INVALID_ARG, "seq_add_prompt: sequence %lld exists", (long long)seq_id);
  const int64_t n = num_tokens;
  const int64_t bs = a->block_size;
  // the longest cached run of full blocks at the start, never the last token
  std::vector<int32_t> hit;
  CacheKey key;
  if (a->cache_on) {
    key.tokens.resize(size_t(bs));
    for (int64_t j = 0; j < (n > 0 ? (n - 1) / bs : 0); ++j) {
      std::copy(tokens + j * bs, tokens + (j + 1) * bs, key.tokens.begin());
      auto it = a->cache.find(key);
      if (it == a->cache.end()) break;
      hit.push_back(it->second);
      key.parent = it->second;
    }
  }
  int64_t revived = 0;
  for (int32_t b : hit) revived += a->dev.is_free(b) ? 1 : 0;
  const int64_t need = a->blocks_for(n) - int64_t(hit.size());
  if (need > a->dev.size() - revived)
    return fail(PKV_ERR_OUT_OF_BLOCKS, "seq_add_prompt: need %lld blocks, %lld free",
                (long long)need, (long long)(a->dev.size() - revived));
  for (int32_t b : hit) {
    if (a->dev.is_free(b)) a->dev.take(b);
    a->refcount[size_t(b)] += 1;
  }
  auto& sq = a->seqs[seq_id];
  sq.blocks = hit;
  sq.len = int64_t(hit.size()) * bs;
  a->grow(sq, n - sq.len, slots_out);
  if (a->cache_on) {
    a->lookups += n > 0 ? (n - 1) / bs : 0;
    a->hits += int64_t(hit.size());
    key.parent = hit.empty() ? -1 : hit.back();
    for (int64_t j = int64_t(hit.size()); j < n / bs; ++j) {
      std::copy(tokens + j * bs, tokens + (j + 1) * bs, key.tokens.begin());
      auto it = a->cache.find(key);
      if (it == a->cache.end()) {  // enter the block; an existing entry keeps its block
        const int32_t b = sq.blocks[size_t(j)];
        it = a->cache.emplace(key, b).first;
        a->block_key[size_t(b)] = key;
        a->block_cached[size_t(b)] = 1;
        if (key.parent >= 0) a->children[size_t(key.parent)].push_back(b);
      }
      key.parent = it->second;
    }
  }
  if (num_cached_out) *num_cached_out = int32_t(hit.size() * size_t(bs));
  return pkv::ok();
}

extern "C" pkv_status pkv_prefix_cache_stats(const pkv_allocator* a, int64_t* lookups,
                                             int64_t* hits, int32_t* num_cached_blocks) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "prefix_cache_stats: NULL allocator");
  if (lookups) *lookups = a->lookups;
  if (hits) *hits = a->hits;
  if (num_cached_blocks) *num_cached_blocks = int32_t(a->cache.size());
  return pkv::ok();
}

extern "C" int32_t pkv_num_free_blocks(const pkv_allocator* a) {
  return a ? int32_t(a->dev.size()) : -1;
}

extern "C" int32_t pkv_block_refcount(const pkv_allocator* a, int32_t block_id) {
  if (!a || block_id < 0 || block_id >= a->num_blocks) return -1;
  return a->refcount[size_t(block_id)];
}

extern "C" int64_t pkv_seq_context_len(const pkv_allocator* a, int64_t seq_id) {
  if (!a) return -1;
  auto it = a->seqs.find(seq_id);
  return it == a->seqs.end() ? -1 : it->second.len;
}

extern "C" int32_t pkv_seq_num_blocks(const pkv_allocator* a, int64_t seq_id) {
  if (!a) return -1;
  auto it = a->seqs.find(seq_id);
  return it == a->seqs.end() ? -1 : int32_t(it->second.blocks.size());
}

extern "C" pkv_status pkv_decode_step_prepare(pkv_allocator* a, const int64_t* seq_ids,
                                              int32_t num_seqs, int32_t max_blocks_per_seq,
                                              int32_t pad_value, int64_t* slots_out,
                                              int32_t* tables_out, int32_t* context_lens_out,
                                              int32_t* max_context_len_out, int32_t* order_out) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "decode_step_prepare: NULL allocator");
  if (num_seqs < 0 || (num_seqs > 0 && (!seq_ids || !slots_out || !tables_out)))
    return fail(PKV_ERR_INVALID_ARG, "decode_step_prepare: bad arguments");
  // every sequence must exist, appear once and fit its grown table before
  // anything changes
  std::unordered_set<int64_t> seen;
  seen.reserve(size_t(num_seqs) * 2);
  for (int32_t i = 0; i < num_seqs; ++i) {
    if (!seen.insert(seq_ids[i]).second)
      return fail(PKV_ERR_INVALID_ARG, "decode_step_prepare: sequence %lld listed twice",
                  (long long)seq_ids[i]);
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end())
      return fail(PKV_ERR_NOT_FOUND, "decode_step_prepare: unknown sequence %lld",
                  (long long)seq_ids[i]);
    if (it->second.swapped)
      return fail(PKV_ERR_SWAPPED, "decode_step_prepare: sequence %lld is swapped out",
                  (long long)seq_ids[i]);
    if (a->blocks_for(it->second.len + 1) > max_blocks_per_seq)
      return fail(PKV_ERR_INVALID_ARG,
                  "decode_step_prepare: sequence %lld would need more than %d blocks",
                  (long long)seq_ids[i], max_blocks_per_seq);
  }
  static thread_local std::vector<int32_t> ones;
  if (int32_t(ones.size()) < num_seqs) ones.assign(size_t(num_seqs), 1);
  pkv_status st = pkv_append_tokens(a, seq_ids, ones.data(), num_seqs, slots_out);
  if (st != PKV_OK) return st;
  st = pkv_build_block_tables(a, seq_ids, num_seqs, max_blocks_per_seq, pad_value, tables_out,
                              context_lens_out);
  if (st != PKV_OK) return st;  // cannot happen: checked above
  if (max_context_len_out) {
    // from the allocator's own state: the output arrays may be pinned,
    // uncached host memory that is slow to read back
    int64_t mx = 0;
    for (int32_t i = 0; i < num_seqs; ++i) {
      const int64_t len = a->seqs.find(seq_ids[i])->second.len;
      mx = len > mx ? len : mx;
    }
    *max_context_len_out = int32_t(mx);
  }
  if (order_out) {
    static thread_local std::vector<int32_t> lens;
    lens.resize(size_t(num_seqs));
    for (int32_t i = 0; i < num_seqs; ++i)
      lens[size_t(i)] = int32_t(a->seqs.find(seq_ids[i])->second.len);
    return pkv_longest_first_order(lens.data(), num_seqs, order_out);
  }
  return pkv::ok();
}

extern "C" pkv_status pkv_longest_first_order(const int32_t* context_lens, int32_t n,
                                              int32_t* order_out) {
  if (n < 0 || (n > 0 && (!context_lens || !order_out)))
    return fail(PKV_ERR_INVALID_ARG, "longest_first_order: bad arguments");
  std::iota(order_out, order_out + n, 0);
  std::stable_sort(order_out, order_out + n,
                   [&](int32_t x, int32_t y) { return context_lens[x] > context_lens[y]; });
  return pkv::ok();
}

// Sequences of a batch that share a prefix: those whose first
// prefix_tokens / block_size blocks are the same physical blocks ("What Is
// vLLM …", section "How does PagedAttention work?", memory-sharing step), with
// at least one private token after it.  Sequences are grouped by that list
// of blocks; the largest group (of at least two) is reported, the one met
// first in seq_ids order on a tie.
extern "C" pkv_status pkv_shared_prefix_members(const pkv_allocator* a, const int64_t* seq_ids,
                                                int32_t num_seqs, int32_t prefix_tokens,
                                                int32_t* members_out, int32_t* member_flag_out,
                                                int32_t* num_members_out) {
  const char* fn = "shared_prefix_members";
  if (!a || num_seqs < 0 || !num_members_out ||
      (num_seqs > 0 && (!seq_ids || !members_out || !member_flag_out)))
    return fail(PKV_ERR_INVALID_ARG, "%s: bad arguments", fn);
  if (prefix_tokens <= 0 || prefix_tokens % a->block_size != 0)
    return fail(PKV_ERR_INVALID_ARG, "%s: prefix_tokens=%d must be a positive multiple of %d",
                fn, prefix_tokens, a->block_size);
  std::unordered_set<int64_t> seen;
  std::vector<const pkv_allocator::Seq*> seq(static_cast<size_t>(num_seqs), nullptr);
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end())
      return fail(PKV_ERR_NOT_FOUND, "%s: unknown sequence %lld", fn, (long long)seq_ids[i]);
    if (it->second.swapped)
      return fail(PKV_ERR_SWAPPED, "%s: sequence %lld is swapped out", fn,
                  (long long)seq_ids[i]);
    if (!seen.insert(seq_ids[i]).second)
      return fail(PKV_ERR_INVALID_ARG, "%s: sequence %lld listed twice", fn,
                  (long long)seq_ids[i]);
    seq[size_t(i)] = &it->second;
  }
  const size_t pb = size_t(prefix_tokens / a->block_size);
  // group id of each eligible sequence: the index of the first sequence
  // with the same prefix blocks
  std::vector<int32_t> group(size_t(num_seqs), -1);
  std::vector<int32_t> count(size_t(num_seqs), 0);
  std::vector<int32_t> heads;  // first sequence of each group, in order
  for (int32_t i = 0; i < num_seqs; ++i) {
    const auto& s = *seq[size_t(i)];
    if (s.len <= prefix_tokens) continue;
    for (int32_t h : heads) {
      const auto& t = *seq[size_t(h)];
      if (std::equal(s.blocks.begin(), s.blocks.begin() + std::ptrdiff_t(pb), t.blocks.begin())) {
        group[size_t(i)] = h;
        break;
      }
    }
    if (group[size_t(i)] < 0) {
      group[size_t(i)] = i;
      heads.push_back(i);
    }
    ++count[size_t(group[size_t(i)])];
  }
  int32_t best = -1;
  for (int32_t h : heads)
    if (count[size_t(h)] >= 2 && (best < 0 || count[size_t(h)] > count[size_t(best)])) best = h;
  int32_t n = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const bool m = best >= 0 && group[size_t(i)] == best;
    member_flag_out[i] = m ? 1 : 0;
    if (m) members_out[n++] = i;
  }
  *num_members_out = n;
  return pkv::ok();
}
