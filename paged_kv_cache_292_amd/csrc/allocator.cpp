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

struct pkv_allocator {
  struct Seq {
    std::vector<int32_t> blocks;  // device blocks, or host blocks while swapped
    int64_t len = 0;
    bool swapped = false;
  };
  struct Pool {
    std::deque<int32_t> free_q;
    std::vector<int32_t> refcount;
  };
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  Pool dev;   // the device cache's blocks
  Pool host;  // the host pool's blocks (empty until set)
  bool has_host = false;
  std::deque<int32_t>& free_q = dev.free_q;
  std::vector<int32_t>& refcount = dev.refcount;
  std::unordered_map<int64_t, Seq> seqs;

  int64_t blocks_for(int64_t tokens) const {
    return (tokens + block_size - 1) / block_size;
  }
  // Whether appending n > 0 tokens to s would write into a block that another
  // sequence also holds (its last block, partly filled and shared).
  bool writes_shared(const Seq& s, int64_t n) const {
    return n > 0 && s.len % block_size != 0 && refcount[s.blocks.back()] > 1;
  }
  // Appends n tokens (preconditions already checked), writing slots.
  void grow(Seq& s, int64_t n, int64_t* slots) {
    for (int64_t pos = s.len; pos < s.len + n; ++pos) {
      if (pos % block_size == 0) {
        int32_t blk = free_q.front();
        free_q.pop_front();
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
  a->refcount.assign(size_t(num_blocks), 0);
  for (int32_t i = 0; i < num_blocks; ++i) a->free_q.push_back(free_order ? free_order[i] : i);
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
  if (need > int64_t(a->free_q.size()))
    return fail(PKV_ERR_OUT_OF_BLOCKS, "append: need %lld blocks, %zu free", (long long)need,
                a->free_q.size());
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
  if (need > int64_t(a->free_q.size()))
    return fail(PKV_ERR_OUT_OF_BLOCKS, "append_cow: need %lld blocks, %zu free",
                (long long)need, a->free_q.size());
  int32_t np = 0;
  int64_t* out = slots_out;
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto& sq = a->seqs[seq_ids[i]];
    if (a->writes_shared(sq, num_tokens[i])) {
      const int32_t old = sq.blocks.back();
      const int32_t fresh = a->free_q.front();
      a->free_q.pop_front();
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
    if (--pool.refcount[size_t(b)] == 0) pool.free_q.push_back(b);
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
  a->host.refcount.assign(size_t(num_host_blocks), 0);
  for (int32_t i = 0; i < num_host_blocks; ++i)
    a->host.free_q.push_back(host_free_order ? host_free_order[i] : i);
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
  pkv_allocator::Pool& src = to_host ? a->dev : a->host;
  pkv_allocator::Pool& dst = to_host ? a->host : a->dev;
  const int64_t need = int64_t(distinct.size());
  if (need > max_pairs)
    return fail(PKV_ERR_INVALID_ARG, "%s: %lld block copies needed, room for %d", what,
                (long long)need, max_pairs);
  if (need > int64_t(dst.free_q.size()))
    return fail(PKV_ERR_OUT_OF_BLOCKS, "%s: need %lld %s blocks, %zu free", what,
                (long long)need, to_host ? "host" : "device", dst.free_q.size());
  std::unordered_map<int32_t, int32_t> moved;  // source block -> destination block
  moved.reserve(size_t(need) * 2);
  int32_t np = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto& sq = a->seqs[seq_ids[i]];
    for (int32_t& b : sq.blocks) {
      auto m = moved.find(b);
      int32_t to;
      if (m == moved.end()) {
        to = dst.free_q.front();
        dst.free_q.pop_front();
        moved.emplace(b, to);
        pairs_out[2 * np] = b;
        pairs_out[2 * np + 1] = to;
        ++np;
      } else {
        to = m->second;
      }
      dst.refcount[size_t(to)] += 1;
      if (--src.refcount[size_t(b)] == 0) src.free_q.push_back(b);
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
  return a && a->has_host ? int32_t(a->host.free_q.size()) : -1;
}

extern "C" int32_t pkv_host_block_refcount(const pkv_allocator* a, int32_t host_block_id) {
  if (!a || host_block_id < 0 || host_block_id >= int32_t(a->host.refcount.size())) return -1;
  return a->host.refcount[size_t(host_block_id)];
}

extern "C" int32_t pkv_num_free_blocks(const pkv_allocator* a) {
  return a ? int32_t(a->free_q.size()) : -1;
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
