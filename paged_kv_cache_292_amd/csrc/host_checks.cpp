// Host-side helpers around the attention calls: how many cache blocks a
// memory budget holds, and a validator of the index arrays the kernels read
// (block tables, context lengths, launch order, shared-prefix members).
//
// The kernels never fault on a bad id: an out-of-range block id reads block
// 0, a context longer than the host's bound is clamped, and a wrong member
// list is trusted.  Those inputs give a meaningless result with PKV_OK, so a
// caller debugging a scheduler can run the same arrays through
// pkv_validate_decode_inputs first (host copies; nothing on the device).
#include <cstdint>
#include <vector>

#include "pkv_internal.h"

using pkv::fail;

extern "C" int32_t pkv_blocks_for_budget(size_t bytes, int32_t num_layers, int32_t block_size,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         pkv_dtype dtype) {
  if (num_layers <= 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      (dtype != PKV_F32 && dtype != PKV_BF16))
    return -1;
  // one block id covers block_size tokens of K and of V in every layer
  uint64_t per_block = dtype == PKV_F32 ? 4 : 2;
  for (uint64_t f : {uint64_t(2), uint64_t(num_layers), uint64_t(block_size),
                     uint64_t(num_kv_heads), uint64_t(head_dim)})
    if (__builtin_mul_overflow(per_block, f, &per_block)) return 0;
  const uint64_t n = uint64_t(bytes) / per_block;
  return n > uint64_t(INT32_MAX) ? INT32_MAX : int32_t(n);
}

extern "C" pkv_status pkv_validate_decode_inputs(
    const int32_t* block_tables, int32_t num_seqs, int32_t max_blocks_per_seq,
    const int32_t* context_lens, const int32_t* seq_order, int32_t max_context_len,
    int32_t block_size, int32_t num_blocks, const int32_t* members, const int32_t* member_flag,
    int32_t num_members, int32_t prefix_tokens) {
  const char* fn = "validate_decode_inputs";
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || block_size <= 0 || num_blocks <= 0 ||
      max_context_len < 0)
    return fail(PKV_ERR_INVALID_ARG,
                "%s: num_seqs=%d max_blocks_per_seq=%d block_size=%d num_blocks=%d "
                "max_context_len=%d", fn, num_seqs, max_blocks_per_seq, block_size, num_blocks,
                max_context_len);
  if (num_seqs > 0 && (!block_tables || !context_lens))
    return fail(PKV_ERR_INVALID_ARG, "%s: NULL tables or context lengths", fn);
  const int64_t cap = int64_t(max_blocks_per_seq) * block_size;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int32_t c = context_lens[b];
    if (c < 0 || c > max_context_len || c > cap)
      return fail(PKV_ERR_INVALID_ARG,
                  "%s: context_lens[%d]=%d outside [0, min(max_context_len=%d, "
                  "max_blocks_per_seq * block_size=%lld)]", fn, b, c, max_context_len,
                  (long long)cap);
    const int32_t* row = block_tables + int64_t(b) * max_blocks_per_seq;
    const int32_t nb = (c + block_size - 1) / block_size;
    for (int32_t j = 0; j < nb; ++j)
      if (row[j] < 0 || row[j] >= num_blocks)
        return fail(PKV_ERR_INVALID_ARG,
                    "%s: block_tables[%d][%d]=%d outside the pool [0, %d) (context %d)", fn,
                    b, j, row[j], num_blocks, c);
  }
  if (seq_order) {
    std::vector<char> seen(size_t(num_seqs), 0);
    for (int32_t i = 0; i < num_seqs; ++i) {
      const int32_t s = seq_order[i];
      if (s < 0 || s >= num_seqs || seen[size_t(s)])
        return fail(PKV_ERR_INVALID_ARG, "%s: seq_order is not a permutation (entry %d = %d)",
                    fn, i, s);
      seen[size_t(s)] = 1;
    }
  }
  if (num_members < 0 || num_members > num_seqs)
    return fail(PKV_ERR_INVALID_ARG, "%s: num_members=%d outside [0, %d]", fn, num_members,
                num_seqs);
  if (num_members == 0) return pkv::ok();
  if (!members || !member_flag)
    return fail(PKV_ERR_INVALID_ARG, "%s: NULL members or member_flag", fn);
  if (prefix_tokens <= 0 || prefix_tokens % block_size != 0)
    return fail(PKV_ERR_INVALID_ARG, "%s: prefix_tokens=%d must be a positive multiple of %d",
                fn, prefix_tokens, block_size);
  const int32_t pb = prefix_tokens / block_size;
  if (pb > max_blocks_per_seq)
    return fail(PKV_ERR_INVALID_ARG, "%s: a prefix of %d blocks exceeds the tables' %d", fn, pb,
                max_blocks_per_seq);
  std::vector<char> is_member(size_t(num_seqs), 0);
  for (int32_t i = 0; i < num_members; ++i) {
    const int32_t s = members[i];
    if (s < 0 || s >= num_seqs || is_member[size_t(s)])
      return fail(PKV_ERR_INVALID_ARG, "%s: members[%d]=%d is out of range or repeated", fn, i,
                  s);
    is_member[size_t(s)] = 1;
    if (context_lens[s] <= prefix_tokens)
      return fail(PKV_ERR_INVALID_ARG,
                  "%s: member %d has context %d, not longer than the %d-token prefix", fn, s,
                  context_lens[s], prefix_tokens);
    const int32_t* row = block_tables + int64_t(s) * max_blocks_per_seq;
    const int32_t* first = block_tables + int64_t(members[0]) * max_blocks_per_seq;
    for (int32_t j = 0; j < pb; ++j)
      if (row[j] != first[j])
        return fail(PKV_ERR_INVALID_ARG,
                    "%s: member %d's block %d is %d, member %d's is %d: the prefix is not "
                    "shared", fn, s, j, row[j], members[0], first[j]);
  }
  for (int32_t b = 0; b < num_seqs; ++b)
    if ((member_flag[b] != 0) != (is_member[size_t(b)] != 0))
      return fail(PKV_ERR_INVALID_ARG, "%s: member_flag[%d]=%d but sequence %d is %sa member",
                  fn, b, member_flag[b], b, is_member[size_t(b)] ? "" : "not ");
  return pkv::ok();
}
