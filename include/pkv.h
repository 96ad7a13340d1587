/*
 * pkv.h — C ABI of libpkv, PagedAttention decode for AMD MI355X (gfx950).
 *
 * The operations follow the pages' statement of the method:
 *   - "vLLM in Production — PagedAttention, Continuous Batching, and
 *     OpenAI-Compatible LLM Serving" (datasops.com), section
 *     "PagedAttention — Virtual Memory for the KV Cache": each sequence's
 *     keys and values live in fixed-size blocks anywhere in GPU memory; a
 *     per-sequence block table maps logical blocks to physical ones and grows
 *     one block at a time as tokens arrive;
 *   - "Serving models with vLLM" (allaboutaibydeep.pages.dev), section
 *     "How it works: PagedAttention": blocks are allocated on demand, only a
 *     sequence's last block is partly empty, and sequences with a common
 *     prefix can point at the same physical blocks;
 *   - "What Is vLLM: The Fast Inference Engine for Large Language Models"
 *     (fp8.co), section "How does PagedAttention work?": attention for a
 *     position looks up the physical block holding that position and indexes
 *     into it; shared blocks are tracked by reference counts.
 *
 * Conventions for every call:
 *   - Device pointers are owned by the caller (typically torch tensors on the
 *     current device) and must stay valid until the work queued on `stream`
 *     has finished.  `stream` is a hipStream_t (NULL = the null stream).
 *   - GPU calls are asynchronous on `stream`; they never allocate, free or
 *     synchronize device memory.
 *   - Every call returns a status.  Arguments are validated on the host
 *     before anything is launched; a failing call launches nothing and leaves
 *     all state unchanged.  pkv_last_error() gives a message for the last
 *     non-OK status returned on the calling thread.
 *   - Element types: PKV_F32 (float32) or PKV_BF16 (bfloat16).  q, caches,
 *     new keys/values and the attention output all share one element type.
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1,  /* a pointer, size or id is out of range          */
  PKV_ERR_UNSUPPORTED = -2,  /* valid but not built (head_dim, block size ...) */
  PKV_ERR_OUT_OF_BLOCKS = -3,/* the pool has too few free blocks               */
  PKV_ERR_NOT_FOUND = -4,    /* unknown sequence id                            */
  PKV_ERR_SHARED_WRITE = -5, /* append into a block another sequence holds     */
  PKV_ERR_WORKSPACE = -6,    /* workspace missing or smaller than required     */
  PKV_ERR_HIP = -7,          /* a HIP runtime call or kernel launch failed     */
  PKV_ERR_SWAPPED = -8       /* the sequence is (or is not) swapped out         */
} pkv_status;

typedef enum pkv_dtype { PKV_F32 = 0, PKV_BF16 = 1 } pkv_dtype;

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* pkv_last_error(void);
/* Library version string. */
const char* pkv_version(void);

/* ------------------------------------------------------------------------
 * Cache write: store new tokens' keys and values through a slot mapping.
 *
 * A sequence's cache fills one token at a time, each token's K/V going into
 * the block its table names for that position ("vLLM in Production …",
 * section "PagedAttention — Virtual Memory for the KV Cache": blocks are
 * allocated on demand as tokens arrive and may sit anywhere in memory;
 * "What Is vLLM …", section "How does PagedAttention work?": a position
 * lives in the physical block the table gives for it, at its offset inside
 * that block).  Token i's rows key[i] and value[i] (each [num_kv_heads, head_dim]) go to
 * row (slot % block_size) of physical block (slot / block_size), where
 * slot = slot_mapping[i] was handed out by the block allocator for that
 * token's position.  A negative slot marks a padding token and is skipped;
 * so is a slot >= num_blocks * block_size.  Slots in one call must be
 * distinct (the allocator never repeats one).  All other cache bytes are
 * left untouched; the copy is bit-exact.
 *
 * key, value    device, [num_tokens, num_kv_heads, head_dim], rows of token i
 *               start at i * key_token_stride / i * value_token_stride
 *               elements (pass num_kv_heads * head_dim when contiguous);
 *               the [num_kv_heads, head_dim] part is contiguous.
 * k_cache,
 * v_cache       device, [num_blocks, block_size, num_kv_heads, head_dim],
 *               contiguous, written in place.
 * slot_mapping  device, int64 [num_tokens].
 * Supported: head_dim in {64, 128}; num_tokens >= 0 (0 launches nothing).
 * ---------------------------------------------------------------------- */
pkv_status pkv_kv_reshape_and_cache(const void* key, const void* value,
                                    void* k_cache, void* v_cache,
                                    const int64_t* slot_mapping,
                                    int32_t num_tokens, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size,
                                    int32_t num_blocks,
                                    int64_t key_token_stride,
                                    int64_t value_token_stride,
                                    pkv_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * Paged decode attention: one query token per sequence.
 *
 * Each new token attends to the keys and values of every earlier token of
 * its sequence and to its own ("vLLM in Production …", section "The KV Cache
 * and the 60–80% Memory Tax"); those K/V rows sit in fixed-size blocks
 * anywhere in the pool, reached through the sequence's block table (same
 * page, section "PagedAttention — Virtual Memory for the KV Cache"; "What Is
 * vLLM …", section "How does PagedAttention work?": the block holding a
 * position is looked up, then indexed into).
 *
 * For sequence b and query head h (kv head g = h / (num_q_heads /
 * num_kv_heads)): out[b, h] = softmax(scale * K_b q[b, h]) V_b, where K_b
 * and V_b are the context_lens[b] rows of kv head g gathered through the
 * block table: token t sits in block block_tables[b, t / block_size] at
 * row t % block_size.  Every token attends to its whole context (no other
 * mask).  context_lens[b] == 0 gives an all-zero output row.  Softmax and
 * the weighted sum accumulate in float32; the output is rounded to the
 * element type (nearest-even for bf16).
 *
 * With partition_size > 0 each sequence is cut into partitions of that
 * many tokens, handled in parallel, then merged by a log-sum-exp reduction;
 * the result equals the single-pass one up to rounding.
 * partition_size == 0: single pass per sequence.
 * partition_size == PKV_PARTITION_AUTO (-1): the library chooses from
 * max_context_len and the kernel that runs (pkv_decode_partition_size tells
 * the choice).  pkv_decode_workspace_bytes(..., PKV_PARTITION_AUTO, ...)
 * covers every automatic choice of every kernel, so the workspace does not
 * depend on the decode-path setting.
 *
 * out           device, [num_seqs, num_q_heads, head_dim].
 * q             device, [num_seqs, num_q_heads, head_dim].
 * k_cache,
 * v_cache       device, [num_blocks, block_size, num_kv_heads, head_dim].
 * block_tables  device, int32 [num_seqs, max_blocks_per_seq]; entries past
 *               a sequence's last block are never read; ids must lie in
 *               [0, num_blocks) (an id outside reads block 0 rather than
 *               faulting, and the result is meaningless).
 * context_lens  device, int32 [num_seqs]; each value is clamped to
 *               [0, min(max_context_len, max_blocks_per_seq * block_size)].
 * seq_order     device, int32 [num_seqs] or NULL: the order in which the
 *               sequences' work is started, a permutation of 0..num_seqs-1
 *               (pkv_longest_first_order gives longest first, which keeps
 *               the longest sequences from finishing last).  It changes only
 *               the speed; NULL = index order.  An entry outside the range
 *               is treated as its own index (no out-of-bounds access, but
 *               a non-permutation leaves some rows unwritten).
 * max_context_len  host-side upper bound of context_lens (sizes the grid).
 * workspace     device scratch of at least pkv_decode_workspace_bytes(...)
 *               bytes when partitions are used (may be NULL otherwise).
 * Supported: head_dim in {64, 128}; block_size in {16, 32};
 *            num_q_heads a multiple of num_kv_heads, the group
 *            G = num_q_heads / num_kv_heads being 1..16 for bf16 and
 *            1, 2, 4 or 8 for f32; partition_size a multiple of block_size
 *            (or 0 / -1); num_seqs <= 65535.
 * Kernels (PKV_PATH_AUTO): f32, and bf16 with G <= 2, run on the vector
 * ALUs: fp32 dot products (bf16 pairs widened by v_dot2), fp32 softmax and
 * fp32 weighted sum of V; rounding only in the fp32 arithmetic and the
 * output store.  bf16 with G >= 3 runs on the matrix cores: q.K on bf16
 * MFMA with fp32 accumulation; the softmax weights p (fp32, each at most
 * 2^8 times the weight of the running maximum) are rounded to bf16 for the
 * P.V product, a bf16 MFMA accumulating in fp32, while the softmax sum adds
 * the unrounded fp32 p.  Rounding p (relative error at most 2^-9 per weight)
 * changes an output element by at most 2^-9 * sum_t p_t |v_t| / sum_t p_t
 * <= 2^-9 * max_t |v_t|, before the output's own rounding (2^-9 relative
 * for bf16).  See pkv_set_decode_path for forcing one kernel.
 * ---------------------------------------------------------------------- */
#define PKV_PARTITION_AUTO (-1)

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int32_t max_context_len,
                                  int32_t partition_size, pkv_dtype dtype);

/* The partition size the library uses for these arguments (resolves AUTO);
 * 0 means single pass. */
int32_t pkv_decode_partition_size(int32_t num_seqs, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int32_t max_context_len,
                                  int32_t partition_size, pkv_dtype dtype);

/* Streaming-read reference for the roofline (no step of the method): reads
 * `bytes` of device memory at `src` once with 16-byte non-temporal loads,
 * the loads the decode kernels stream K and V with, and no other work.  The
 * rate it reaches on a buffer far larger than the caches is the read
 * ceiling the decode kernels are compared with.  `out` (device, uint32
 * [workgroups], caller-owned) receives one XOR of the 32-bit words each
 * workgroup read; the XOR of all entries is the XOR of every word of the
 * buffer.  `workgroups` (1 .. 2^20) sets the grid of 256-thread workgroups.
 * src must be 16-byte aligned and bytes a multiple of 16; errors are
 * reported before any launch.  Asynchronous on `stream`. */
pkv_status pkv_stream_read(const void* src, size_t bytes, uint32_t* out, int32_t workgroups,
                           void* stream);

/* Which decode kernel later calls use, process-wide (for tests and
 * benchmarks): PKV_PATH_AUTO (default) picks the matrix-core kernel for bf16
 * groups of 4..16 query heads and the vector kernel otherwise; PKV_PATH_VALU
 * forces the vector kernel where it is built (G = 1, 2, 4, 8); PKV_PATH_MFMA
 * forces the matrix-core kernel for every bf16 group of 2..16.  Not
 * thread-safe against concurrent decode calls. */
#define PKV_PATH_AUTO 0
#define PKV_PATH_VALU 1
#define PKV_PATH_MFMA 2
pkv_status pkv_set_decode_path(int32_t path);
int32_t pkv_get_decode_path(void);

pkv_status pkv_paged_attention_decode(void* out, const void* q,
                                      const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables,
                                      int32_t max_blocks_per_seq,
                                      const int32_t* context_lens,
                                      const int32_t* seq_order,
                                      int32_t max_context_len, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size,
                                      int32_t num_blocks, float scale,
                                      int32_t partition_size, void* workspace,
                                      size_t workspace_bytes, pkv_dtype dtype,
                                      void* stream);

/* Decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): pkv_paged_attention_decode with the
 * split-K partials kept in a static device array of
 * PKV_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends.  The call itself allocates and frees nothing.
 * Arguments, results and errors as pkv_paged_attention_decode; a call whose
 * partitions need more than PKV_NOALLOC_SCRATCH_BYTES (partition_size and
 * pkv_decode_workspace_bytes tell the need) is refused with
 * PKV_ERR_WORKSPACE before any launch.  The array's address on a device is
 * looked up on the first call with that device current; `stream` must
 * belong to the current device.  Every call on one GPU shares its array:
 * calls that overlap on one GPU (concurrent streams, or host threads on
 * different streams) race and give wrong results; calls in one stream are
 * ordered and safe.  Nothing in the array needs to start at any value. */
#define PKV_NOALLOC_SCRATCH_BYTES (64u << 20)
pkv_status pkv_paged_attention_decode_noalloc(void* out, const void* q,
                                              const void* k_cache, const void* v_cache,
                                              const int32_t* block_tables,
                                              int32_t max_blocks_per_seq,
                                              const int32_t* context_lens,
                                              const int32_t* seq_order,
                                              int32_t max_context_len, int32_t num_seqs,
                                              int32_t num_q_heads, int32_t num_kv_heads,
                                              int32_t head_dim, int32_t block_size,
                                              int32_t num_blocks, float scale,
                                              int32_t partition_size, pkv_dtype dtype,
                                              void* stream);

/* Paged decode for a batch in which some sequences share a prefix ("What Is
 * vLLM …", section "How does PagedAttention work?", the memory-sharing
 * step: sequences that share a prefix point at the same physical blocks).
 * The result is that of pkv_paged_attention_decode (equal up to rounding):
 * a member's context is split into a first partition of prefix_tokens
 * tokens and then partitions of max(2048, prefix_tokens) tokens, every other
 * context into partitions of max(2048, prefix_tokens) tokens, all merged by
 * log-sum-exp.  Partition 0 of every member, the shared prefix, is computed
 * once for tiles of 16 / G members (G = num_q_heads / num_kv_heads): each
 * K/V row of the prefix is read once per tile instead of once per member.
 * The tiles run first in the same launch as the other partitions, all tiles
 * of one kv head on one XCD (with the kv heads in eights), so that the
 * prefix comes from HBM about once per kv head.  With num_members = 0 the
 * call is pkv_paged_attention_decode with partition_size = prefix_tokens.
 * pkv_shared_prefix_members derives members and member_flag from the
 * allocator's tables, and pkv_validate_decode_inputs checks them.
 * members       device int32 [num_members]: the sharing sequences (distinct
 *               indices into the batch).  Each member's first
 *               prefix_tokens / block_size table entries must be the same
 *               blocks, and its context must be longer than prefix_tokens;
 *               otherwise its result is undefined (no access leaves the
 *               tables, caches or workspace).
 * member_flag   device int32 [num_seqs]: nonzero exactly for the members.
 * prefix_tokens the shared length: a multiple of block_size and of 16, at
 *               most max_context_len.
 * workspace     at least pkv_decode_workspace_bytes(..., partition_size =
 *               prefix_tokens, ...) bytes.
 * Supported: bf16, grouped query heads on the matrix-core kernel (G 2..16);
 * PKV_ERR_UNSUPPORTED otherwise.  Other arguments and errors as
 * pkv_paged_attention_decode.
 */
pkv_status pkv_paged_attention_decode_shared_prefix(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* seq_order, int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    const int32_t* members, const int32_t* member_flag, int32_t num_members,
    int32_t prefix_tokens, void* workspace, size_t workspace_bytes, pkv_dtype dtype,
    void* stream);

/* pkv_paged_attention_decode_shared_prefix and, in the same launch, the
 * next step's upload of pkv_paged_attention_decode_step: next_bytes from
 * next_src_host (pinned, device-mapped host memory) to next_dst (device) by
 * the workgroups of one extra grid row dispatched before the prefix tiles
 * ("vLLM in Production …", section "Continuous Batching Keeps the GPU
 * Full": the batch is re-formed at every step).  next_dst must not overlap
 * anything the call reads or writes; next_src_host must not change until
 * the call has completed.  next_bytes = 0: exactly the shared-prefix call.
 * next_bytes and both addresses must be multiples of 16, the batch 1 ..
 * 65534 sequences; PKV_ERR_INVALID_ARG (nothing launched) otherwise or if
 * the source is not pinned, mapped host memory.  Other arguments and errors
 * as pkv_paged_attention_decode_shared_prefix. */
pkv_status pkv_paged_attention_decode_shared_prefix_step(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* seq_order, int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    const int32_t* members, const int32_t* member_flag, int32_t num_members,
    int32_t prefix_tokens, void* workspace, size_t workspace_bytes, void* next_dst,
    const void* next_src_host, size_t next_bytes, pkv_dtype dtype, void* stream);

/* The decode step in one launch (the cache write fused into the attention):
 * for every sequence b with context_lens[b] > 0, its new token is its last
 * position p = context_lens[b] - 1 (already appended by the allocator), and
 * new_key[b] / new_value[b] (device, num_kv_heads x head_dim elements from
 * element b * key_seq_stride / b * value_seq_stride) are written into the
 * caches at the slot the block table gives for p; then the result is that
 * of pkv_paged_attention_decode.  Equivalent to pkv_kv_reshape_and_cache of
 * those rows at those slots followed by pkv_paged_attention_decode, in one
 * kernel (plus the merge when partitioned): the row of p is read from
 * new_key / new_value, never from the slot being written.  Strides must be
 * >= num_kv_heads * head_dim and multiples of 16 bytes; pointers 16-byte
 * aligned (PKV_ERR_INVALID_ARG otherwise).  A table entry outside the pool
 * skips the write.  Other arguments and errors as pkv_paged_attention_decode.
 */
pkv_status pkv_paged_attention_decode_write(void* out, const void* q,
                                            const void* new_key, const void* new_value,
                                            int64_t key_seq_stride, int64_t value_seq_stride,
                                            void* k_cache, void* v_cache,
                                            const int32_t* block_tables,
                                            int32_t max_blocks_per_seq,
                                            const int32_t* context_lens,
                                            const int32_t* seq_order,
                                            int32_t max_context_len, int32_t num_seqs,
                                            int32_t num_q_heads, int32_t num_kv_heads,
                                            int32_t head_dim, int32_t block_size,
                                            int32_t num_blocks, float scale,
                                            int32_t partition_size, void* workspace,
                                            size_t workspace_bytes, pkv_dtype dtype,
                                            void* stream);

/* The decode step's device work in one launch, for a serving loop that
 * prepares each step's index arrays one step ahead: pkv_paged_attention_
 * decode_write, and in the same launch a copy of next_bytes from next_src_host
 * (pinned host memory mapped into the device's address space, e.g. a torch
 * tensor from pin_memory()) to next_dst (device): the next step's block
 * tables, lengths, launch order and slots.  The copy runs on the workgroups
 * of one extra grid row, dispatched first; so the next step needs no upload
 * launch of its own and no event between the two streams ("vLLM in
 * Production …", section "Continuous Batching Keeps the GPU Full": the
 * batch is re-formed at every step).  next_dst must not overlap anything
 * this call reads or writes (the current step's arrays sit in another
 * buffer); the caller must not change next_src_host until the call has
 * completed.  next_bytes = 0: exactly pkv_paged_attention_decode_write.
 * new_key and new_value both NULL: a step without new tokens (strides
 * ignored, nothing written into the caches): the attention of
 * pkv_paged_attention_decode plus the upload; only one of them NULL is
 * PKV_ERR_INVALID_ARG.
 * next_bytes and both addresses must be multiples of 16, the batch 1 ..
 * 65534 sequences; PKV_ERR_INVALID_ARG (nothing launched) otherwise or if
 * the source is not pinned, mapped host memory.  Other arguments and
 * errors as pkv_paged_attention_decode_write. */
pkv_status pkv_paged_attention_decode_step(void* out, const void* q,
                                           const void* new_key, const void* new_value,
                                           int64_t key_seq_stride, int64_t value_seq_stride,
                                           void* k_cache, void* v_cache,
                                           const int32_t* block_tables,
                                           int32_t max_blocks_per_seq,
                                           const int32_t* context_lens,
                                           const int32_t* seq_order,
                                           int32_t max_context_len, int32_t num_seqs,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size,
                                           int32_t num_blocks, float scale,
                                           int32_t partition_size, void* workspace,
                                           size_t workspace_bytes, void* next_dst,
                                           const void* next_src_host, size_t next_bytes,
                                           pkv_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * Chunked prefill: several new tokens per sequence attend to the paged cache
 * (long prompts are processed in pieces so that one large prefill does not
 * stall decoding: "Serving models with vLLM", section "How it works:
 * continuous batching").  Sequence b owns query rows query_start[b] ..
 * query_start[b+1]-1 of q and out; its n_b new tokens are the last n_b of its
 * context (their K/V already written, e.g. by pkv_kv_reshape_and_cache), so
 * query i sits at position context_lens[b] - n_b + i and attends to tokens
 * 0 .. that position (causal).  A query with a negative position (a chunk
 * longer than its context) gets zeros; a sequence with no queries is
 * skipped.  n_b = 1 for every sequence is the decode step.
 *
 * out, q        device, [total_queries, num_q_heads, head_dim] (bf16).
 * query_start   device, int32 [num_seqs + 1], non-decreasing, last entry
 *               total_queries (entries are clamped into [0, total_queries]).
 * max_queries_per_seq  host-side upper bound of n_b (sizes the grid; rows
 *               past it are not computed).
 * Other arguments as pkv_paged_attention_decode; the workspace size is
 * pkv_prefill_workspace_bytes(...) (for AUTO it covers the partitioned
 * case; pkv_prefill_partition_size tells what AUTO resolves to: single pass
 * unless the query tiles give fewer than about four workgroups per CU).  Runs on the matrix cores: each tile holds
 * 16 (query, head) rows — floor(16 / G) queries of one sequence times the G
 * query heads of one kv head — and the tiles of a workgroup share each K/V
 * chunk through LDS.  bf16 only; head_dim in {64, 128};
 * block_size in {16, 32}; G = num_q_heads / num_kv_heads in 1..16.
 * ---------------------------------------------------------------------- */
size_t pkv_prefill_workspace_bytes(int32_t total_queries, int32_t num_q_heads,
                                   int32_t head_dim, int32_t max_context_len,
                                   int32_t partition_size);

/* The partition size a prefill call with these arguments uses (resolves
 * AUTO); 0 means single pass. */
int32_t pkv_prefill_partition_size(int32_t num_seqs, int32_t max_queries_per_seq,
                                   int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t max_context_len, int32_t partition_size);

pkv_status pkv_paged_attention_prefill(void* out, const void* q,
                                       const int32_t* query_start,
                                       int32_t total_queries,
                                       int32_t max_queries_per_seq,
                                       const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables,
                                       int32_t max_blocks_per_seq,
                                       const int32_t* context_lens,
                                       const int32_t* seq_order,
                                       int32_t max_context_len, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size,
                                       int32_t num_blocks, float scale,
                                       int32_t partition_size, void* workspace,
                                       size_t workspace_bytes, pkv_dtype dtype,
                                       void* stream);

/* ------------------------------------------------------------------------
 * Block copy: cache[dst] = cache[src] for each (src, dst) pair, K and V.
 * Used to give a sequence a private copy of a block that others still hold
 * (copy-on-write of a shared block, "What Is vLLM …", section "How does
 * PagedAttention work?", memory-sharing step).
 * pairs  device, int64 [num_pairs, 2] as (src, dst); ids outside
 *        [0, num_blocks) are skipped; a dst must not appear twice nor be
 *        any pair's src.
 * ---------------------------------------------------------------------- */
pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, const int64_t* pairs,
                           int32_t num_pairs, int32_t num_blocks,
                           int32_t block_size, int32_t num_kv_heads,
                           int32_t head_dim, pkv_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * Host-to-device staging by the GPU: copies `bytes` from pinned host memory
 * (allocated pinned and mapped into the device's address space, e.g. a torch
 * tensor from pin_memory()) to device memory, as a kernel on `stream`.  Used
 * for each decode step's tables, lengths and slots: the launch is queued like
 * any kernel and never waits for earlier work, unlike a runtime copy that may
 * block the host.  The caller must not rewrite `src_host` until the copy has
 * run (e.g. a ring of staging buffers guarded by events).
 * bytes and both addresses must be multiples of 16; PKV_ERR_INVALID_ARG if
 * the source is not pinned, mapped host memory (nothing is launched).
 * ---------------------------------------------------------------------- */
pkv_status pkv_upload_pinned(void* dst, const void* src_host, size_t bytes, void* stream);

/* ------------------------------------------------------------------------
 * Swap copy: moves whole blocks between the device cache and a cache pool in
 * pinned host memory, the data movement of preemption by swapping ("What Is
 * vLLM …", section "What is continuous batching in vLLM?", step 2: under
 * memory pressure low-priority sequences are preempted and their KV caches
 * moved to CPU memory; its configuration list sizes that CPU space).
 *
 * direction PKV_SWAP_OUT: host[dst] = device[src] for each (src, dst) pair;
 * PKV_SWAP_IN: device[dst] = host[src].  The pairs come from
 * pkv_swap_out / pkv_swap_in below.
 * k_cache, v_cache  device, [num_blocks, block_size, num_kv_heads, head_dim].
 * k_host, v_host    pinned, mapped host memory (hipHostMalloc, or a torch
 *                   tensor from pin_memory()), [num_host_blocks, block_size,
 *                   num_kv_heads, head_dim]; the caller owns both pools.
 * pairs             device, int64 [num_pairs, 2]; a pair with an id outside
 *                   its pool is skipped; destinations must be distinct.
 * Runs as a kernel on `stream` that reads or writes the host pool over the
 * host link; nothing else synchronizes.  The caller must not touch the host
 * blocks involved until the copy has run.  PKV_ERR_INVALID_ARG (nothing
 * launched) if a host pool is not pinned, mapped memory.
 * ---------------------------------------------------------------------- */
#define PKV_SWAP_OUT 0
#define PKV_SWAP_IN 1
pkv_status pkv_swap_blocks(void* k_cache, void* v_cache, void* k_host, void* v_host,
                           const int64_t* pairs, int32_t num_pairs, int32_t num_blocks,
                           int32_t num_host_blocks, int32_t block_size,
                           int32_t num_kv_heads, int32_t head_dim, pkv_dtype dtype,
                           int32_t direction, void* stream);

/* ------------------------------------------------------------------------
 * Host block allocator (host memory only; single-threaded use).
 *
 * The pool of fixed-size blocks, the per-sequence block tables mapping
 * logical blocks to physical ones like a page table, and growth one block
 * at a time ("vLLM in Production …", section "PagedAttention — Virtual Memory
 * for the KV Cache"); only a sequence's last block is partly empty
 * ("Serving models with vLLM", section "How it works: PagedAttention");
 * blocks shared between sequences carry reference counts ("What Is vLLM …",
 * section "How does PagedAttention work?", memory-sharing step).
 *
 * Fixed-size blocks are handed out one at a time as a sequence grows; a
 * sequence's table lists its physical blocks in logical order and token
 * pos is stored at slot table[pos / block_size] * block_size +
 * pos % block_size.  Free blocks are handed out first-in first-out,
 * starting from free_order (a permutation of 0..num_blocks-1, or ascending
 * when NULL); a freed block joins the tail when its reference count drops
 * to zero.  Forked sequences share blocks by reference count.
 * ---------------------------------------------------------------------- */
typedef struct pkv_allocator pkv_allocator;

/* Creates an allocator over a pool of num_blocks blocks of block_size
 * tokens ("vLLM in Production …", section "PagedAttention — Virtual Memory
 * for the KV Cache": the cache is cut into fixed-size blocks); *out receives
 * the handle (library-owned memory, released by pkv_allocator_destroy).
 * PKV_ERR_INVALID_ARG for a negative num_blocks, a non-positive block_size
 * or a free_order that is not a permutation of 0..num_blocks-1. */
pkv_status pkv_allocator_create(int32_t num_blocks, int32_t block_size,
                                const int32_t* free_order, pkv_allocator** out);
void pkv_allocator_destroy(pkv_allocator* a);

/* New empty sequence: no block is reserved up front ("Serving models with
 * vLLM", section "How it works: PagedAttention": blocks are allocated on
 * demand).  PKV_ERR_INVALID_ARG if the id exists. */
pkv_status pkv_seq_add(pkv_allocator* a, int64_t seq_id);

/* dst (existing, empty) shares the blocks holding src's first num_tokens
 * tokens (each block's reference count + 1): sequences with a common prefix
 * point at the same physical blocks ("What Is vLLM …", section "How does
 * PagedAttention work?", memory-sharing step).  num_tokens must be a
 * multiple of block_size or src's whole length (PKV_ERR_INVALID_ARG);
 * PKV_ERR_NOT_FOUND for an unknown id. */
pkv_status pkv_seq_fork_prefix(pkv_allocator* a, int64_t src, int64_t dst,
                               int32_t num_tokens);

/* Grows seq_id by num_tokens, opening a new block only when the last one is
 * full ("vLLM in Production …", section "PagedAttention — Virtual Memory for
 * the KV Cache": blocks are added one at a time as tokens arrive, so no
 * final length is guessed); slots_out (host, int64 [num_tokens], may be
 * NULL) receives their slots.  PKV_ERR_OUT_OF_BLOCKS if the pool is short,
 * PKV_ERR_SHARED_WRITE if a token would land in a block another sequence
 * holds; both leave the allocator unchanged. */
pkv_status pkv_seq_append(pkv_allocator* a, int64_t seq_id, int32_t num_tokens,
                          int64_t* slots_out);

/* Batched append: sequence seq_ids[i] grows by num_tokens[i], in order;
 * slots_out (host, int64 [sum of num_tokens]) receives all new slots in
 * that order.  All-or-nothing. */
pkv_status pkv_append_tokens(pkv_allocator* a, const int64_t* seq_ids,
                             const int32_t* num_tokens, int32_t num_seqs,
                             int64_t* slots_out);

/* Copy-on-write append ("What Is vLLM …", section "How does PagedAttention
 * work?", memory-sharing step): like pkv_append_tokens, but a sequence whose
 * last block is partly filled and held by other sequences too (after a full
 * fork, as beam candidates do) first gets a private copy: a fresh block
 * replaces it in the sequence's table and the shared block's count drops by
 * one.  Each copy is reported as a (source, destination) block pair in
 * copy_pairs_out (host int64 [max_pairs, 2], the pkv_copy_blocks layout) and
 * *num_pairs_out; the caller copies those blocks (pkv_copy_blocks) before
 * writing the new tokens.  A full shared block is never copied (the next token
 * opens a new block).  All-or-nothing: PKV_ERR_OUT_OF_BLOCKS counts the
 * copies; PKV_ERR_INVALID_ARG if more than max_pairs copies are needed. */
pkv_status pkv_append_tokens_cow(pkv_allocator* a, const int64_t* seq_ids,
                                 const int32_t* num_tokens, int32_t num_seqs,
                                 int64_t* slots_out, int64_t* copy_pairs_out,
                                 int32_t max_pairs, int32_t* num_pairs_out);

/* Releases the sequence; blocks whose reference count drops to zero are
 * freed ("What Is vLLM …", section "How does PagedAttention work?",
 * memory-sharing step: a shared block stays while any holder remains).
 * PKV_ERR_NOT_FOUND for an unknown id. */
pkv_status pkv_seq_free(pkv_allocator* a, int64_t seq_id);

/* The block tables the attention calls read ("vLLM in Production …",
 * section "PagedAttention — Virtual Memory for the KV Cache": a
 * per-sequence table from logical to physical blocks).
 * tables_out (host, int32 [num_seqs, max_blocks_per_seq]) receives each
 * sequence's block table padded with pad_value; context_lens_out (host,
 * int32 [num_seqs], may be NULL) their lengths.  PKV_ERR_INVALID_ARG if a
 * sequence has more than max_blocks_per_seq blocks. */
pkv_status pkv_build_block_tables(const pkv_allocator* a, const int64_t* seq_ids,
                                  int32_t num_seqs, int32_t max_blocks_per_seq,
                                  int32_t pad_value, int32_t* tables_out,
                                  int32_t* context_lens_out);

/* Host helper: order_out (host int32 [n]) receives 0..n-1 sorted by
 * context_lens (host int32 [n]) descending, ties by index — the launch order
 * pkv_paged_attention_decode's seq_order expects. */
pkv_status pkv_longest_first_order(const int32_t* context_lens, int32_t n, int32_t* order_out);

/* One decode step's host work in one call: every sequence in seq_ids grows
 * by one token (slots_out, host int64 [num_seqs], receives the new slots in
 * order), then tables_out (host int32 [num_seqs, max_blocks_per_seq]) and
 * context_lens_out (host int32 [num_seqs]) receive the grown tables and
 * lengths, *max_context_len_out their maximum and order_out (host int32
 * [num_seqs]) the longest-first launch order (any of the last three may be
 * NULL).
 * seq_ids must be distinct.  All-or-nothing: PKV_ERR_NOT_FOUND,
 * PKV_ERR_INVALID_ARG (a repeated id, or a table that would not fit),
 * PKV_ERR_OUT_OF_BLOCKS or PKV_ERR_SHARED_WRITE leave the allocator
 * unchanged. */
pkv_status pkv_decode_step_prepare(pkv_allocator* a, const int64_t* seq_ids,
                                   int32_t num_seqs, int32_t max_blocks_per_seq,
                                   int32_t pad_value, int64_t* slots_out,
                                   int32_t* tables_out, int32_t* context_lens_out,
                                   int32_t* max_context_len_out, int32_t* order_out);

/* ------------------------------------------------------------------------
 * Preemption by swapping ("What Is vLLM …", section "What is continuous
 * batching in vLLM?", step 2).  The allocator also manages a pool of
 * num_host_blocks blocks in host memory with its own first-in first-out
 * free list (host_free_order, a permutation, or ascending when NULL).
 *
 * pkv_swap_out moves the listed sequences (distinct, resident) to host
 * blocks: their device blocks are visited sequence by sequence in table
 * order; each distinct device block gets one host block (blocks shared
 * inside the group stay shared, one copy), reported as a (device, host) pair
 * in pairs_out (host int64 [max_pairs, 2]) and *num_pairs_out; the
 * sequences' tables then hold the host blocks, and each device block loses
 * one reference per holder in the group (freed at zero, in visiting order).
 * A device block also held by a sequence outside the group is still copied
 * and stays with that sequence.  pkv_swap_in does the reverse with fresh
 * device blocks: (host, device) pairs, host blocks freed at zero.
 * The caller runs pkv_swap_blocks over the pairs before anything can write
 * into the freed blocks (stream order is enough).  All-or-nothing:
 * PKV_ERR_OUT_OF_BLOCKS if the target pool is short, PKV_ERR_SWAPPED if a
 * sequence is already in the other state, PKV_ERR_INVALID_ARG for a
 * repeated id, no host pool, or more than max_pairs pairs.
 *
 * While a sequence is swapped out, append, copy-on-write append, fork (as
 * source or destination), table building and the decode-step call refuse it
 * with PKV_ERR_SWAPPED; pkv_seq_free releases its host blocks.
 * ---------------------------------------------------------------------- */
/* Gives the allocator its host pool (once; PKV_ERR_INVALID_ARG otherwise). */
pkv_status pkv_allocator_set_host_pool(pkv_allocator* a, int32_t num_host_blocks,
                                       const int32_t* host_free_order);
pkv_status pkv_swap_out(pkv_allocator* a, const int64_t* seq_ids, int32_t num_seqs,
                        int64_t* pairs_out, int32_t max_pairs, int32_t* num_pairs_out);
pkv_status pkv_swap_in(pkv_allocator* a, const int64_t* seq_ids, int32_t num_seqs,
                       int64_t* pairs_out, int32_t max_pairs, int32_t* num_pairs_out);
/* 1 if swapped out, 0 if resident, -1 if unknown. */
int32_t pkv_seq_is_swapped(const pkv_allocator* a, int64_t seq_id);
/* Free host blocks, -1 without a host pool. */
int32_t pkv_num_free_host_blocks(const pkv_allocator* a);
/* Reference count of a host block (0 = free), -1 for an id outside the pool. */
int32_t pkv_host_block_refcount(const pkv_allocator* a, int32_t host_block_id);

/* ------------------------------------------------------------------------
 * Automatic prefix caching: requests with the same prefix (a system prompt,
 * a document) point at the same physical blocks ("Serving models with vLLM",
 * section "How it works: PagedAttention"; "What Is vLLM …", memory-sharing
 * step).  With the cache enabled, a full block is entered under the tokens
 * of the whole prefix it ends.  pkv_seq_add_prompt creates sequence seq_id
 * for a prompt (host int32 tokens [num_tokens]): it shares the longest run
 * of cached full blocks at the prompt's start, but never the block holding
 * the last token (that token is always computed), allocates the rest and
 * enters the prompt's other full blocks.  slots_out (host int64, [num_tokens
 * - cached]) receives the slots of the tokens after the shared part and
 * *num_cached_out the shared token count: the caller writes only those
 * tokens' K/V (pkv_kv_reshape_and_cache) before any later reader's attention
 * runs, and runs prefill for them over the whole context.  A freed block
 * keeps its entry (and can be shared again, leaving the free list with the
 * others' order kept) until the free list hands it out for other tokens;
 * then its entry and every entry extending it are dropped.  Without the
 * cache enabled the call is seq_add + append.  All-or-nothing:
 * PKV_ERR_OUT_OF_BLOCKS, PKV_ERR_INVALID_ARG (the id exists).
 * ---------------------------------------------------------------------- */
pkv_status pkv_allocator_enable_prefix_cache(pkv_allocator* a);
pkv_status pkv_seq_add_prompt(pkv_allocator* a, int64_t seq_id, const int32_t* tokens,
                              int32_t num_tokens, int64_t* slots_out,
                              int32_t* num_cached_out);
/* Full-block lookups and hits so far (the cache hit rate is hits / lookups)
 * and the number of blocks holding a cached prefix; any pointer may be NULL. */
pkv_status pkv_prefix_cache_stats(const pkv_allocator* a, int64_t* lookups, int64_t* hits,
                                  int32_t* num_cached_blocks);

/* Free blocks of the pool (the unused share of the KV-cache memory). */
int32_t pkv_num_free_blocks(const pkv_allocator* a);
/* Reference count of a block (0 = free), -1 for an id outside the pool: the
 * number of sequences whose tables hold it ("What Is vLLM …", section "How
 * does PagedAttention work?", memory-sharing step). */
int32_t pkv_block_refcount(const pkv_allocator* a, int32_t block_id);
/* Length in tokens of a sequence, -1 if unknown. */
int64_t pkv_seq_context_len(const pkv_allocator* a, int64_t seq_id);
/* Number of blocks of a sequence (device or host), -1 if unknown. */
int32_t pkv_seq_num_blocks(const pkv_allocator* a, int64_t seq_id);

/* The shared-prefix members of a batch, derived from the tables ("What Is
 * vLLM …", section "How does PagedAttention work?", memory-sharing step:
 * sequences with a common prefix point at the same physical blocks).  Among
 * seq_ids (distinct, resident), the sequences longer than prefix_tokens
 * whose first prefix_tokens / block_size blocks are the same physical blocks
 * form a group; the largest group of at least two (the one met first in
 * seq_ids order on a tie) is reported: members_out (host int32 [num_seqs])
 * receives its positions in seq_ids, ascending, *num_members_out their
 * count (0 if no two sequences share), member_flag_out (host int32
 * [num_seqs]) 1 for the members and 0 otherwise: the members / member_flag
 * arguments of pkv_paged_attention_decode_shared_prefix for a batch in
 * seq_ids order.  PKV_ERR_INVALID_ARG (prefix_tokens not a positive multiple
 * of the block size, a repeated id), PKV_ERR_NOT_FOUND, PKV_ERR_SWAPPED. */
pkv_status pkv_shared_prefix_members(const pkv_allocator* a, const int64_t* seq_ids,
                                     int32_t num_seqs, int32_t prefix_tokens,
                                     int32_t* members_out, int32_t* member_flag_out,
                                     int32_t* num_members_out);

/* ------------------------------------------------------------------------
 * Pool size from a memory budget: the memory left for the KV cache becomes
 * blocks ("vLLM in Production …", section "Scaling Up — Tensor Parallelism
 * and Engine Args": what the memory-utilization setting leaves after the
 * weights becomes KV-cache blocks).  One block id covers block_size tokens
 * of K and of V in each of num_layers layers, i.e. 2 * num_layers *
 * block_size * num_kv_heads * head_dim elements; the result is
 * floor(bytes / that size in bytes), at most INT32_MAX (0 if one block does
 * not fit, or its size overflows 64 bits), -1 for a non-positive size or an
 * unknown dtype.
 * ---------------------------------------------------------------------- */
int32_t pkv_blocks_for_budget(size_t bytes, int32_t num_layers, int32_t block_size,
                              int32_t num_kv_heads, int32_t head_dim, pkv_dtype dtype);

/* ------------------------------------------------------------------------
 * Debug validator of a decode call's index arrays, on host copies: the
 * kernels never fault on a bad id (an id outside the pool reads block 0, a
 * length beyond max_context_len is clamped, members are trusted), so such
 * inputs return PKV_OK with a meaningless result.  This call returns
 * PKV_ERR_INVALID_ARG, its message naming the first bad entry, unless
 *   - 0 <= context_lens[b] <= min(max_context_len,
 *     max_blocks_per_seq * block_size) for every b;
 *   - every table entry a context reads (the first ceil(context_lens[b] /
 *     block_size) of row b) lies in [0, num_blocks);
 *   - seq_order (may be NULL) is a permutation of 0..num_seqs-1;
 *   - with num_members > 0: members are distinct indices, member_flag is
 *     nonzero exactly for them, every member's context is longer than
 *     prefix_tokens (a positive multiple of block_size), and every member's
 *     first prefix_tokens / block_size table entries equal the first
 *     member's.
 * All arrays are host int32: block_tables [num_seqs, max_blocks_per_seq],
 * context_lens, seq_order, member_flag [num_seqs], members [num_members].
 * ---------------------------------------------------------------------- */
pkv_status pkv_validate_decode_inputs(const int32_t* block_tables, int32_t num_seqs,
                                      int32_t max_blocks_per_seq, const int32_t* context_lens,
                                      const int32_t* seq_order, int32_t max_context_len,
                                      int32_t block_size, int32_t num_blocks,
                                      const int32_t* members, const int32_t* member_flag,
                                      int32_t num_members, int32_t prefix_tokens);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
