// Definitions shared by the decode and chunked-prefill attention kernels:
// the argument block, the sequence and query lookups with their clamps, the
// matrix-core operand types, and the host-side partition and workspace rules.
#pragma once

#include <algorithm>
#include <cfloat>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

using namespace dev;


// Workgroup -> (partition, kv head [x query tile], sequence).  The dispatcher
// deals consecutive workgroups round-robin to the 8 XCDs.  Partitions of one
// sequence are kept adjacent (they read neighbouring blocks of the same
// table), and the partition dimension of the grid is odd, so the partitions
// of consecutive (head, sequence) pairs rotate over the XCDs instead of
// partition p always landing on XCD p mod 8 (measured: a grid of exactly 8
// partition columns ran 2.3x slower).  Columns past a sequence's partition
// count are empty and exit at once.
inline dim3 work_grid(int parts, int y, int seqs) { return dim3(parts | 1, y, seqs); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kChunk = 16;          // tokens per wave iteration
constexpr int kSingle = 1 << 30;    // "partition" length of single-pass mode

struct AttnArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* tables;
  const int32_t* ctx_lens;
  const int32_t* order;  // optional launch order of the sequences (a permutation)
  const int32_t* query_start;  // prefill: first query row of each sequence [B + 1]
  int32_t q_tiles;             // prefill: query tiles per sequence (grid y = kv heads x tiles)
  int32_t q_groups;            // prefill: workgroups of query tiles per (sequence, kv head)
  int32_t total_queries;       // prefill: rows of q / out
  float* part_o;   // [B, Hq, max_parts, D]
  float* part_ml;  // [B, Hq, max_parts, 2] (max in log2 units, sum)
  int32_t num_seqs;
  int32_t max_blocks;
  int32_t ctx_cap;  // min(max_context_len, max_blocks * block_size)
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t partition;  // tokens per partition (multiple of 16), kSingle = one
  int32_t max_parts;
  // Shared prefix (decode): grid rows z >= group_z0 compute partition 0 (the
  // prefix) once for tiles of members whose tables start with the same
  // blocks; member_flag[b] != 0 makes the sequence's own partition-0
  // workgroup skip it.  members == nullptr: off.
  const int32_t* members;
  const int32_t* member_flag;
  int32_t num_members;
  int32_t group_z0;    // first grid row of the shared-prefix tiles
  int32_t group_z1;    // one past their last row
  int32_t seq_z0;      // first grid row of the sequences
  int32_t first_part;  // > 0: a member's partition 0 is this many tokens, the rest `partition` each
  float scale_log2;   // scale * log2(e): logits are kept in base-2 units
};

// Sequence handled by grid row z: the caller's launch order if given (e.g.
// longest first, so the longest sequences do not finish last), else z.
// Entries are clamped into range, so a bad order cannot read out of bounds.
__device__ __forceinline__ int seq_of(const AttnArgs& a, int z) {
  if (!a.order) return z;
  const int b = scalar_read(a.order + z);
  return (unsigned)b < (unsigned)a.num_seqs ? b : z;
}

// Prefill: first query row and query count of sequence b, clamped so that a
// bad query_start can never address rows outside [0, total_queries).
__device__ __forceinline__ void query_range(const AttnArgs& a, int b, int& first, int& count) {
  int lo = scalar_read(a.query_start + b);
  int hi = scalar_read(a.query_start + b + 1);
  lo = lo < 0 ? 0 : (lo > a.total_queries ? a.total_queries : lo);
  hi = hi < lo ? lo : (hi > a.total_queries ? a.total_queries : hi);
  first = lo;
  count = hi - lo;
}

// Token range [start, start + length) of partition p and the number of
// partitions of a ctx-token context: uniform partitions of a.partition
// tokens, or (fp > 0) a first partition of fp tokens and then uniform ones.
__device__ __forceinline__ int part_begin(const AttnArgs& a, int fp, int p) {
  return fp > 0 ? (p == 0 ? 0 : fp + (p - 1) * a.partition) : p * a.partition;
}
__device__ __forceinline__ int part_length(const AttnArgs& a, int fp, int p) {
  return fp > 0 && p == 0 ? fp : a.partition;
}
__device__ __forceinline__ int part_count(const AttnArgs& a, int fp, int ctx) {
  if (fp > 0) return ctx <= fp ? 1 : 1 + (ctx - fp + a.partition - 1) / a.partition;
  return (ctx + a.partition - 1) / a.partition;
}

// First-partition length of sequence b: in a shared-prefix call, the prefix
// for the sharing sequences (their partition 0 is computed once per tile);
// every other sequence keeps uniform partitions.
__device__ __forceinline__ int first_part_of(const AttnArgs& a, int b) {
  return a.first_part > 0 && a.member_flag[b] != 0 ? a.first_part : 0;
}

__device__ __forceinline__ int clamp_ctx(const AttnArgs& a, int b) {
  int c = a.ctx_lens[b];
  return c < 0 ? 0 : (c > a.ctx_cap ? a.ctx_cap : c);
}

// Matrix-core operand and accumulator types.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4_t;
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x2v_t __attribute__((ext_vector_type(2)));

constexpr float kLazyMax = 8.0f;  // log2 of the largest p allowed before rescaling

// Maximum of two scores (never NaN: finite or -inf).  The IEEE 754-2019
// maximum lowers to v_maximum3_f32 with no quieting of its inputs, where
// fmaxf canonicalises any input the compiler cannot prove canonical (one
// extra instruction per score where masked and unmasked scores merge).
__device__ __forceinline__ float vmax(float x, float y) {
  return __builtin_elementwise_maximum(x, y);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2v_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v_t));  // RNE
}

// Host side.
#ifndef PKV_AUTO_PARTITION
#define PKV_AUTO_PARTITION 2048
#endif

// Partition length actually used, 0 = single pass.  AUTO splits contexts
// longer than 2048 tokens into 2048-token partitions (measured on MI355X over
// the five decode shapes with a longest-first launch order).
int32_t resolve_partition(int32_t max_context_len, int32_t partition_size) {
  if (partition_size == PKV_PARTITION_AUTO)
    return max_context_len > PKV_AUTO_PARTITION ? PKV_AUTO_PARTITION : 0;
  return partition_size;
}

size_t workspace_for(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                     int32_t max_context_len, int32_t partition) {
  if (partition <= 0 || max_context_len <= 0) return 0;
  const size_t parts = size_t((int64_t(max_context_len) + partition - 1) / partition);
  const size_t heads = size_t(num_seqs) * size_t(num_q_heads);
  return heads * parts * (size_t(head_dim) + 2) * sizeof(float);
}

}  // namespace
}  // namespace pkv
