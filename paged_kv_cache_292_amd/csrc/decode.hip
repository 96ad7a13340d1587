// Paged decode attention for gfx950.
//
// One query token per sequence attends to its whole context, whose keys and
// values sit in fixed-size blocks reached through the sequence's block table
// ("vLLM in Production …", section "PagedAttention — Virtual Memory for the
// KV Cache"; "What Is vLLM …", section "How does PagedAttention work?", the
// position-to-block lookup).  Cache layout: [num_blocks][block_size]
// [num_kv_heads][head_dim]; one token's row of one kv head is head_dim
// contiguous elements.
//
// Work split.  A workgroup owns (sequence, HG adjacent kv heads, partition)
// with NW / HG waves per head; the waves of one head take its 16-token chunks
// round-robin, and the HG waves of one stream work on the same chunk of the
// adjacent heads, whose rows sit side by side in the cache.  Inside a wave
// the four 16-lane rows each own one token slot of the chunk and every lane
// holds head_dim/16 elements of a row, so one 16-byte load per lane fetches
// four token rows (4 x 256 B for bf16, head_dim 128).  q·k is summed over the 16
// lanes of a row with DPP; each row keeps its own online-softmax state (max,
// sum, accumulator) per query head, and rows and waves are merged at the end.
// The next chunk's K/V loads are issued before the current chunk is reduced.
//
// Long contexts are split into partitions handled by separate workgroups;
// each writes its normalised partial output with its max and sum, and a
// second kernel merges them by log-sum-exp weights.
//
// Chunked prefill (several queries per sequence) shares the argument block
// and helpers in attn_common.h and lives in prefill.hip.
#include <mutex>

#include "attn_common.h"

namespace pkv {
namespace {

// ---------------------------------------------------------------------------
// The decode step's new tokens, for the fused cache write (kernels built with
// WRITE): sequence b's new token is its last position, ctx_b - 1; its K and V
// rows (kv heads contiguous, head_dim elements each) start at element
// b * stride of new_k / new_v.  In the workgroup whose partition holds that
// position, the first wave of each kv head loads the head's new rows, stores
// them into the cache at the slot the block table gives and adds the token to
// its softmax after the chunk loop, which stops one position early: nothing
// in the launch reads the slot being written.
struct NewRows {
  const void* new_k;
  const void* new_v;
  int64_t k_stride;  // elements between sequences' rows
  int64_t v_stride;
  // The next step's index arrays, copied within the launch (decode step
  // only): pf_n16 16-byte pieces from pinned host memory (device-mapped
  // address pf_src) to pf_dst by the workgroups of the first pf_rows grid
  // rows; the sequences' rows follow them.
  const uint4* pf_src;
  uint4* pf_dst;
  int64_t pf_n16;
  int32_t pf_rows;
};

// The next step's upload by the workgroups of the first w.pf_rows grid rows:
// each thread issues up to four 16-byte loads over the host link before its
// stores.
__device__ __forceinline__ void copy_next_step(const NewRows& w) {
  const int64_t nthreads = int64_t(gridDim.x) * gridDim.y * w.pf_rows * blockDim.x;
  const int64_t t =
      ((int64_t(blockIdx.z) * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) * blockDim.x +
      threadIdx.x;
  for (int64_t i = t; i < w.pf_n16; i += 4 * nthreads) {
    uint4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (i + k * nthreads < w.pf_n16) v[k] = w.pf_src[i + k * nthreads];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (i + k * nthreads < w.pf_n16) w.pf_dst[i + k * nthreads] = v[k];
  }
}

// Stores a lane's fragment (the counterpart of load_frag).
template <int WORDS>
__device__ __forceinline__ void store_frag(void* p, const Frag<WORDS>& f) {
  if constexpr (WORDS % 4 == 0) {
    uint4* v = reinterpret_cast<uint4*>(p);
#pragma unroll
    for (int i = 0; i < WORDS / 4; ++i)
      v[i] = make_uint4(f.w[4 * i + 0], f.w[4 * i + 1], f.w[4 * i + 2], f.w[4 * i + 3]);
  } else {
    static_assert(WORDS == 2, "8- or 16-byte multiples only");
    *reinterpret_cast<uint2*>(p) = make_uint2(f.w[0], f.w[1]);
  }
}

// ---------------------------------------------------------------------------
// Partition kernel, query-head group G on the vector ALUs.
//
// HG adjacent kv heads per workgroup (measured on MI355X, LLaMA-13B decode
// batch: 4 heads x 4 waves each reads HBM at 6.76 TB/s where one head x 4
// waves reads at 6.34 TB/s: the four waves reading one chunk of four adjacent
// heads fetch 1 KB contiguous per token row instead of 256 B pieces 10 KB
// apart).
template <typename T, int D, int BS, int G, int NW, int HG, bool WRITE>
__global__ __launch_bounds__(NW * 64) void decode_valu_kernel(AttnArgs a, NewRows w) {
  constexpr int EPL = D / 16;                      // elements per lane
  constexpr int WORDS = EPL * int(sizeof(T)) / 4;  // 32-bit words per lane
  constexpr int S = NW / HG;                       // waves (chunk streams) per head
  static_assert(NW % HG == 0, "waves must split evenly over the heads");
  using F = Frag<WORDS>;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane >> 4;
  const int r = lane & 15;
  if (int(blockIdx.z) < w.pf_rows) {  // the next step's upload
    copy_next_step(w);
    return;
  }
  const int part = blockIdx.x;
  const int kvh0 = blockIdx.y * HG;     // first kv head of the workgroup
  const int kvh = kvh0 + wave % HG;     // this wave's kv head
  const int stream = wave / HG;         // this wave's chunk stream
  const int b = seq_of(a, int(blockIdx.z) - w.pf_rows);
  const int Hq = a.num_q_heads;
  const int Hkv = a.num_kv_heads;

  const int ctx = clamp_ctx(a, b);
  const int t0 = part * a.partition;
  const int t1 = min(ctx, t0 + a.partition);
  const int nparts = (ctx + a.partition - 1) / a.partition;
  if (t0 >= t1) {
    if (ctx == 0 && part == 0) {
      for (int i = threadIdx.x; i < HG * G * D; i += NW * 64)
        store_elem<T>(a.out, (size_t(b) * Hq + kvh0 * G) * D + i, 0.0f);
    }
    return;
  }
  // Fused write: the new token (position `last`) belongs to the workgroup
  // whose partition holds it.  There the first stream of each head loads the
  // head's new K/V rows from the input together with q; after the chunk loop,
  // which stops before the token, it stores them into the cache slot and adds
  // the token to its softmax: no load of this launch touches the slot being
  // written.
  const int last = ctx - 1;
  const bool own_new = WRITE && last >= t0 && last < t1;
  const int t1l = own_new ? last : t1;  // end of the chunk loop
  // The token goes to the stream with the fewest chunks: stream k takes
  // chunks k, k + S, ... of the partition's n, so stream n % S is one short
  // unless S divides n.
  const int n_chunks = (t1l + kChunk - 1) / kChunk - t0 / kChunk;
  const bool add_new = own_new && stream == n_chunks % S;

  // q for the G heads of this kv head, same lane layout as K rows.
  F qf[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    load_frag(qf[h], static_cast<const T*>(a.q) + (size_t(b) * Hq + kvh * G + h) * D + r * EPL);
  F kn, vn;  // the new token's rows (every row group holds a copy)
  if constexpr (WRITE) {
    if (add_new) {
      const size_t nrow = size_t(kvh) * D + size_t(r) * EPL;
      load_frag(kn, static_cast<const T*>(w.new_k) + size_t(b) * w.k_stride + nrow);
      load_frag(vn, static_cast<const T*>(w.new_v) + size_t(b) * w.v_stride + nrow);
    }
  }

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -FLT_MAX;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.0f;
  }

  const int row_stride = Hkv * D;  // elements between tokens of one block
  const T* kc = static_cast<const T*>(a.k_cache);
  const T* vc = static_cast<const T*>(a.v_cache);
  const int32_t* tbl = a.tables + size_t(b) * a.max_blocks;
  const int c_begin = t0 / kChunk;
  const int c_end = (t1l + kChunk - 1) / kChunk;

  // Issues the loads of chunk c.  Every lane loads: slots past t1 re-read the
  // chunk's first row (always inside the context) and are masked to -inf
  // later, so the loads stay unconditional and the compiler can keep the next
  // chunk's loads in flight while the current one is reduced.
  // Per-lane byte offsets of the four slots inside a chunk (loop invariant).
  uint32_t slot_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    slot_off[i] = uint32_t(((4 * i + grp) * row_stride + r * EPL) * int(sizeof(T)));
  const uint32_t lane_off = uint32_t(r * EPL * int(sizeof(T)));
  // `live` false: the prefetch past a wave's last chunk, which only keeps the
  // loop free of branches; every lane then reads the cache's first 16 bytes
  // (one line per wave instead of re-reading a whole chunk from HBM).
  auto load_chunk = [&](int c, F (&kd)[4], F (&vd)[4], bool live) {
    const int tc = __builtin_amdgcn_readfirstlane(c * kChunk);  // wave-uniform: scalar loads
    int bid = scalar_read(tbl + tc / BS);
    bid = (unsigned)bid < (unsigned)a.num_blocks ? bid : 0;
    const size_t rowbase =
        live ? ((size_t(bid) * BS + (tc % BS)) * row_stride + kvh * D) * sizeof(T) : 0;
    const char* kb = reinterpret_cast<const char*>(kc) + rowbase;
    const char* vb = reinterpret_cast<const char*>(vc) + rowbase;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t off = !live ? 0u : (tc + 4 * i + grp < t1l ? slot_off[i] : lane_off);
      load_frag_stream(kd[i], kb + off);
      load_frag_stream(vd[i], vb + off);
    }
  };

  // Online-softmax update of every query head with chunk c's rows.
  // Online-softmax update with the rows of tokens tc .. tc+15 below thi.
  auto consume_at = [&](int tc, int thi, const F (&kd)[4], const F (&vd)[4]) {
    float s[G][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool valid = tc + 4 * i + grp < thi;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = 0.0f;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int w = 0; w < WORDS; ++w) d = dot2_bf16(qf[h].w[w], kd[i].w[w], d);
        } else {
#pragma unroll
          for (int e = 0; e < EPL; ++e) d = fmaf(elem<T>(qf[h], e), elem<T>(kd[i], e), d);
        }
        d = row_sum16(d) * a.scale_log2;
        s[h][i] = valid ? d : -INFINITY;
      }
    }
    float vv[4][EPL];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < EPL; ++e) vv[i][e] = elem<T>(vd[i], e);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mx = fmaxf(fmaxf(s[h][0], s[h][1]), fmaxf(s[h][2], s[h][3]));
      const float mn = fmaxf(m[h], mx);
      const float alpha = fast_exp2(m[h] - mn);
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = fast_exp2(s[h][i] - mn);
      l[h] = l[h] * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float x = acc[h][e] * alpha;
        x = fmaf(p[0], vv[0][e], x);
        x = fmaf(p[1], vv[1][e], x);
        x = fmaf(p[2], vv[2][e], x);
        x = fmaf(p[3], vv[3][e], x);
        acc[h][e] = x;
      }
      m[h] = mn;
    }
  };

  auto consume = [&](int c, const F (&kd)[4], const F (&vd)[4]) {
    consume_at(c * kChunk, t1l, kd, vd);
  };

  // Two register buffers, alternating.
  F ka[4], va[4], kb2[4], vb2[4];
  int c = c_begin + stream;
  if (c < c_end) {
    load_chunk(c, ka, va, true);
    while (true) {
      bool live = c + S < c_end;
      load_chunk(live ? c + S : c, kb2, vb2, live);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the math
      consume(c, ka, va);
      c += S;
      if (c >= c_end) break;
      live = c + S < c_end;
      load_chunk(live ? c + S : c, ka, va, live);
      __builtin_amdgcn_sched_barrier(0);
      consume(c, kb2, vb2);
      c += S;
      if (c >= c_end) break;
    }
  }

  if constexpr (WRITE) {
    if (add_new) {  // the new token (only slot 0 of row group 0 is below last + 1)
      // Stored only now: a store right after the loads above would wait for
      // them before the first chunk's loads could issue.
      const int bid = tbl[last / BS];
      if (grp == 0 && (unsigned)bid < (unsigned)a.num_blocks) {
        const size_t dst = ((size_t(bid) * BS + last % BS) * Hkv + kvh) * D + size_t(r) * EPL;
        store_frag(const_cast<T*>(kc) + dst, kn);
        store_frag(const_cast<T*>(vc) + dst, vn);
      }
      // Online-softmax update with one row (row group 0's copy; the others
      // score -inf): the same arithmetic as a chunk whose other slots are
      // masked, a quarter of the work.
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = 0.0f;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int x = 0; x < WORDS; ++x) d = dot2_bf16(qf[h].w[x], kn.w[x], d);
        } else {
#pragma unroll
          for (int e = 0; e < EPL; ++e) d = fmaf(elem<T>(qf[h], e), elem<T>(kn, e), d);
        }
        d = row_sum16(d) * a.scale_log2;
        const float sc = grp == 0 ? d : -INFINITY;
        const float mn = fmaxf(m[h], sc);
        const float alpha = fast_exp2(m[h] - mn);
        const float p = fast_exp2(sc - mn);
        l[h] = l[h] * alpha + p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p, elem<T>(vn, e), acc[h][e] * alpha);
        m[h] = mn;
      }
    }
  }

  // Merge the four rows of the wave (lanes r, r+16, r+32, r+48).
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mw = fmaxf(m[h], __shfl_xor(m[h], 16));
    mw = fmaxf(mw, __shfl_xor(mw, 32));
    const float f = fast_exp2(m[h] - mw);
    float lw = l[h] * f;
    lw += __shfl_xor(lw, 16);
    lw += __shfl_xor(lw, 32);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float x = acc[h][e] * f;
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      acc[h][e] = x;
    }
    m[h] = mw;
    l[h] = lw;
  }

  const bool single = nparts == 1;
  // output of query head h of kv head kv (dims d), or its partial
  auto finish = [&](int kv, int h, int d, float o, float mm, float ll) {
    const size_t head = size_t(b) * Hq + size_t(kv) * G + h;
    if (single) {
      store_elem<T>(a.out, head * D + d, o / ll);
    } else {
      const size_t pi = head * a.max_parts + part;
      a.part_o[pi * D + d] = o / ll;
      if (d == 0) {
        a.part_ml[2 * pi] = mm;
        a.part_ml[2 * pi + 1] = ll;
      }
    }
  };

  if constexpr (S == 1) {  // one wave per head: it holds all of the head's tokens
    if (grp == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) finish(kvh, h, r * EPL + e, acc[h][e], m[h], l[h]);
    }
  } else {
    // merge the S streams of each head; wave w holds head w % HG, stream w / HG
    __shared__ float s_o[NW][G][D];
    __shared__ float s_ml[NW][G][2];
    if (grp == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) s_o[wave][h][r * EPL + e] = acc[h][e];
        if (r == 0) {
          s_ml[wave][h][0] = m[h];
          s_ml[wave][h][1] = l[h];
        }
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < HG * G * D; i += NW * 64) {
      const int hh = i / (G * D);  // head of the workgroup
      const int h = (i / D) % G;
      const int d = i % D;
      float M = s_ml[hh][h][0];
#pragma unroll
      for (int s2 = 1; s2 < S; ++s2) M = fmaxf(M, s_ml[hh + s2 * HG][h][0]);
      float L = 0.0f, O = 0.0f;
#pragma unroll
      for (int s2 = 0; s2 < S; ++s2) {
        const int w = hh + s2 * HG;
        const float f = fast_exp2(s_ml[w][h][0] - M);
        L = fmaf(s_ml[w][h][1], f, L);
        O = fmaf(s_o[w][h][d], f, O);
      }
      finish(kvh0 + hh, h, d, O, M, L);
    }
  }
}

// ---------------------------------------------------------------------------
// Partition kernel on the matrix cores (bf16, 1..16 q heads per kv head).
//
// Per 16-token chunk and kv head, with the group's q heads padded to 16:
//   S^T[16 tokens x 16 heads] = K[16 x D] . Q^T[D x 16]    bf16 MFMA 16x16x32
//     (K rows as operand A, q heads as operand B, D/32 steps)
//   O^T[D x 16 heads] += V^T[D x 16 tokens] . P^T[16 x 16] bf16 MFMA 16x16x16
//     (D/16 calls, one per group of 16 output dims)
// Lane l (c = l / 16, n = l % 16) gets the scores of head n for tokens
// 4c..4c+3, exactly the four k entries of P^T it must supply, and it has
// loaded V rows 4c..4c+3 at dims EPL*n .. EPL*n+EPL-1, whose element t of
// each row forms its V^T operand for output tile t (dims EPL*m + t).  So no
// data crosses lanes between the two products: only half-words are packed.
// Lane l accumulates head n's output at dims EPL*(4c + r) + t (r < 4, t <
// EPL), i.e. the contiguous range [4*EPL*c, 4*EPL*(c+1)).
//
// Online softmax with a lazy maximum: a head's reference max m only moves
// when a chunk's score exceeds it by more than 2^8 (in base-2 units), so
// p = 2^(s - m) <= 256 and the accumulator is rescaled only in those rare
// chunks (a wave-uniform branch).  The final division by the sum makes the
// result independent of the reference chosen.  P is rounded to bf16 for the
// second product; sums and accumulators stay fp32.
// The q.K^T k order is permuted identically in both operands (lane group c,
// step j covers dims 8c + 32j .. +7), which leaves the dot product unchanged.

// Load flavours of the matrix-core kernel.  Its V loads read whole 256-byte
// rows per 16 lanes and stream them (non-temporal); its K loads read a 64-byte
// quarter of each row per instruction, so they keep the normal caching that
// lets the next instructions find the rest of the line.
#ifndef PKV_MFMA_K_NT
#define PKV_MFMA_K_NT 0
#endif
#ifndef PKV_MFMA_V_NT
#define PKV_MFMA_V_NT 1
#endif
constexpr bool kMfmaKNT = PKV_MFMA_K_NT;
constexpr bool kMfmaVNT = PKV_MFMA_V_NT;

template <int D, int BS, int NW, int HG, bool WRITE>
__global__ __launch_bounds__(NW * 64) void decode_mfma_kernel(AttnArgs a, NewRows w) {
  constexpr int KSTEPS = D / 32;  // q.K^T MFMA steps over head_dim
  constexpr int EPL = D / 16;     // V elements per lane per token row = PV tiles
  constexpr int VW = EPL / 2;     // 32-bit words per V load
  constexpr int S = NW / HG;      // waves (chunk streams) per kv head
  static_assert(NW % HG == 0, "waves must split evenly over the heads");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane >> 4;
  const int n = lane & 15;
  const int Hq = a.num_q_heads;
  const int Hkv = a.num_kv_heads;
  const int G = Hq / Hkv;
  if (int(blockIdx.z) < w.pf_rows) {  // the next step's upload
    copy_next_step(w);
    return;
  }

  // Shared-prefix rows: a tile of 16 / G members sharing the prefix; its
  // operand columns are (member, query head) pairs, and it computes the
  // members' partition 0 (the prefix) with one read of the prefix's K/V.
  // Grid rows: the upload's first, then the tiles' from group_z0 to
  // group_z1, then the sequences' from seq_z0 + pf_rows.
  const bool group = !WRITE && a.members != nullptr && int(blockIdx.z) >= a.group_z0 &&
                     int(blockIdx.z) < a.group_z1;
  // The tiles' workgroups in launch order: workgroup w takes kv head
  // w % Hkv and tiles NW * (w / Hkv) .. + NW - 1, so with the kv heads in
  // eights every tile of a kv head lands on the same XCD (workgroups are
  // dealt to the 8 XCDs round-robin) and reads the prefix rows the others
  // fetched into its L2.
  const int gw = group ? int(blockIdx.x) + int(gridDim.x) * (int(blockIdx.y) +
                                                             int(gridDim.y) * (int(blockIdx.z) - a.group_z0))
                       : 0;
  const int kvh0 = group ? gw % Hkv : int(blockIdx.y) * HG;  // first kv head
  const int kvh = kvh0 + wave % HG;  // this wave's kv head
  // A tiles' workgroup holds NW tiles of one kv head, one per wave, each
  // wave over the whole prefix: its waves read the same rows, the later ones
  // from L1 (measured on MI355X, GQA batch with 128 of 256 sequences sharing
  // 1,024 tokens: 656.7-658.0 us against 663.3-665.5 with one tile per
  // workgroup and its prefix split over the waves)
  const int stream = group ? 0 : wave / HG;  // this wave's chunk stream
  const int mpg = 16 / G;  // members per tile
  const int tile = group ? (gw / Hkv) * NW + wave : 0;
  const int tile_members = group ? min(mpg, a.num_members - tile * mpg) : 0;
  if (group && tile_members <= 0) return;
  auto member_seq = [&](int i) {
    const int s = a.members[i];
    return (unsigned)s < (unsigned)a.num_seqs ? s : 0;
  };
  const int part = group ? 0 : int(blockIdx.x);
  const int b = group ? member_seq(tile * mpg)
                      : seq_of(a, int(blockIdx.z) - a.seq_z0 - w.pf_rows);

  // The 16 operand columns are the G query heads of this kv head (padded
  // with zero columns); the query sees the sequence's whole context.
  const int fp = group ? a.first_part : first_part_of(a, b);
  const int ctx = group ? min(a.first_part, a.ctx_cap) : clamp_ctx(a, b);
  const int t0 = part_begin(a, fp, part);
  const int t1 = min(ctx, t0 + part_length(a, fp, part));
  const int nparts = group ? 2 : part_count(a, fp, ctx);  // group: partials
  if (!group && a.member_flag != nullptr && part == 0 && nparts >= 2 && a.member_flag[b] != 0)
    return;  // the shared-prefix rows compute this partition
  const int rows = group ? tile_members * G : G;  // valid operand columns
  const bool row_ok = n < rows;
  auto out_row_of = [&](int kv, int r) {  // (sequence, query head) index of column r
    return group ? size_t(member_seq(tile * mpg + r / G)) * Hq + size_t(kv) * G + r % G
                 : size_t(b) * Hq + size_t(kv) * G + r;
  };
  auto out_row = [&](int r) { return out_row_of(kvh, r); };
  if (t0 >= t1) {
    if (ctx == 0 && part == 0)  // nothing visible: zero outputs (HG heads, contiguous)
      for (int i = threadIdx.x; i < HG * rows * D; i += NW * 64)
        store_elem<uint16_t>(a.out, out_row_of(kvh0, 0) * D + i, 0.0f);
    return;
  }
  // Fused write: as in the vector kernel, the chunk loop stops before the new
  // token and the first stream of each head stores it and adds it from the
  // input.
  const int last = ctx - 1;
  const bool own_new = WRITE && last >= t0 && last < t1;
  const int t1l = own_new ? last : t1;  // end of the chunk loop
  const int n_chunks = (t1l + kChunk - 1) / kChunk - t0 / kChunk;
  const bool add_new = own_new && stream == n_chunks % S;  // the stream with the fewest chunks

  // Q^T operand: row n (zeros past the valid rows), dims 8c + 32j .. +7.
  uint4 qop[KSTEPS];
  {
    const uint16_t* qh = static_cast<const uint16_t*>(a.q) + out_row(row_ok ? n : 0) * D + 8 * c;
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j) {
      const uint4 v = *reinterpret_cast<const uint4*>(qh + 32 * j);
      qop[j] = row_ok ? v : make_uint4(0u, 0u, 0u, 0u);
    }
  }

  f32x4_t acc[EPL];
#pragma unroll
  for (int t = 0; t < EPL; ++t) acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m = -FLT_MAX;  // reference max of row n (same in its four lanes)
  float l = 0.0f;      // this lane's share of row n's sum

  const int row_stride = Hkv * D;
  const char* kc = static_cast<const char*>(a.k_cache);
  const char* vc = static_cast<const char*>(a.v_cache);
  const int32_t* tbl = a.tables + size_t(b) * a.max_blocks;
  const int c_begin = t0 / kChunk;
  const int c_end = (t1l + kChunk - 1) / kChunk;

  // Byte offsets inside a chunk: K row of token n (dims 8c + 32j), V row of
  // token 4c + i (dims EPL*n ..).  Masked slots fall back to the chunk's row 0.
  uint32_t koff[KSTEPS], kmask[KSTEPS], voff[4];
#pragma unroll
  for (int j = 0; j < KSTEPS; ++j) {
    kmask[j] = uint32_t((8 * c + 32 * j) * 2);
    koff[j] = uint32_t((n * row_stride + 8 * c + 32 * j) * 2);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) voff[i] = uint32_t(((4 * c + i) * row_stride + EPL * n) * 2);
  const uint32_t vmask = uint32_t(EPL * n * 2);

  struct Regs {
    uint4 k[KSTEPS];
    uint32_t v[4][VW];
  };
  // The new token as the operands of token 0 of a chunk: every lane holds
  // K dims 8c + 32j and V dims EPL*n of the new rows.
  uint4 nk[KSTEPS];
  uint32_t nv[VW];
  if constexpr (WRITE) {
    if (add_new) {
      const char* kn = static_cast<const char*>(w.new_k) + (size_t(b) * w.k_stride + size_t(kvh) * D) * 2;
      const char* vn = static_cast<const char*>(w.new_v) + (size_t(b) * w.v_stride + size_t(kvh) * D) * 2;
#pragma unroll
      for (int j = 0; j < KSTEPS; ++j) nk[j] = load16<false>(kn + kmask[j]);
      if constexpr (VW == 4) {
        const uint4 x = load16<false>(vn + vmask);
        nv[0] = x.x;
        nv[1] = x.y;
        nv[2] = x.z;
        nv[3] = x.w;
      } else {
        const uint2 x = load8<false>(vn + vmask);
        nv[0] = x.x;
        nv[1] = x.y;
      }
    }
  }
  // `live` false: the branch-free prefetch past a wave's last chunk; every
  // lane then reads the cache's first 16 bytes.
  auto load_chunk = [&](int ch, Regs& r, bool live) {
    const int tc = __builtin_amdgcn_readfirstlane(ch * kChunk);
    int bid = scalar_read(tbl + tc / BS);
    bid = (unsigned)bid < (unsigned)a.num_blocks ? bid : 0;
    const size_t rowbase =
        live ? ((size_t(bid) * BS + (tc % BS)) * row_stride + size_t(kvh) * D) * 2 : 0;
    const char* kb = kc + rowbase;
    const char* vb = vc + rowbase;
    const bool kvalid = tc + n < t1l;
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j)
      r.k[j] = load16<kMfmaKNT>(kb + (!live ? 0u : (kvalid ? koff[j] : kmask[j])));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t off = !live ? 0u : (tc + 4 * c + i < t1l ? voff[i] : vmask);
      const char* vsrc = vb + off;
      // the tiles' V loads are cached: the workgroup's other waves read them too
      if constexpr (VW == 4) {
        const uint4 x = group ? load16<false>(vsrc) : load16<kMfmaVNT>(vsrc);
        r.v[i][0] = x.x;
        r.v[i][1] = x.y;
        r.v[i][2] = x.z;
        r.v[i][3] = x.w;
      } else {
        const uint2 x = group ? load8<false>(vsrc) : load8<kMfmaVNT>(vsrc);
        r.v[i][0] = x.x;
        r.v[i][1] = x.y;
      }
    }
  };

  // Online-softmax update with the rows of tokens tc .. tc+15 below thi.
  auto consume_at = [&](int tc, int thi, const Regs& r) {
    f32x4_t s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, r.k[j]),
                                                  __builtin_bit_cast(bf16x8_t, qop[j]), s, 0, 0,
                                                  0);
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = tc + 4 * c + i;
      sc[i] = t < thi ? s[i] * a.scale_log2 : -INFINITY;
    }
    const float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    if (__ballot(mx > m + kLazyMax)) {  // rare: move the reference max
      float hm = fmaxf(mx, __shfl_xor(mx, 16));
      hm = fmaxf(hm, __shfl_xor(hm, 32));
      const float mn = hm > m + kLazyMax ? hm : m;
      const float alpha = fast_exp2(m - mn);
      l *= alpha;
#pragma unroll
      for (int t = 0; t < EPL; ++t) acc[t] *= alpha;
      m = mn;
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(sc[i] - m);
    l += (p[0] + p[1]) + (p[2] + p[3]);
    const uint32_t p01 = pack_bf16x2(p[0], p[1]);
    const uint32_t p23 = pack_bf16x2(p[2], p[3]);
    const s16x4_t pb = __builtin_bit_cast(s16x4_t, make_uint2(p01, p23));
#pragma unroll
    for (int t = 0; t < EPL; ++t) {
      // element t of rows 4c..4c+3 as bf16 pairs: one byte permute per word
      // (bytes 0-1 of the first row's word, then of the second's; 2-3 for odd t)
      const int w = t >> 1;
      const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t lo = __builtin_amdgcn_perm(r.v[1][w], r.v[0][w], sel);
      const uint32_t hi = __builtin_amdgcn_perm(r.v[3][w], r.v[2][w], sel);
      const s16x4_t vb = __builtin_bit_cast(s16x4_t, make_uint2(lo, hi));
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vb, pb, acc[t], 0, 0, 0);
    }
  };

  auto consume = [&](int ch, const Regs& r) { consume_at(ch * kChunk, t1l, r); };

  const int WSTEP = group ? 1 : S;  // chunks between one wave's iterations
  Regs ra, rb;
  int ch = c_begin + stream;
  if (ch < c_end) {
    load_chunk(ch, ra, true);
    while (true) {
      bool live = ch + WSTEP < c_end;
      load_chunk(live ? ch + WSTEP : ch, rb, live);
      __builtin_amdgcn_sched_barrier(0);
      consume(ch, ra);
      ch += WSTEP;
      if (ch >= c_end) break;
      live = ch + WSTEP < c_end;
      load_chunk(live ? ch + WSTEP : ch, ra, live);
      __builtin_amdgcn_sched_barrier(0);
      consume(ch, rb);
      ch += WSTEP;
      if (ch >= c_end) break;
    }
  }
  if constexpr (WRITE) {
    if (add_new) {  // the new token (only token 0 of the chunk is below last + 1)
      // Stored after the loop so the first chunk's loads do not wait for it.
      const int bid = tbl[last / BS];
      if ((unsigned)bid < (unsigned)a.num_blocks) {
        const size_t dst = ((size_t(bid) * BS + last % BS) * row_stride + size_t(kvh) * D) * 2;
        char* kd = const_cast<char*>(kc) + dst;
        char* vd = const_cast<char*>(vc) + dst;
        if (n == 0) {  // lanes 0, 16, 32, 48: K dims 8c + 32j
#pragma unroll
          for (int j = 0; j < KSTEPS; ++j) *reinterpret_cast<uint4*>(kd + kmask[j]) = nk[j];
        }
        if (c == 0) {  // lanes 0 .. 15: V dims EPL*n
          if constexpr (VW == 4)
            *reinterpret_cast<uint4*>(vd + vmask) = make_uint4(nv[0], nv[1], nv[2], nv[3]);
          else
            *reinterpret_cast<uint2*>(vd + vmask) = make_uint2(nv[0], nv[1]);
        }
      }
      Regs rn;
#pragma unroll
      for (int j = 0; j < KSTEPS; ++j) rn.k[j] = nk[j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int x = 0; x < VW; ++x) rn.v[i][x] = nv[x];
      consume_at(last, last + 1, rn);
    }
  }
  // the four lanes of row n hold partial sums of the same reference max
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);

  // acc[t][r] = O[row n][EPL*(4c + r) + t] (unnormalised, this wave's tokens).
  // A row with no visible token in this partition has l = 0 and stores zeros.
  const bool single = nparts == 1;
  auto finish = [&](int kv, int row, int d, float o, float mm, float ll) {
    const float v = ll > 0.0f ? o / ll : 0.0f;
    if (single) {
      store_elem<uint16_t>(a.out, out_row_of(kv, row) * D + d, v);
    } else {
      const size_t pi = out_row_of(kv, row) * a.max_parts + part;
      a.part_o[pi * D + d] = v;
      if (d == 0) {
        a.part_ml[2 * pi] = mm;
        a.part_ml[2 * pi + 1] = ll;
      }
    }
  };
  if (S == 1 || group) {  // this wave holds all of its rows' tokens
    if (row_ok) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < EPL; ++t) finish(kvh, n, EPL * (4 * c + r) + t, acc[t][r], m, l);
    }
  } else {
    // merge the S streams of each head; wave w holds head w % HG, stream w / HG
    __shared__ float s_o[NW][16][D];
    __shared__ float s_ml[NW][16][2];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int t = 0; t < EPL; ++t) s_o[wave][n][EPL * (4 * c + r) + t] = acc[t][r];
    if (c == 0) {
      s_ml[wave][n][0] = m;
      s_ml[wave][n][1] = l;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < HG * rows * D; i += NW * 64) {
      const int hh = i / (rows * D);  // head of the workgroup
      const int h = (i / D) % rows;
      const int d = i % D;
      float M = s_ml[hh][h][0];
#pragma unroll
      for (int s2 = 1; s2 < S; ++s2) M = fmaxf(M, s_ml[hh + s2 * HG][h][0]);
      float L = 0.0f, O = 0.0f;
#pragma unroll
      for (int s2 = 0; s2 < S; ++s2) {
        const int w = hh + s2 * HG;
        const float f = fast_exp2(s_ml[w][h][0] - M);
        L = fmaf(s_ml[w][h][1], f, L);
        O = fmaf(s_o[w][h][d], f, O);
      }
      finish(kvh0 + hh, h, d, O, M, L);
    }
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the partitions of one (sequence, query head).
// out = sum_p w_p o_p / sum_p w_p with w_p = l_p 2^(m_p - max_p m_p).
// Lane p computes partition p's weight (64 partitions at a time); the
// weighted sum then walks the partitions with every lane on its own dims,
// unrolled so that the loads of several partitions are in flight together
// (one partition at a time left the kernel waiting on memory latency).
template <typename T, int D>
__global__ __launch_bounds__(64) void reduce_partitions_kernel(AttnArgs a) {
  constexpr int DPT = D / 64;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int ctx = clamp_ctx(a, b);
  const int nparts = part_count(a, first_part_of(a, b), ctx);
  if (nparts <= 1) return;  // written directly by the partition kernel
  const size_t head = size_t(b) * a.num_q_heads + h;
  const float* ml = a.part_ml + 2 * head * a.max_parts;
  const float* po = a.part_o + head * a.max_parts * D;
  const int t = threadIdx.x;

  float M = -FLT_MAX;
  for (int p = t; p < nparts; p += 64) M = fmaxf(M, ml[2 * p]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));

  float L = 0.0f;
  float O[DPT];
#pragma unroll
  for (int j = 0; j < DPT; ++j) O[j] = 0.0f;
  for (int p0 = 0; p0 < nparts; p0 += 64) {
    const int p = p0 + t;
    const float w = p < nparts ? ml[2 * p + 1] * fast_exp2(ml[2 * p] - M) : 0.0f;
    L += w;
    const int cnt = min(64, nparts - p0);
    const float* pg = po + size_t(p0) * D + t;
    for (int q0 = 0; q0 < cnt; q0 += 8) {
      // eight partitions' loads first (past the count: the last one again,
      // with weight 0), then their products
      float v[8][DPT];
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int j = 0; j < DPT; ++j) v[r][j] = pg[size_t(min(q0 + r, cnt - 1)) * D + j * 64];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float wr = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), min(q0 + r, 63)));
        const float wq = q0 + r < cnt ? wr : 0.0f;
#pragma unroll
        for (int j = 0; j < DPT; ++j) O[j] = fmaf(wq, v[r][j], O[j]);
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
  const float inv = 1.0f / L;
#pragma unroll
  for (int j = 0; j < DPT; ++j) store_elem<T>(a.out, head * D + j * 64 + t, O[j] * inv);
}

// ---------------------------------------------------------------------------
// Host side.
#ifndef PKV_DECODE_WAVES
#define PKV_DECODE_WAVES 4
#endif
constexpr int kNW = PKV_DECODE_WAVES;  // waves per workgroup

// Vector kernel: bf16 with at most 2 query heads per kv head (registers fit
// 16 waves without spilling) uses groups of 4 adjacent kv heads x 4 waves
// each where the kv heads split into fours; else one kv head x 4 waves.
#ifndef PKV_VALU_HG
#define PKV_VALU_HG 4
#endif
#ifndef PKV_VALU_WAVES
#define PKV_VALU_WAVES 16
#endif
constexpr int kValuHG = PKV_VALU_HG;     // adjacent kv heads per workgroup (wide layout)
constexpr int kValuNW = PKV_VALU_WAVES;  // waves per workgroup (wide layout)

template <bool WRITE, typename T, int D, int BS, int G>
hipError_t launch_valu(const AttnArgs& a, const NewRows& w, int num_seqs, hipStream_t st,
                       int grid_parts) {
  if constexpr (sizeof(T) == 2 && G <= 2) {
    if (a.num_kv_heads % 4 == 0) {  // wide_layout() decides the same
      const dim3 grid = work_grid(grid_parts, a.num_kv_heads / kValuHG, num_seqs + w.pf_rows);
      hipLaunchKernelGGL((decode_valu_kernel<T, D, BS, G, kValuNW, kValuHG, WRITE>), grid,
                         dim3(kValuNW * 64), 0, st, a, w);
      return hipGetLastError();
    }
  }
  const dim3 grid = work_grid(grid_parts, a.num_kv_heads, num_seqs + w.pf_rows);
  hipLaunchKernelGGL((decode_valu_kernel<T, D, BS, G, kNW, 1, WRITE>), grid, dim3(kNW * 64), 0, st,
                     a, w);
  return hipGetLastError();
}

#ifndef PKV_MFMA_HG
#define PKV_MFMA_HG 1
#endif
#ifndef PKV_MFMA_WAVES
#define PKV_MFMA_WAVES 4
#endif
constexpr int kMfmaHG = PKV_MFMA_HG;     // adjacent kv heads per workgroup
constexpr int kMfmaNW = PKV_MFMA_WAVES;  // waves per workgroup

template <bool WRITE, int D, int BS>
hipError_t launch_mfma(const AttnArgs& a, const NewRows& w, int num_seqs, hipStream_t st,
                       int grid_parts) {
  if (kMfmaHG > 1 && a.num_kv_heads % kMfmaHG == 0) {
    const dim3 grid = work_grid(grid_parts, a.num_kv_heads / kMfmaHG, num_seqs + w.pf_rows);
    hipLaunchKernelGGL((decode_mfma_kernel<D, BS, kMfmaNW, kMfmaHG, WRITE>), grid,
                       dim3(kMfmaNW * 64), 0, st, a, w);
  } else {
    dim3 grid = work_grid(grid_parts, a.num_kv_heads, num_seqs + w.pf_rows);
    AttnArgs ag = a;
    if (!WRITE && a.members != nullptr && a.num_members > 0) {
      // shared-prefix tiles: grid.x * num_kv_heads workgroups per row, in
      // the rows before the sequences' (measured on MI355X, GQA batch with
      // 128 of 256 sequences sharing 1,024 tokens: 663 us against 666 us with
      // the tiles after the sequences)
      const int mpg = 16 / (a.num_q_heads / a.num_kv_heads);
      const int tiles = (a.num_members + mpg - 1) / mpg;
      const int tile_wgs = (tiles + kNW - 1) / kNW;  // kNW tiles per workgroup
      const int rows = (tile_wgs + int(grid.x) - 1) / int(grid.x);
      // first (after the next step's upload row, if any): the tiles read the
      // prefix while the rest starts
      ag.group_z0 = w.pf_rows;
      ag.group_z1 = w.pf_rows + rows;
      ag.seq_z0 = rows;  // the sequences' rows follow the upload row and the tiles
      grid.z += unsigned(rows);
    }
    hipLaunchKernelGGL((decode_mfma_kernel<D, BS, kNW, 1, WRITE>), grid, dim3(kNW * 64), 0, st, ag,
                       w);
  }
  return hipGetLastError();
}

// Process-wide kernel choice (tests and benchmarks compare the two paths).
int g_decode_path = PKV_PATH_AUTO;

// Matrix cores for bf16 groups of 4..16 query heads per kv head (and for the
// group sizes the vector kernel is not built for); vector ALUs otherwise.
bool use_mfma(bool bf16, int G) {
  if (!bf16) return false;
  const bool valu_ok = G == 1 || G == 2 || G == 4 || G == 8;
  if (g_decode_path == PKV_PATH_VALU && valu_ok) return false;
  if (g_decode_path == PKV_PATH_MFMA) return true;
  if (g_decode_path == PKV_PATH_AUTO) return G >= 4 || !valu_ok;
  return false;
}

// Whether the vector kernel's 4-kv-heads-per-workgroup layout serves a call.
bool wide_layout(bool bf16, int G, int num_kv_heads) {
  return bf16 && G <= 2 && num_kv_heads % 4 == 0 && !use_mfma(true, G);
}

// Partition length of a decode call, 0 = single pass.  AUTO for the 4-heads
// layout: single pass up to 8192 tokens, 4096-token partitions beyond
// (measured on MI355X, 40 heads of 128: single pass is best on the LLaMA-13B
// batch, lengths up to 4096, and equal to partitioned over lengths 2k..8k;
// with one 32k sequence among 127 short ones, 4096-token partitions give 6.5
// TB/s where single pass gives 2.3).  Other kernels: resolve_partition.
// Shared-prefix decode: the partitions after the prefix are the automatic
// length (2048 tokens) or the prefix's, whichever is longer, so there are
// never more partitions than with prefix-length partitions throughout (the
// workspace size the call documents).
int32_t shared_partition(int32_t max_context_len, int32_t prefix_tokens) {
  (void)max_context_len;
  return std::max<int32_t>(PKV_AUTO_PARTITION, prefix_tokens);
}

int32_t decode_partition(bool bf16, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t max_context_len, int32_t partition_size) {
  if (partition_size == PKV_PARTITION_AUTO && num_kv_heads > 0 &&
      num_q_heads % num_kv_heads == 0 && wide_layout(bf16, num_q_heads / num_kv_heads, num_kv_heads))
    return max_context_len > 8192 ? 4096 : 0;
  return resolve_partition(max_context_len, partition_size);
}

template <bool WRITE, typename T, int D, int BS>
hipError_t dispatch_group(const AttnArgs& a, const NewRows& w, int G, int num_seqs,
                          hipStream_t st, int grid_parts) {
  if constexpr (sizeof(T) == 2) {
    if (use_mfma(true, G)) return launch_mfma<WRITE, D, BS>(a, w, num_seqs, st, grid_parts);
  }
  switch (G) {
    case 1: return launch_valu<WRITE, T, D, BS, 1>(a, w, num_seqs, st, grid_parts);
    case 2: return launch_valu<WRITE, T, D, BS, 2>(a, w, num_seqs, st, grid_parts);
    case 4: return launch_valu<WRITE, T, D, BS, 4>(a, w, num_seqs, st, grid_parts);
    case 8: return launch_valu<WRITE, T, D, BS, 8>(a, w, num_seqs, st, grid_parts);
    default: return hipErrorInvalidValue;
  }
}

template <bool WRITE, typename T, int D>
hipError_t dispatch_bs(const AttnArgs& a, const NewRows& w, int BS, int G, int num_seqs,
                       hipStream_t st, int grid_parts) {
  return BS == 16 ? dispatch_group<WRITE, T, D, 16>(a, w, G, num_seqs, st, grid_parts)
                  : dispatch_group<WRITE, T, D, 32>(a, w, G, num_seqs, st, grid_parts);
}

// Every (element type, head_dim) of the attention kernels.
template <bool WRITE>
hipError_t dispatch_all(const AttnArgs& a, const NewRows& w, bool f32, int head_dim, int BS,
                        int G, int num_seqs, hipStream_t st, int grid_parts) {
  if (head_dim == 64)
    return f32 ? dispatch_bs<WRITE, float, 64>(a, w, BS, G, num_seqs, st, grid_parts)
               : dispatch_bs<WRITE, uint16_t, 64>(a, w, BS, G, num_seqs, st, grid_parts);
  return f32 ? dispatch_bs<WRITE, float, 128>(a, w, BS, G, num_seqs, st, grid_parts)
             : dispatch_bs<WRITE, uint16_t, 128>(a, w, BS, G, num_seqs, st, grid_parts);
}

template <typename T, int D>
hipError_t launch_reduce(const AttnArgs& a, int num_seqs, hipStream_t st) {
  hipLaunchKernelGGL((reduce_partitions_kernel<T, D>), dim3(a.num_q_heads, num_seqs), dim3(64),
                     0, st, a);
  return hipGetLastError();
}

bool group_supported(bool bf16, int g) {
  if (g == 1 || g == 2 || g == 4 || g == 8) return true;
  return bf16 && g >= 2 && g <= 16;
}

}  // namespace
}  // namespace pkv

using pkv::fail;

extern "C" pkv_status pkv_set_decode_path(int32_t path) {
  if (path != PKV_PATH_AUTO && path != PKV_PATH_VALU && path != PKV_PATH_MFMA)
    return fail(PKV_ERR_INVALID_ARG, "set_decode_path: unknown path %d", path);
  pkv::g_decode_path = path;
  return pkv::ok();
}

extern "C" int32_t pkv_get_decode_path(void) { return pkv::g_decode_path; }

extern "C" int32_t pkv_decode_partition_size(int32_t, int32_t num_q_heads, int32_t num_kv_heads,
                                             int32_t, int32_t, int32_t max_context_len,
                                             int32_t partition_size, pkv_dtype dtype) {
  return pkv::decode_partition(dtype == PKV_BF16, num_q_heads, num_kv_heads, max_context_len,
                               partition_size);
}

extern "C" size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim,
                                             int32_t block_size, int32_t max_context_len,
                                             int32_t partition_size, pkv_dtype dtype) {
  (void)block_size;
  (void)num_kv_heads;
  (void)dtype;
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  // AUTO: sized for the finest automatic partitioning of any kernel (the
  // vector kernel's 4-heads layout partitions more coarsely or not at all),
  // so the size does not depend on which kernel the call will take
  return pkv::workspace_for(num_seqs, num_q_heads, head_dim, max_context_len,
                            pkv::resolve_partition(max_context_len, partition_size));
}

namespace {

// Decode, optionally with the step's new tokens written first (w non-null):
// the argument checks, partition choice and launches of both entry points.
pkv_status decode_call(const char* fn, void* out, const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* context_lens,
                       const int32_t* seq_order, int32_t max_context_len, int32_t num_seqs,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t num_blocks, float scale,
                       int32_t partition_size, void* workspace, size_t workspace_bytes,
                       pkv_dtype dtype, void* stream, const pkv::NewRows* w,
                       const int32_t* members = nullptr, const int32_t* member_flag = nullptr,
                       int32_t num_members = 0, const pkv::NewRows* upload_only = nullptr) {
  if (dtype != PKV_F32 && dtype != PKV_BF16)
    return fail(PKV_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, int(dtype));
  if (num_seqs < 0 || num_seqs > 65535)
    return fail(PKV_ERR_INVALID_ARG, "%s: num_seqs=%d outside [0, 65535]", fn,
                num_seqs);
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_kv_heads > 65535 ||
      num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG,
                "%s: num_q_heads=%d must be a positive multiple of "
                "num_kv_heads=%d", fn, num_q_heads, num_kv_heads);
  const int G = num_q_heads / num_kv_heads;
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "%s: head_dim=%d (64 or 128)", fn, head_dim);
  if (block_size != 16 && block_size != 32)
    return fail(PKV_ERR_UNSUPPORTED, "%s: block_size=%d (16 or 32)", fn,
                block_size);
  if (!pkv::group_supported(dtype == PKV_BF16, G))
    return fail(PKV_ERR_UNSUPPORTED,
                "%s: query heads per kv head = %d (1..16 for bf16; "
                "1, 2, 4 or 8 for f32)", fn, G);
  if (num_blocks <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0 ||
      max_context_len > (1 << 29))
    return fail(PKV_ERR_INVALID_ARG,
                "%s: num_blocks=%d max_blocks_per_seq=%d "
                "max_context_len=%d", fn, num_blocks, max_blocks_per_seq, max_context_len);
  if (int64_t(num_seqs) * max_blocks_per_seq > INT32_MAX)
    return fail(PKV_ERR_INVALID_ARG, "%s: block table too large", fn);
  if (partition_size < PKV_PARTITION_AUTO ||
      (partition_size > 0 && partition_size % block_size != 0))
    return fail(PKV_ERR_INVALID_ARG,
                "%s: partition_size=%d must be 0, -1 or a multiple of "
                "block_size=%d", fn, partition_size, block_size);
  if (num_seqs == 0) return pkv::ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PKV_ERR_INVALID_ARG, "%s: NULL pointer argument", fn);

  // Shared prefix: a member's partition 0 is the prefix (first_part tokens),
  // its later partitions and every other sequence's partitions are of the
  // shared-prefix length rule (max(2048, prefix) tokens); the workspace and
  // the grid are sized for the members' scheme, which has the most.
  const int32_t first_part = num_members > 0 ? partition_size : 0;
  const int32_t partition =
      first_part > 0 ? pkv::shared_partition(max_context_len, first_part)
                     : pkv::decode_partition(dtype == PKV_BF16, num_q_heads, num_kv_heads,
                                             max_context_len, partition_size);
  const int32_t cap = int32_t(std::min<int64_t>(max_context_len,
                                                int64_t(max_blocks_per_seq) * block_size));
  // partitions of a context of n tokens
  auto parts_of = [&](int64_t n) -> int64_t {
    if (first_part > 0) return n <= first_part ? 1 : 1 + (n - first_part + partition - 1) / partition;
    return (n + partition - 1) / partition;
  };
  pkv::AttnArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.tables = block_tables;
  a.ctx_lens = context_lens;
  a.order = seq_order;
  a.members = num_members > 0 ? members : nullptr;
  a.member_flag = num_members > 0 ? member_flag : nullptr;
  a.num_members = num_members;
  a.group_z0 = num_seqs;
  a.group_z1 = 1 << 30;
  a.seq_z0 = 0;
  a.num_seqs = num_seqs;
  a.max_blocks = max_blocks_per_seq;
  a.ctx_cap = cap;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.num_blocks = num_blocks;
  a.scale_log2 = scale * pkv::kLog2e;
  a.first_part = first_part;
  int grid_parts = 1;
  if (partition > 0) {
    const size_t need =
        first_part > 0 ? size_t(num_seqs) * num_q_heads * size_t(parts_of(max_context_len)) *
                             (size_t(head_dim) + 2) * sizeof(float)
                       : pkv::workspace_for(num_seqs, num_q_heads, head_dim, max_context_len,
                                            partition);
    if (need > 0 && (!workspace || workspace_bytes < need))
      return fail(PKV_ERR_WORKSPACE,
                  "%s: workspace of %zu bytes needed, %zu given", fn, need,
                  workspace ? workspace_bytes : size_t(0));
    a.partition = partition;
    // the workspace is sized from max_context_len; partitions past the clamped
    // context are never launched
    a.max_parts = int32_t(parts_of(max_context_len));
    if (a.max_parts < 1) a.max_parts = 1;
    float* ws = static_cast<float*>(workspace);
    a.part_o = ws;
    a.part_ml = ws + size_t(num_seqs) * num_q_heads * a.max_parts * head_dim;
    grid_parts = int(parts_of(cap));
    if (grid_parts < 1) grid_parts = 1;
    if (grid_parts > 65535)
      return fail(PKV_ERR_INVALID_ARG,
                  "%s: %d partitions of %d tokens exceed the grid limit", fn,
                  grid_parts, partition);
  } else {
    a.partition = pkv::kSingle;
    a.max_parts = 1;
  }

  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool f32 = dtype == PKV_F32;
  hipError_t e =
      w ? pkv::dispatch_all<true>(a, *w, f32, head_dim, block_size, G, num_seqs, st, grid_parts)
        : pkv::dispatch_all<false>(a, upload_only ? *upload_only : pkv::NewRows{}, f32, head_dim,
                                   block_size, G, num_seqs, st, grid_parts);
  if (e == hipSuccess && partition > 0) {
    if (head_dim == 64)
      e = f32 ? pkv::launch_reduce<float, 64>(a, num_seqs, st)
              : pkv::launch_reduce<uint16_t, 64>(a, num_seqs, st);
    else
      e = f32 ? pkv::launch_reduce<float, 128>(a, num_seqs, st)
              : pkv::launch_reduce<uint16_t, 128>(a, num_seqs, st);
  }
  if (e != hipSuccess)
    return fail(PKV_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return pkv::ok();
}

}  // namespace

extern "C" pkv_status pkv_paged_attention_decode(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* seq_order, int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    int32_t partition_size, void* workspace, size_t workspace_bytes, pkv_dtype dtype,
    void* stream) {
  return decode_call("paged_attention_decode", out, q, k_cache, v_cache, block_tables,
                     max_blocks_per_seq, context_lens, seq_order, max_context_len, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                     partition_size, workspace, workspace_bytes, dtype, stream, nullptr);
}

namespace {

// The next step's upload within a decode launch: checks the buffers and
// fills w's upload fields (one more grid row of workgroups, dispatched
// first).  next_bytes = 0: no upload.
pkv_status next_step_upload(const char* fn, void* next_dst, const void* next_src_host,
                            size_t next_bytes, int32_t num_seqs, pkv::NewRows& w) {
  if (next_bytes == 0) return pkv::ok();
  if (!next_dst || !next_src_host || next_bytes % 16 ||
      (reinterpret_cast<uintptr_t>(next_dst) & 15u) ||
      (reinterpret_cast<uintptr_t>(next_src_host) & 15u))
    return fail(PKV_ERR_INVALID_ARG,
                "%s: the next step's upload needs non-NULL 16-byte aligned buffers and a "
                "multiple of 16 bytes (%zu)", fn, next_bytes);
  if (num_seqs <= 0 || num_seqs > 65534)
    return fail(PKV_ERR_INVALID_ARG,
                "%s: the next step's upload needs 1 .. 65534 sequences (its grid row comes "
                "first), got %d", fn, num_seqs);
  void* src_dev = pkv::mapped_host(const_cast<void*>(next_src_host));
  if (!src_dev)
    return fail(PKV_ERR_INVALID_ARG, "%s: next_src_host is not pinned, device-mapped host memory",
                fn);
  w.pf_src = static_cast<const uint4*>(src_dev);
  w.pf_dst = static_cast<uint4*>(next_dst);
  w.pf_n16 = int64_t(next_bytes / 16);
  w.pf_rows = 1;
  return pkv::ok();
}

// The shared-prefix decode, optionally with the next step's upload.
pkv_status shared_prefix_call(const char* fn, void* out, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* context_lens,
                              const int32_t* seq_order, int32_t max_context_len,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              float scale, const int32_t* members, const int32_t* member_flag,
                              int32_t num_members, int32_t prefix_tokens, void* workspace,
                              size_t workspace_bytes, void* next_dst, const void* next_src_host,
                              size_t next_bytes, pkv_dtype dtype, void* stream) {
  if (dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "%s: bf16 only", fn);
  if (num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads != 0 ||
      !pkv::use_mfma(true, num_q_heads / num_kv_heads) || pkv::kMfmaHG != 1)
    return fail(PKV_ERR_UNSUPPORTED,
                "%s: needs the matrix-core kernel (grouped query heads, %d / %d)", fn,
                num_q_heads, num_kv_heads);
  if (num_members < 0 || num_members > num_seqs)
    return fail(PKV_ERR_INVALID_ARG, "%s: num_members=%d outside [0, num_seqs=%d]", fn,
                num_members, num_seqs);
  if (num_members > 0 && (!members || !member_flag))
    return fail(PKV_ERR_INVALID_ARG, "%s: NULL members or member_flag", fn);
  const int32_t mpg = 16 / (num_q_heads / num_kv_heads);
  const int64_t upload_rows = next_bytes > 0 ? 1 : 0;
  if (int64_t(num_seqs) + (int64_t(num_members) + mpg - 1) / mpg + upload_rows > 65535)
    return fail(PKV_ERR_INVALID_ARG, "%s: %d sequences and %d members exceed the grid", fn,
                num_seqs, num_members);
  if (prefix_tokens <= 0 || block_size <= 0 || prefix_tokens % block_size != 0 ||
      prefix_tokens % pkv::kChunk != 0 || prefix_tokens > max_context_len)
    return fail(PKV_ERR_INVALID_ARG,
                "%s: prefix_tokens=%d must be a positive multiple of block_size=%d and of %d, "
                "at most max_context_len=%d", fn, prefix_tokens, block_size, pkv::kChunk,
                max_context_len);
  pkv::NewRows w{};
  const pkv_status st = next_step_upload(fn, next_dst, next_src_host, next_bytes, num_seqs, w);
  if (st != PKV_OK) return st;
  return decode_call(fn, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                     context_lens, seq_order, max_context_len, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, scale, prefix_tokens,
                     workspace, workspace_bytes, dtype, stream, nullptr, members, member_flag,
                     num_members, &w);
}

}  // namespace

extern "C" pkv_status pkv_paged_attention_decode_shared_prefix(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* seq_order, int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    const int32_t* members, const int32_t* member_flag, int32_t num_members,
    int32_t prefix_tokens, void* workspace, size_t workspace_bytes, pkv_dtype dtype,
    void* stream) {
  return shared_prefix_call("paged_attention_decode_shared_prefix", out, q, k_cache, v_cache,
                            block_tables, max_blocks_per_seq, context_lens, seq_order,
                            max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim,
                            block_size, num_blocks, scale, members, member_flag, num_members,
                            prefix_tokens, workspace, workspace_bytes, nullptr, nullptr, 0, dtype,
                            stream);
}

extern "C" pkv_status pkv_paged_attention_decode_shared_prefix_step(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* seq_order, int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    const int32_t* members, const int32_t* member_flag, int32_t num_members,
    int32_t prefix_tokens, void* workspace, size_t workspace_bytes, void* next_dst,
    const void* next_src_host, size_t next_bytes, pkv_dtype dtype, void* stream) {
  return shared_prefix_call("paged_attention_decode_shared_prefix_step", out, q, k_cache,
                            v_cache, block_tables, max_blocks_per_seq, context_lens, seq_order,
                            max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim,
                            block_size, num_blocks, scale, members, member_flag, num_members,
                            prefix_tokens, workspace, workspace_bytes, next_dst, next_src_host,
                            next_bytes, dtype, stream);
}

namespace {

// The decode step with its cache write, and optionally the next step's
// upload, in one launch: the checks of both entry points.  rows_optional:
// new_key and new_value both NULL mean a step without new tokens (no cache
// write, the attention of pkv_paged_attention_decode).
pkv_status decode_write_call(const char* fn, bool rows_optional, void* out, const void* q,
                             const void* new_key, const void* new_value, int64_t key_seq_stride,
                             int64_t value_seq_stride, void* k_cache, void* v_cache,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, const int32_t* seq_order,
                             int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, float scale, int32_t partition_size,
                             void* workspace, size_t workspace_bytes, void* next_dst,
                             const void* next_src_host, size_t next_bytes, pkv_dtype dtype,
                             void* stream) {
  const int64_t esize = dtype == PKV_F32 ? 4 : 2;
  const int64_t row = int64_t(num_kv_heads) * head_dim;
  const bool write = !rows_optional || new_key || new_value;
  if (num_seqs > 0 && write && (!new_key || !new_value))
    return fail(PKV_ERR_INVALID_ARG, "%s: NULL new key/value", fn);
  if (write && (key_seq_stride < row || value_seq_stride < row || (key_seq_stride * esize) % 16 ||
      (value_seq_stride * esize) % 16 || (reinterpret_cast<uintptr_t>(new_key) & 15u) ||
      (reinterpret_cast<uintptr_t>(new_value) & 15u) ||
      (reinterpret_cast<uintptr_t>(k_cache) & 15u) || (reinterpret_cast<uintptr_t>(v_cache) & 15u)))
    return fail(PKV_ERR_INVALID_ARG,
                "%s: sequence strides (%lld, %lld) must be >= %lld "
                "elements and multiples of 16 bytes, pointers 16-byte aligned", fn,
                (long long)key_seq_stride, (long long)value_seq_stride, (long long)row);
  pkv::NewRows w{new_key, new_value, key_seq_stride, value_seq_stride, nullptr, nullptr, 0, 0};
  const pkv_status st = next_step_upload(fn, next_dst, next_src_host, next_bytes, num_seqs, w);
  if (st != PKV_OK) return st;
  return decode_call(fn, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                     context_lens, seq_order, max_context_len, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, scale, partition_size,
                     workspace, workspace_bytes, dtype, stream, write ? &w : nullptr, nullptr,
                     nullptr, 0, write ? nullptr : &w);
}

}  // namespace

extern "C" pkv_status pkv_paged_attention_decode_write(
    void* out, const void* q, const void* new_key, const void* new_value,
    int64_t key_seq_stride, int64_t value_seq_stride, void* k_cache, void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* seq_order, int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    int32_t partition_size, void* workspace, size_t workspace_bytes, pkv_dtype dtype,
    void* stream) {
  return decode_write_call("paged_attention_decode_write", false, out, q, new_key, new_value,
                           key_seq_stride, value_seq_stride, k_cache, v_cache, block_tables,
                           max_blocks_per_seq, context_lens, seq_order, max_context_len, num_seqs,
                           num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                           partition_size, workspace, workspace_bytes, nullptr, nullptr, 0, dtype,
                           stream);
}

extern "C" pkv_status pkv_paged_attention_decode_step(
    void* out, const void* q, const void* new_key, const void* new_value,
    int64_t key_seq_stride, int64_t value_seq_stride, void* k_cache, void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* seq_order, int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    int32_t partition_size, void* workspace, size_t workspace_bytes, void* next_dst,
    const void* next_src_host, size_t next_bytes, pkv_dtype dtype, void* stream) {
  return decode_write_call("paged_attention_decode_step", true, out, q, new_key, new_value,
                           key_seq_stride, value_seq_stride, k_cache, v_cache, block_tables,
                           max_blocks_per_seq, context_lens, seq_order, max_context_len, num_seqs,
                           num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                           partition_size, workspace, workspace_bytes, next_dst, next_src_host,
                           next_bytes, dtype, stream);
}

// ---------------------------------------------------------------------------
// Decode without a caller workspace, for callers that cannot allocate (code
// under graph capture, tight serving loops): the split-K partials live in a
// static device array of PKV_NOALLOC_SCRATCH_BYTES, one per GPU for the life
// of the process.  Host code never passes the array's name to a kernel (on
// the host it is only a stand-in); it looks up the array's device address
// once per device, with that device current, and passes that.
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the
// first call on that device).
pkv_status scratch_of_current_device(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(PKV_ERR_HIP, "%s: no current device (%s)", fn, hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(PKV_ERR_HIP, "%s: device address of the scratch array on device %d: %s", fn,
                  dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return pkv::ok();
}

}  // namespace

extern "C" pkv_status pkv_paged_attention_decode_noalloc(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* seq_order, int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    int32_t partition_size, pkv_dtype dtype, void* stream) {
  const char* fn = "paged_attention_decode_noalloc";
  void* ws = nullptr;
  const pkv_status st = scratch_of_current_device(fn, &ws);
  if (st != PKV_OK) return st;
  // the same checks and launches as pkv_paged_attention_decode, with the
  // scratch array as a workspace of its fixed size (a larger need is
  // refused with PKV_ERR_WORKSPACE before any launch)
  return decode_call(fn, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                     context_lens, seq_order, max_context_len, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, scale, partition_size, ws,
                     size_t(PKV_NOALLOC_SCRATCH_BYTES), dtype, stream, nullptr);
}
