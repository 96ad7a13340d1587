// Chunked prefill for gfx950: several new tokens of each sequence attend,
// causally, to its paged context (long prompts are processed in pieces so
// that one large prefill does not stall the decoding sequences: "Serving
// models with vLLM", section "How it works: continuous batching").  Query i
// of a chunk of n sits at position ctx - n + i and sees tokens 0 .. that
// position; the K/V rows are reached through the block table as in decode
// ("vLLM in Production …", section "PagedAttention — Virtual Memory for the
// KV Cache").
//
// Both products are dense tile contractions and run on the matrix cores; the
// K/V chunk a workgroup reads from HBM is shared by all of its query tiles
// through LDS.
#include "attn_common.h"

// Tokens of K/V staged in LDS per barrier by 8-wave workgroups (a multiple
// of 32).  Measured on MI355X (16 sequences x 40 heads of 128, 512-token
// chunks): 32 tokens 738 TFLOP/s, 64 tokens 761, 96 713, 128 722; two
// 32-token passes of the products per barrier halve the barriers.
#ifndef PKV_PREFILL_CHUNK
#define PKV_PREFILL_CHUNK 64
#endif
// Register stages of the K/V prefetch (chunks in flight per workgroup; even;
// 0 = 128 tokens in flight).
#ifndef PKV_PREFILL_STAGES
#define PKV_PREFILL_STAGES 0
#endif

namespace pkv {
namespace {

// ---------------------------------------------------------------------------
// Chunked prefill on the matrix cores, K/V shared through LDS.
//
// A workgroup of NWP waves owns NWP * TPW query tiles of one (sequence, kv
// head, partition); a tile is 16 (query, head) rows, floor(16 / G)
// consecutive queries times the G query heads of the kv head, the 16 operand
// columns of the matrix products (the decode kernel's layout, with queries
// added), and each wave owns TPW consecutive tiles.  Each K/V chunk (64
// tokens for 8-wave workgroups, 32 for 4-wave ones) is loaded once by the
// whole workgroup — whole rows, cached in L2 for the kv head's other
// workgroups (placed on the same XCD) — into a double-buffered LDS tile,
// one barrier per chunk; every wave reads each K and V operand from LDS once
// and uses it for all of its tiles (LDS reads per flop fall with TPW).  The
// products run over the chunk in 32-token passes, both on 32-deep matrix
// instructions: q.K^T over head_dim, and P.V over the pass's 32 tokens, its
// V operand read transposed from LDS.  The q.K^T products of one k step are
// issued together (2 * TPW independent chains); the softmax keeps its running
// maximum from the raw products and applies the scale inside the exponent
// (p = 2^(s * |scale| - m), one fma per score).
// The next chunks' loads are in flight while the current one is computed.
// Tiles that see no token of a chunk (the causal boundary) skip its math;
// their waves keep to the barriers.
// Grid row y -> (kv head, query-tile group).  With the kv heads in eights,
// the groups of one kv head sit 8 workgroups apart: the dispatcher deals
// workgroups to the 8 XCDs round-robin, so they land on one XCD back to back,
// stream the same K/V rows at about the same time and the later ones find
// them in that XCD's L2 (measured on MI355X, 16 sequences x 40 heads x
// 512-token chunks, two groups per kv head: HBM reads 1.46x the K/V bytes
// with the groups 40 workgroups apart and non-temporal loads, 0.98x paired
// with cached loads, and 5% faster).
__device__ __forceinline__ void prefill_group_of(const AttnArgs& a, int y, int& kvh, int& grp) {
  if (a.num_kv_heads % 8 == 0) {
    const int groups = a.q_groups;
    const int blk = y / (8 * groups);  // block of 8 kv heads
    const int r = y % (8 * groups);
    kvh = blk * 8 + r % 8;
    grp = r / 8;
  } else {
    kvh = y % a.num_kv_heads;
    grp = y / a.num_kv_heads;
  }
}

template <int D, int BS, int NWP, int TPW>
__global__ __launch_bounds__(NWP * 64) void prefill_lds_kernel(AttnArgs a) {
  constexpr int KSTEPS = D / 32;
  constexpr int EPL = D / 16;
  constexpr int RB = D * 2;            // bytes of one token's K (or V) row
  // LDS row pitch (bytes), chosen from measured bank conflicts on gfx950
  // for 256-byte rows: at 288 bytes both operand reads are conflict-free —
  // the K read (ds_read_b128, lane (c, n): row n, bytes 16c + 64j; twice as
  // long at 272) and the transposing V read (ds_read_b64_tr_b16, rows 4c +
  // k/4; 8x as long unpadded) — and the chunk stores run at full write rate.
  constexpr int PITCH_K = D == 128 ? RB + 32 : RB + 16;
  constexpr int PITCH_V = PITCH_K;
  // tokens per K/V chunk (one barrier each): 4-wave workgroups keep 32, as
  // their lanes would need twice the staging registers for longer chunks
  constexpr int CH = NWP >= 8 ? PKV_PREFILL_CHUNK : 32;
  constexpr int SUB = 32;              // tokens per pass of the products
  static_assert(CH % SUB == 0, "a chunk is whole passes");
  constexpr int NBC = CH / BS;         // cache blocks per chunk
  static_assert(CH % BS == 0, "a chunk covers whole blocks");
  constexpr int LPR = RB / 16;         // 16-byte pieces per row
  constexpr int PIECES = CH * LPR;     // pieces per chunk, per cache
  __shared__ __attribute__((aligned(16))) char s_k[2][CH * PITCH_K];  // [buffer]
  __shared__ __attribute__((aligned(16))) char s_v[2][CH * PITCH_V];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane >> 4;
  const int n = lane & 15;
  const int part = blockIdx.x;
  int kvh_, grp_;
  prefill_group_of(a, int(blockIdx.y), kvh_, grp_);
  const int kvh = kvh_;
  const int grp = grp_;
  const int tile0 = (grp * NWP + wave) * TPW;  // first own tile
  const int b = seq_of(a, blockIdx.z);
  const int Hq = a.num_q_heads;
  const int Hkv = a.num_kv_heads;
  const int G = Hq / Hkv;
  const int QPT = 16 / G > 0 ? 16 / G : 1;

  const int ctx = clamp_ctx(a, b);
  int qrow0, nq;
  query_range(a, b, qrow0, nq);
  // workgroup-wide token range: the causal end of its last tile with queries
  const int g_first = grp * NWP * TPW * QPT;
  if (g_first >= nq) return;  // uniform over the workgroup
  const int g_last = min(g_first + NWP * TPW * QPT, nq) - 1;
  const int t0 = part * a.partition;
  const int g_end = max(0, ctx - nq + g_last + 1);
  const int g_t1 = min(g_end, t0 + a.partition);

  // this wave's tiles (all fields wave-uniform except the per-lane row ones)
  int q_first[TPW], t_end[TPW], t1[TPW], rows[TPW], pos_n[TPW], pos_lo[TPW];
  bool has_tile[TPW], row_ok[TPW];
  int t1_max = 0;
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    q_first[u] = (tile0 + u) * QPT;
    has_tile[u] = q_first[u] < nq;
    const int q_last = has_tile[u] ? min(q_first[u] + QPT, nq) - 1 : q_first[u];
    t_end[u] = has_tile[u] ? max(0, ctx - nq + q_last + 1) : 0;
    t1[u] = min(t_end[u], t0 + a.partition);
    t1_max = max(t1_max, t1[u]);
    rows[u] = has_tile[u] ? (q_last - q_first[u] + 1) * G : 0;
    row_ok[u] = n < rows[u];
    const int qi = q_first[u] + (row_ok[u] ? n / G : 0);
    pos_n[u] = row_ok[u] ? ctx - nq + qi : -1;
    pos_lo[u] = ctx - nq + q_first[u];  // position of the tile's first query
  }
  auto out_row = [&](int u, int r) {
    return (size_t(qrow0) + q_first[u] + r / G) * Hq + size_t(kvh) * G + r % G;
  };
  auto zero_tile = [&](int u) {
    for (int i = lane; i < rows[u] * D; i += 64)
      store_elem<uint16_t>(a.out, out_row(u, i / D) * D + i % D, 0.0f);
  };
  if (t0 >= g_t1) {  // uniform: no token of this partition for any tile
    if (part == 0)
#pragma unroll
      for (int u = 0; u < TPW; ++u)
        if (has_tile[u] && t_end[u] == 0) zero_tile(u);
    return;
  }

  // logits = scale * (q . k): with a negative scale the q operand is negated
  // (exact in bf16) and |scale| used, so that the largest product is the
  // largest logit; a zero scale becomes the smallest normal float, which
  // leaves every weight 2^0 = 1 as it should
  const bool neg_scale = a.scale_log2 < 0.0f;
  const float sp = neg_scale ? -a.scale_log2 : (a.scale_log2 > 0.0f ? a.scale_log2 : FLT_MIN);
  const uint32_t qsign = neg_scale ? 0x80008000u : 0u;
  uint4 qop[TPW][KSTEPS];
  f32x4_t acc[TPW][EPL];
  float m[TPW], l[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const uint16_t* qh =
        static_cast<const uint16_t*>(a.q) + out_row(u, row_ok[u] ? n : 0) * D + 8 * c;
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j) {
      uint4 v = row_ok[u] ? *reinterpret_cast<const uint4*>(qh + 32 * j)
                          : make_uint4(0u, 0u, 0u, 0u);
      v.x ^= qsign;
      v.y ^= qsign;
      v.z ^= qsign;
      v.w ^= qsign;
      qop[u][j] = v;
    }
#pragma unroll
    for (int t = 0; t < EPL; ++t) acc[u][t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    m[u] = -FLT_MAX;
    l[u] = 0.0f;
  }

  const int row_stride = Hkv * D;
  const char* kc = static_cast<const char*>(a.k_cache);
  const char* vc = static_cast<const char*>(a.v_cache);
  const int32_t* tbl = a.tables + size_t(b) * a.max_blocks;
  const int c_begin = t0 / CH;
  const int c_end = (g_t1 + CH - 1) / CH;

  // Cooperative chunk load: piece p (< 2 * PIECES) of the chunk is 16 bytes of
  // K (p < PIECES) or V, token p % PIECES / LPR, bytes 16 * (p % LPR).
  constexpr int PER_LANE = (2 * PIECES + NWP * 64 - 1) / (NWP * 64);
  using Stage = uint4[PER_LANE];
  // Per piece, the parts of its address that do not change from chunk to
  // chunk: the cache, the block of the chunk it falls in, and its byte offset
  // inside that block (and the same for the chunk's first row, which pieces
  // past the end of the range re-read).
  const char* pbase[PER_LANE];
  int ptok[PER_LANE];
  uint32_t poff[PER_LANE], poff0[PER_LANE];
#pragma unroll
  for (int k = 0; k < PER_LANE; ++k) {
    // every lane loads (lanes past the chunk's pieces re-read piece 0 and
    // store nothing), so no lane-masked branch hides the loads from the
    // compiler's wait-count tracking
    const int p0 = threadIdx.x + k * NWP * 64;
    const int p = p0 < 2 * PIECES ? p0 : 0;
    const int pp = p % PIECES;
    ptok[k] = pp / LPR;
    pbase[k] = p < PIECES ? kc : vc;
    poff0[k] = uint32_t((size_t(kvh) * D) * 2 + 16 * (pp % LPR));
    poff[k] = poff0[k] + uint32_t((ptok[k] % BS) * row_stride * 2);
  }
  // `live` false: the prefetch past the last chunk, issued anyway so that no
  // branch hides the loads from the wait-count tracking; every lane then
  // reads the cache's first 16 bytes (one line per wave).
  auto fetch = [&](int ch, Stage& stage, bool live) {
    const int tc = __builtin_amdgcn_readfirstlane(ch * CH);
    // the chunk's blocks (entries past the range repeat its first block, so
    // no table entry beyond the context is read)
    const int last_blk = (g_t1 - 1) / BS;
    size_t blk[NBC];
#pragma unroll
    for (int j = 0; j < NBC; ++j) {
      int bid = scalar_read(tbl + min(tc / BS + j, last_blk));
      bid = (unsigned)bid < (unsigned)a.num_blocks ? bid : 0;
      blk[j] = live ? size_t(bid) * BS * row_stride * 2 : 0;
    }
#pragma unroll
    for (int k = 0; k < PER_LANE; ++k) {
      // rows past the range re-read the chunk's first row (masked later)
      const bool in = tc + ptok[k] < g_t1;
      const size_t b0 = NBC > 1 && in ? blk[ptok[k] / BS] : blk[0];
      const uint32_t off = !live ? 0u : (in ? poff[k] : poff0[k]);
      // cached loads: the other query-tile groups of this kv head read the
      // same rows from L2 shortly after
      stage[k] = load16<false>(pbase[k] + b0 + off);
    }
  };
  auto store = [&](int buf, const Stage& stage) {
#pragma unroll
    for (int k = 0; k < PER_LANE; ++k) {
      const int p = threadIdx.x + k * NWP * 64;
      if (p < 2 * PIECES) {
        const int pp = p % PIECES;
        char* dst = p < PIECES ? &s_k[buf][(pp / LPR) * PITCH_K] : &s_v[buf][(pp / LPR) * PITCH_V];
        *reinterpret_cast<uint4*>(dst + 16 * (pp % LPR)) = stage[k];
      }
    }
  };

  // S^T = K . Q^T for every tile and each 16-token half h of a 32-token pass,
  // each K operand read once; the k step outermost, so the 2 * TPW products
  // of one step are independent
  auto qk = [&](const char* ks, f32x4_t (&s)[TPW][2]) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) s[u][0] = s[u][1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j) {
      bf16x8_t kop[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
        kop[h] = __builtin_bit_cast(
            bf16x8_t,
            *reinterpret_cast<const uint4*>(ks + (16 * h + n) * PITCH_K + 16 * c + 64 * j));
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int u = 0; u < TPW; ++u)
          s[u][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              kop[h], __builtin_bit_cast(bf16x8_t, qop[u][j]), s[u][h], 0, 0, 0);
    }
  };
  // Tile u's scores of the pass at token tc: the raw products (masked: -inf)
  // into sc, and the running maximum moved (with the rescale) where a score
  // passed it by more than 2^kLazyMax.
  auto scores = [&](int tc, int u, const f32x4_t (&su)[2], float (&sc)[8]) {
    // sc[4h + i]: token tc + 16h + 4c + i of query row n
    if (tc >= t0 && tc + SUB <= t1[u] && tc + SUB - 1 <= pos_lo[u]) {  // all visible
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[4 * h + i] = su[h][i];
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = tc + 16 * h + 4 * c + i;
          sc[4 * h + i] = (t >= t0 && t < t1[u] && t <= pos_n[u]) ? su[h][i] : -INFINITY;
        }
    }
    const float mx = vmax(vmax(vmax(sc[0], sc[1]), vmax(sc[2], sc[3])),
                          vmax(vmax(sc[4], sc[5]), vmax(sc[6], sc[7]))) * sp;
    if (__ballot(mx > m[u] + kLazyMax)) {
      float hm = fmaxf(mx, __shfl_xor(mx, 16));
      hm = fmaxf(hm, __shfl_xor(hm, 32));
      const float mn = hm > m[u] + kLazyMax ? hm : m[u];
      const float alpha = fast_exp2(m[u] - mn);
      l[u] *= alpha;
#pragma unroll
      for (int t = 0; t < EPL; ++t) acc[u][t] *= alpha;
      m[u] = mn;
    }
  };
  // The weights p = 2^(s |scale| - m) of tile u, added to its sum and packed
  // to bf16 as the P^T operand.
  auto weights = [&](int u, const float (&sc)[8]) {
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = fast_exp2(fmaf(sc[i], sp, -m[u]));
    l[u] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    return __builtin_bit_cast(
        bf16x8_t, make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                             pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])));
  };
  // O^T += V^T . P^T, tile by tile (one tile's V operand live at a time).
  // The V^T operand of output tile t (dims 16t .. 16t+15) over the pass's 32
  // tokens has k-slots 8c .. 8c+7 = tokens 4c .. 4c+3 and 16+4c .. 16+4c+3,
  // the tokens whose scores lane (c, n) holds.  It comes straight from LDS
  // with the transposing read: in each 16-lane group, lane k reads 8 bytes
  // of row r0 + k/4 at dims 16t + 4(k%4), and lane j receives element j%4 of
  // the reads of lanes j/4, j/4 + 4, + 8, + 12, i.e. dim 16t + j of rows
  // r0 .. r0+3.
  auto pv = [&](const char* vs, const bf16x8_t (&pb)[TPW]) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s* lds_v4s;
    const char* vrow = vs + (4 * c + (n >> 2)) * PITCH_V + 8 * (n & 3);
#pragma unroll
    for (int t = 0; t < EPL; ++t) {
      const uint2 lo = __builtin_bit_cast(
          uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(vrow + 32 * t)));
      const uint2 hi = __builtin_bit_cast(
          uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(vrow + 16 * PITCH_V + 32 * t)));
      const bf16x8_t vb = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
      for (int u = 0; u < TPW; ++u)
        acc[u][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, pb[u], acc[u][t], 0, 0, 0);
    }
  };
  constexpr int NP = CH / SUB;  // 32-token passes per chunk
  const bf16x8_t pzero = __builtin_bit_cast(bf16x8_t, make_uint4(0u, 0u, 0u, 0u));

  auto compute = [&](int ch, int buf) {
#pragma unroll
    for (int sb = 0; sb < NP; ++sb) {
      const int tc = ch * CH + sb * SUB;
      if (tc >= t1_max) break;  // none of this wave's tiles sees a token from here on
      f32x4_t s[TPW][2];
      qk(s_k[buf] + sb * SUB * PITCH_K, s);
      bf16x8_t pb[TPW];
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        if (tc >= t1[u]) {  // wave-uniform: the tile adds nothing (every V row in LDS is finite)
          pb[u] = pzero;
          continue;
        }
        float sc[8];
        scores(tc, u, s[u], sc);
        pb[u] = weights(u, sc);
      }
      pv(s_v[buf] + sb * SUB * PITCH_V, pb);
    }
  };

  // Pipeline, prefetch distance NST (4 chunks of 32 tokens or 2 of 64: 128
  // tokens either way): the global loads of chunk x + NST are issued before
  // chunk x is computed and reach LDS only after chunk x + NST - 1 is
  // computed.  With one 32-token chunk in flight the loads, not the math, set
  // the pace (measured: 2.3x slower than the same kernel without global
  // loads): a workgroup needs tens of KB in flight to cover the memory
  // latency (128 tokens are 64 KB per workgroup at head_dim 128).  NST
  // register stages rotate; two LDS buffers alternate by the chunk's parity;
  // one barrier per chunk.  The loop starts NST chunks early (those steps
  // only fetch and store), so every fetch comes from the same loop body.
  // the query operands (loaded above) are complete before the pipeline
  // starts, so no wait inside it has to cover them
  __builtin_amdgcn_s_waitcnt(0);
  constexpr int NST = PKV_PREFILL_STAGES > 0 ? PKV_PREFILL_STAGES : (CH >= 64 ? 2 : 4);
  static_assert(NST % 2 == 0, "chunk x uses LDS buffer (x - c_begin) % 2 in every round");
  Stage st[NST];
  // step of chunk x (its register stage `mine`, the next chunk's `next`)
  auto step = [&](int x, Stage& mine, const Stage& next, int buf) {
    fetch(x + NST < c_end ? x + NST : c_begin, mine, x + NST < c_end);
    if (x >= c_begin) compute(x, buf);
    if (x + 1 >= c_begin && x + 1 < c_end) store(buf ^ 1, next);
    __syncthreads();
  };
  for (int x = c_begin - NST; x < c_end; x += NST) {
#pragma unroll
    for (int k = 0; k < NST; ++k) {
      step(x + k, st[k], st[(k + 1) % NST], k & 1);
      if (x + k + 1 >= c_end) break;
    }
  }

#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    float lu = l[u];
    lu += __shfl_xor(lu, 16);
    lu += __shfl_xor(lu, 32);
    if (!has_tile[u]) continue;
    if (t_end[u] == 0) {  // every query of this tile sits before position 0
      if (part == 0) zero_tile(u);
      continue;
    }
    const int nparts = (t_end[u] + a.partition - 1) / a.partition;
    if (part >= nparts) continue;
    const bool single = nparts == 1;
    if (row_ok[u]) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < EPL; ++t) {
          const int d = 16 * t + 4 * c + r;  // row 4c + r of output tile t
          const float o = lu > 0.0f ? acc[u][t][r] / lu : 0.0f;
          if (single) {
            store_elem<uint16_t>(a.out, out_row(u, n) * D + d, o);
          } else {
            const size_t pi = out_row(u, n) * a.max_parts + part;
            a.part_o[pi * D + d] = o;
            if (d == 0) {
              a.part_ml[2 * pi] = m[u];
              a.part_ml[2 * pi + 1] = lu;
            }
          }
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the partitions of one prefill query tile (its valid
// (query, head) rows), the same weights as the decode merge below.
template <int D>
__global__ __launch_bounds__(256) void merge_prefill_kernel(AttnArgs a) {
  const int kvh = int(blockIdx.y) % a.num_kv_heads;
  const int tile = int(blockIdx.y) / a.num_kv_heads;
  const int b = blockIdx.z;
  const int Hq = a.num_q_heads;
  const int G = Hq / a.num_kv_heads;
  const int QPT = 16 / G > 0 ? 16 / G : 1;
  const int ctx = clamp_ctx(a, b);
  int qrow0, nq;
  query_range(a, b, qrow0, nq);
  const int q_first = tile * QPT;
  if (q_first >= nq) return;
  const int q_last = min(q_first + QPT, nq) - 1;
  const int t_end = max(0, ctx - nq + q_last + 1);
  const int nparts = (t_end + a.partition - 1) / a.partition;
  if (nparts <= 1) return;  // written directly by the partition kernel
  const int rows = (q_last - q_first + 1) * G;
  // One wave per valid row: lane p weighs partition p (64 at a time), then
  // every lane sums its D/64 dims over the partitions, eight partitions'
  // loads in flight per step (the decode merge's scheme).
  constexpr int DPT = D / 64;
  const int lane = threadIdx.x & 63;
  for (int r = threadIdx.x >> 6; r < rows; r += 4) {
    const size_t row = (size_t(qrow0) + q_first + r / G) * Hq + size_t(kvh) * G + r % G;
    const float* ml = a.part_ml + 2 * row * a.max_parts;
    const float* po = a.part_o + row * a.max_parts * D;
    float M = -FLT_MAX;
    for (int p = lane; p < nparts; p += 64) M = fmaxf(M, ml[2 * p]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    float L = 0.0f;
    float O[DPT];
#pragma unroll
    for (int j = 0; j < DPT; ++j) O[j] = 0.0f;
    for (int p0 = 0; p0 < nparts; p0 += 64) {
      const int p = p0 + lane;
      const float w = p < nparts ? ml[2 * p + 1] * fast_exp2(ml[2 * p] - M) : 0.0f;
      L += w;
      const int cnt = min(64, nparts - p0);
      const float* pg = po + size_t(p0) * D + lane;
      for (int q0 = 0; q0 < cnt; q0 += 8) {
        float v[8][DPT];
#pragma unroll
        for (int k = 0; k < 8; ++k)
#pragma unroll
          for (int j = 0; j < DPT; ++j) v[k][j] = pg[size_t(min(q0 + k, cnt - 1)) * D + j * 64];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float wk = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), min(q0 + k, 63)));
          const float wq = q0 + k < cnt ? wk : 0.0f;
#pragma unroll
          for (int j = 0; j < DPT; ++j) O[j] = fmaf(wq, v[k][j], O[j]);
        }
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
#pragma unroll
    for (int j = 0; j < DPT; ++j)
      store_elem<uint16_t>(a.out, row * D + j * 64 + lane, L > 0.0f ? O[j] / L : 0.0f);
  }
}
// ---------------------------------------------------------------------------
// Host side.


// Measured on MI355X (16 sequences x 40 heads, 512-token chunks, contexts
// to 31K): 8 waves x 2 tiles 774 TFLOP/s, 16 x 1 742, 8 x 1 556, 4 x 4 496.
// Two tiles per wave share each K and V operand read from LDS; 16 tiles per
// workgroup share each K/V chunk read from memory.
#ifndef PKV_PREFILL_WAVES
#define PKV_PREFILL_WAVES 8
#endif
#ifndef PKV_PREFILL_TPW
#define PKV_PREFILL_TPW 2
#endif
constexpr int kPrefillNW = PKV_PREFILL_WAVES;  // waves per workgroup, long chunks
constexpr int kPrefillTPW = PKV_PREFILL_TPW;   // query tiles per wave, long chunks

// Query tiles per prefill workgroup: long chunks use kPrefillNW waves of
// kPrefillTPW tiles each; shorter ones as many single-tile waves (4 or 8) as
// they fill.  Every K/V chunk read from HBM serves all tiles of a workgroup.
int prefill_tiles_per_group(int q_tiles) {
  return q_tiles > 8 ? kPrefillNW * kPrefillTPW : q_tiles > 4 ? 8 : 4;
}

template <int D, int BS>
hipError_t launch_prefill(const AttnArgs& a, int num_seqs, hipStream_t st, int grid_parts) {
  const int tpg = prefill_tiles_per_group(a.q_tiles);
  const int groups = (a.q_tiles + tpg - 1) / tpg;
  const dim3 grid = work_grid(grid_parts, a.num_kv_heads * groups, num_seqs);
  if (a.q_tiles > 8)
    hipLaunchKernelGGL((prefill_lds_kernel<D, BS, kPrefillNW, kPrefillTPW>), grid,
                       dim3(kPrefillNW * 64), 0, st, a);
  else if (tpg == 8)
    hipLaunchKernelGGL((prefill_lds_kernel<D, BS, 8, 1>), grid, dim3(8 * 64), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_lds_kernel<D, BS, 4, 1>), grid, dim3(4 * 64), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.partition >= kSingle) return e;
  hipLaunchKernelGGL((merge_prefill_kernel<D>), dim3(1, a.num_kv_heads * a.q_tiles, num_seqs),
                     dim3(256), 0, st, a);
  return hipGetLastError();
}

// Partition size of a prefill call.  AUTO: the query tiles already give the
// grid enough workgroups in most cases and splitting the tokens only adds
// merge work, so partitions are used only when there are fewer than about
// four workgroups per CU.
int32_t prefill_partition(int32_t num_seqs, int32_t max_queries_per_seq, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t max_context_len,
                          int32_t partition_size) {
  if (partition_size != PKV_PARTITION_AUTO || num_kv_heads <= 0 || num_q_heads <= 0)
    return resolve_partition(max_context_len, partition_size);
  const int G = num_q_heads / num_kv_heads;
  const int qpt = 16 / G > 0 ? 16 / G : 1;
  const int64_t tiles = (int64_t(max_queries_per_seq) + qpt - 1) / qpt;
  const int64_t tpg = prefill_tiles_per_group(int(std::min<int64_t>(tiles, 1 << 20)));
  const int64_t groups = (tiles + tpg - 1) / tpg;
  return int64_t(num_seqs) * num_kv_heads * groups >= 1024
             ? 0
             : resolve_partition(max_context_len, partition_size);
}
}  // namespace
}  // namespace pkv

using pkv::fail;

extern "C" int32_t pkv_prefill_partition_size(int32_t num_seqs, int32_t max_queries_per_seq,
                                              int32_t num_q_heads, int32_t num_kv_heads,
                                              int32_t max_context_len, int32_t partition_size) {
  return pkv::prefill_partition(num_seqs, max_queries_per_seq, num_q_heads, num_kv_heads,
                                max_context_len, partition_size);
}

extern "C" size_t pkv_prefill_workspace_bytes(int32_t total_queries, int32_t num_q_heads,
                                              int32_t head_dim, int32_t max_context_len,
                                              int32_t partition_size) {
  if (total_queries <= 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  return pkv::workspace_for(total_queries, num_q_heads, head_dim, max_context_len,
                            pkv::resolve_partition(max_context_len, partition_size));
}

extern "C" pkv_status pkv_paged_attention_prefill(
    void* out, const void* q, const int32_t* query_start, int32_t total_queries,
    int32_t max_queries_per_seq, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* seq_order, int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    int32_t partition_size, void* workspace, size_t workspace_bytes, pkv_dtype dtype,
    void* stream) {
  if (dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "paged_attention_prefill: bf16 only (matrix cores)");
  if (num_seqs < 0 || num_seqs > 65535 || total_queries < 0 || max_queries_per_seq < 0)
    return fail(PKV_ERR_INVALID_ARG,
                "paged_attention_prefill: num_seqs=%d total_queries=%d max_queries_per_seq=%d",
                num_seqs, total_queries, max_queries_per_seq);
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 ||
      num_q_heads / num_kv_heads > 16)
    return fail(PKV_ERR_UNSUPPORTED,
                "paged_attention_prefill: num_q_heads=%d / num_kv_heads=%d must be a group of 1..16",
                num_q_heads, num_kv_heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "paged_attention_prefill: head_dim=%d (64 or 128)", head_dim);
  if (block_size != 16 && block_size != 32)
    return fail(PKV_ERR_UNSUPPORTED, "paged_attention_prefill: block_size=%d (16 or 32)",
                block_size);
  if (num_blocks <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0 ||
      max_context_len > (1 << 29))
    return fail(PKV_ERR_INVALID_ARG, "paged_attention_prefill: bad pool or context sizes");
  if (partition_size < PKV_PARTITION_AUTO ||
      (partition_size > 0 && partition_size % block_size != 0))
    return fail(PKV_ERR_INVALID_ARG,
                "paged_attention_prefill: partition_size=%d must be 0, -1 or a multiple of %d",
                partition_size, block_size);
  if (num_seqs == 0 || total_queries == 0 || max_queries_per_seq == 0) return pkv::ok();
  if (!out || !q || !query_start || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PKV_ERR_INVALID_ARG, "paged_attention_prefill: NULL pointer argument");
  const int G = num_q_heads / num_kv_heads;
  const int qpt = 16 / G > 0 ? 16 / G : 1;
  const int64_t tiles = (int64_t(max_queries_per_seq) + qpt - 1) / qpt;
  if (tiles * num_kv_heads > 65535)
    return fail(PKV_ERR_INVALID_ARG,
                "paged_attention_prefill: %lld query tiles x %d kv heads exceed the grid limit",
                (long long)tiles, num_kv_heads);
  const int32_t partition = pkv::prefill_partition(num_seqs, max_queries_per_seq, num_q_heads,
                                                   num_kv_heads, max_context_len, partition_size);
  const int32_t cap = int32_t(std::min<int64_t>(max_context_len,
                                                int64_t(max_blocks_per_seq) * block_size));
  pkv::AttnArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.tables = block_tables;
  a.ctx_lens = context_lens;
  a.order = seq_order;
  a.query_start = query_start;
  a.q_tiles = int32_t(tiles);
  {
    const int tpg = pkv::prefill_tiles_per_group(int(tiles));
    a.q_groups = int32_t((tiles + tpg - 1) / tpg);
  }
  a.total_queries = total_queries;
  a.num_seqs = num_seqs;
  a.max_blocks = max_blocks_per_seq;
  a.ctx_cap = cap;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.num_blocks = num_blocks;
  a.scale_log2 = scale * pkv::kLog2e;
  int grid_parts = 1;
  if (partition > 0) {
    const size_t need =
        pkv::workspace_for(total_queries, num_q_heads, head_dim, max_context_len, partition);
    if (need > 0 && (!workspace || workspace_bytes < need))
      return fail(PKV_ERR_WORKSPACE,
                  "paged_attention_prefill: workspace of %zu bytes needed, %zu given", need,
                  workspace ? workspace_bytes : size_t(0));
    a.partition = partition;
    a.max_parts = int32_t((int64_t(max_context_len) + partition - 1) / partition);
    if (a.max_parts < 1) a.max_parts = 1;
    float* ws = static_cast<float*>(workspace);
    a.part_o = ws;
    a.part_ml = ws + size_t(total_queries) * num_q_heads * a.max_parts * head_dim;
    grid_parts = int((int64_t(cap) + partition - 1) / partition);
    if (grid_parts < 1) grid_parts = 1;
  } else {
    a.partition = pkv::kSingle;
    a.max_parts = 1;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (head_dim == 64)
    e = block_size == 16 ? pkv::launch_prefill<64, 16>(a, num_seqs, st, grid_parts)
                         : pkv::launch_prefill<64, 32>(a, num_seqs, st, grid_parts);
  else
    e = block_size == 16 ? pkv::launch_prefill<128, 16>(a, num_seqs, st, grid_parts)
                         : pkv::launch_prefill<128, 32>(a, num_seqs, st, grid_parts);
  if (e != hipSuccess)
    return fail(PKV_ERR_HIP, "paged_attention_prefill: launch failed: %s", hipGetErrorString(e));
  return pkv::ok();
}

