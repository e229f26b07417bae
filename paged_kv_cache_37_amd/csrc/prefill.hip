// Multi-token (prefill / chunked-prefill) paged attention on the CDNA4
// matrix cores.
//
// "Optimizing KV Cache Memory Management in vLLM with PagedAttention and
// Dynamic Block Allocation", The Block Manager and Dynamic Allocation
// Lifecycle (The Prefill Phase: a prompt's K/V are computed in one parallel
// step and written into its blocks) and Production Tuning, Failure Mode 2
// (chunked prefill: a long prompt is processed in chunks).  Sequence s's
// chunk holds its last q_len positions; the query at position p attends the
// keys at positions lo(p) .. p (lo(p) = 0, or p + 1 - W under a window W),
// walking the sequence's block table like decode does.
//
// Unlike decode this is a dense contraction: q_len * G query rows of one KV
// head meet the same keys.  A workgroup takes 128 query rows of one
// (sequence, KV head) (rows r = token * G + head); its four waves hold 32
// rows each as two 16-column blocks of the MFMA B operand.  Keys go 64 at a
// time (four 16-token tiles): the workgroup copies their K and V from the
// pool into LDS once (double-buffered, the next step's loads in flight
// during this step's compute) and every wave reads its operands there,
// 32 keys per MFMA round.
//   S^T = K Q^T   v_mfma_f32_16x16x32_bf16, per 16-key tile, A = K rows
//   O  += P V     v_mfma_f32_16x16x32_bf16, A = P (the two tiles' S^T
//                 outputs of a lane are its 8 reduction values), B = V:
//                 LDS holds a round's V as [quad][dim'][tile][4 keys], so
//                 one 16-byte read gives a dim's four keys of both tiles,
//                 the 8 keys of B in the order of A; within each 32-dim
//                 group dim' puts the even dims first, then the odd ones,
//                 so the 16 lanes reading dims 2 col (or 2 col + 1) read
//                 16 consecutive 16-byte rows (no LDS bank conflicts)
// with the base-2 online softmax of the decode kernels: scores c (K . q)
// with c = |scale| log2(e) > 0 (a negative scale flips the queries' signs),
// the running max raised only past a slack, the row sums an MFMA of P with
// a ones operand.  An FP8 pool's codes are widened to bf16 when a step is
// staged into LDS, so the operand reads are the bf16 path's.  P is rounded
// to bf16 once (the result stays within the bf16 tolerance; decode's
// two-term P keeps split-K invariance, which prefill does not need).
//
// The key walk is three loops over steps: leading steps that need masks
// (window start, first slots, bad tiles), the unmasked interior (one basic
// block apart from the rare rescale, so softmax and MFMAs interleave), and
// trailing masked steps (the causal diagonal, the last block).
//
// The same kernel (PREFIX) runs the shared-prefix pass of cascade decode:
// every sequence's decode query as a row, a chunk of the shared prefix as
// the keys, two-term P like the decode kernels, a partial result out.
#include "mfma_tile.h"

namespace kvp {
namespace {

constexpr int kPfRows = 128;         // query rows per workgroup (32 per wave)
constexpr int kLptMaxPairs = 256;    // (sequence, query tile) pairs ranked by work in every workgroup
constexpr int kTiles = 4;            // 16-token tiles per step
constexpr int kStep = 16 * kTiles;   // keys per step (loaded together; computed 32 at a time)

template <bool FP8>
using Elt = std::conditional_t<FP8, uint8_t, uint16_t>;


// Wave-wide min / max, returned as a scalar (uniform) value.
__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return __builtin_amdgcn_readfirstlane(v);
}
__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return __builtin_amdgcn_readfirstlane(v);
}

// PREFIX: the shared-prefix pass of cascade decode instead: the rows are
// the decode queries of all sequences, the keys one chunk of the shared
// prefix blocks (no causal mask), and a partial result goes out.
template <int D, bool FP8, int BS, bool PREFIX>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(const PrefillParams P) {
  using E = Elt<FP8>;
  constexpr int CH = 16 / sizeof(E);           // elements per 16-byte copy
  constexpr int KROW = D + 8;                  // LDS K row (bf16): 16 bytes of padding, so 16 rows hit distinct banks
  constexpr int TCH = 16 * D / CH;             // 16-byte chunks of one tile's K (and of its V)
  static_assert(kTiles % 2 == 0, "steps of whole 32-key rounds");
  static_assert(TCH <= kThreads, "one chunk per thread and tile");
  // LDS holds bf16 whatever the pool's type: FP8 codes are widened once,
  // when a step is staged, not by each of the four waves that read them
  __shared__ __align__(16) uint16_t k_s[2][kStep * KROW];
  __shared__ __align__(16) uint16_t v_s[2][kStep * D];  // per 32-key round: [4 quads][D][2 tiles][4 keys]
  __shared__ int lpt_cost[PREFIX ? 1 : kLptMaxPairs];
  __shared__ int lpt_pick;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = P.group;
  const int B = kBlock << BS;
  const int q4 = lane >> 4, col = lane & 15;
  // Per workgroup: the table row and span of the keys, the steps, the KV
  // head; per lane: this column's query in each of the wave's two blocks
  // and the span slots it attends.
  const int32_t* row;
  int kvh, t0, so, send, ntiles, k_lo, k_hi;
  uint4_v qop[2][D / 32];
  int lo_c[2], hi_c[2];
  int hrow[2];  // query row of the column, -1 past the rows
  int s = 0, c0 = 0, kc = 0;
  if constexpr (PREFIX) {
    // rows r = s * G + g of one KV head, 128 per workgroup, against key
    // chunk kc; every workgroup of KV head h on XCD h mod 8 (the head's
    // prefix fetched into one L2)
    const int rows = P.num_seqs * G;
    const int per_head = P.qtiles * P.prefix_pieces;
    int rest;
    if (P.num_kv_heads % 8 == 0) {
      const int x = blockIdx.x & 7, k = blockIdx.x >> 3, nx = P.num_kv_heads >> 3;
      rest = k / nx;
      kvh = x + 8 * (k - rest * nx);
    } else {
      kvh = blockIdx.x / per_head;
      rest = blockIdx.x - kvh * per_head;
    }
    kc = rest / P.qtiles;
    const int qt = rest - kc * P.qtiles;
    const int r_wg = qt * kPfRows;
    if (r_wg >= rows) return;  // the whole workgroup: before any barrier
    // every prefix block is full and attended by every row; the chunk's
    // tiles [j0, ntiles) start on a step
    row = P.block_tables;
    t0 = 0;  // the shared prefix starts at position 0
    so = 0;
    const int j0 = kc * P.prefix_chunk;
    ntiles = min(j0 + P.prefix_chunk, P.prefix_blocks << BS);
    send = ntiles * kBlock;
    k_lo = j0 / kTiles;
    k_hi = (send - 1) / kStep;
    for (int nb = 0; nb < 2; ++nb) {
      const int r = r_wg + wave * 32 + nb * 16 + col;
      const bool ok = r < rows;
      const int sq = r / G, g = r - sq * G;
      hrow[nb] = ok ? r : -1;
      lo_c[nb] = ok ? 0 : INT32_MAX;
      hi_c[nb] = ok ? send - 1 : -1;
      const uint16_t* qp = (const uint16_t*)P.q + ((size_t)sq * P.num_q_heads + kvh * G + g) * D + 8 * q4;
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) qop[nb][kk] = ok ? *(const uint4_v*)(qp + 32 * kk) : uint4_v{0, 0, 0, 0};
      if (P.scale_log2 < 0.f) {  // c |scale| (-q) = scale q
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) qop[nb][kk] ^= 0x80008000u;
      }
    }
  } else {
    const int SK = P.num_seqs * P.num_kv_heads;  // (sequence, KV head) groups
    // Workgroups start in index order as slots free up, so the heaviest go
    // first: the (sequence, query tile) pairs are ranked by the keys their
    // rows attend (the prior context dominates), workgroup b takes the pair
    // of rank b / Hkv and KV head b mod Hkv.  Workgroup b runs on XCD b mod
    // 8, so with 8 KV heads XCD x holds head x of every sequence: all query
    // tiles of a (sequence, KV head) share one L2 (its K/V fetched once).
    // Larger batches take tiles by query-tile index, latest first.
    int qt, grp;
    const int npairs = P.num_seqs * P.qtiles;
    auto pair_cost = [&](int i) {  // keys the workgroup of pair i attends; -1 if it has no rows
      const int ps = i / P.qtiles, pq = i - ps * P.qtiles;
      const int pc0 = P.cu_q_lens[ps], pql = P.cu_q_lens[ps + 1] - pc0, pctx = P.seq_lens[ps];
      const int prows = max(0, min(min(pql, P.max_q_len), P.total_q - pc0)) * G;
      if (pq * kPfRows >= prows || pc0 < 0) return -1;
      const int pp0 = pctx - pql, plast = min(pq * kPfRows + kPfRows, prows) - 1;
      const int pa = max(pp0 + pq * kPfRows / G, 0), pb = pp0 + plast / G;
      if (pb < 0) return 0;
      return pb - (P.window > 0 ? max(0, pa + 1 - P.window) : 0) + 1;
    };
    if (npairs <= kLptMaxPairs) {
      for (int i = threadIdx.x; i < npairs; i += kThreads) lpt_cost[i] = pair_cost(i);
      __syncthreads();
      const int target = (int)(blockIdx.x / P.num_kv_heads);
      for (int i = threadIdx.x; i < npairs; i += kThreads) {
        const int ci = lpt_cost[i];
        int rank = 0;
        for (int j = 0; j < npairs; ++j) {
          const int cj = lpt_cost[j];
          rank += (cj > ci) | ((cj == ci) & (j < i));
        }
        if (rank == target) lpt_pick = i;
      }
      __syncthreads();
      const int pick = lpt_pick;
      kvh = (int)(blockIdx.x % P.num_kv_heads);
      s = pick / P.qtiles;
      qt = pick - s * P.qtiles;
    } else {
      if (SK % 8 == 0) {
        const int x = blockIdx.x & 7, k = blockIdx.x >> 3, nx = SK >> 3;
        qt = P.qtiles - 1 - k / nx;
        grp = x + 8 * (k - (k / nx) * nx);
      } else {
        qt = P.qtiles - 1 - (int)(blockIdx.x / SK);
        grp = blockIdx.x - (P.qtiles - 1 - qt) * SK;
      }
      s = grp / P.num_kv_heads;
      kvh = grp - s * P.num_kv_heads;
    }
    c0 = P.cu_q_lens[s];
    const int q_len = P.cu_q_lens[s + 1] - c0;
    const int ctx = P.seq_lens[s];
    // rows computed: the chunk's, up to max_q_len tokens and inside q / out
    const int rows = max(0, min(min(q_len, P.max_q_len), P.total_q - c0)) * G;
    const int r_wg = qt * kPfRows;
    if (r_wg >= rows || c0 < 0) return;  // the whole workgroup (uniform), before the steps' barriers

    // Positions: token i at p = ctx - q_len + i.  The table row starts at the
    // block holding `first`, the first key any query of the chunk attends;
    // span slot u is position first - so + u.
    const int p0 = ctx - q_len;
    const int first = P.window > 0 ? max(0, p0 + 1 - P.window) : 0;
    const int off = first & (B - 1);
    t0 = off >> 4;
    so = off & (kBlock - 1);
    const int base = first - so;                   // position of span slot 0
    // span slots holding keys: [so, send); a row longer than its table
    // attends what the table holds
    send = min(so + max(ctx - first, 0), P.max_blocks * B - kBlock * t0);
    ntiles = (send + kBlock - 1) / kBlock;
    row = P.block_tables + (size_t)s * P.max_blocks;
    auto lo_of = [&](int p) { return P.window > 0 ? max(0, p + 1 - P.window) : 0; };

    // The workgroup's key range (rows are in position order).
    const int r_last = min(r_wg + kPfRows, rows) - 1;
    const int pa = max(p0 + r_wg / G, 0), pb = p0 + r_last / G;
    const int u_lo = lo_of(pa) - base, u_hi = pb - base;  // span slots some row attends
    k_lo = max(u_lo, 0) / kStep;
    k_hi = pb >= 0 ? u_hi / kStep : k_lo - 1;  // no steps when no row has a position

    for (int nb = 0; nb < 2; ++nb) {
      const int r = r_wg + wave * 32 + nb * 16 + col;
      const int i = r / G, g = r - (r / G) * G;
      const int p = p0 + i;
      const bool ok = r < rows && p >= 0;  // a row without a position (chunk longer than its context) stores zeros
      hrow[nb] = r < rows ? r : -1;
      lo_c[nb] = ok ? lo_of(p) - base : INT32_MAX;
      hi_c[nb] = ok ? p - base : -1;
      const uint16_t* qp = (const uint16_t*)P.q + ((size_t)(c0 + i) * P.num_q_heads + kvh * G + g) * D + 8 * q4;
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) qop[nb][kk] = ok ? *(const uint4_v*)(qp + 32 * kk) : uint4_v{0, 0, 0, 0};
      if (P.scale_log2 < 0.f) {  // c |scale| (-q) = scale q
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) qop[nb][kk] ^= 0x80008000u;
      }
    }
  }
  // the wave's own key range (its columns' union), for skipping steps
  const int w_lo = wave_min(min(lo_c[0], lo_c[1]));
  const int w_hi = wave_max(max(hi_c[0], hi_c[1]));
  // keys every column of the wave attends: a round inside [w_in_lo, w_in_hi]
  // needs no per-column mask (a wave with a column that attends nothing
  // always masks)
  const bool all_cols = wave_min((lo_c[0] != INT32_MAX) & (lo_c[1] != INT32_MAX)) != 0;
  const int w_in_lo = all_cols ? wave_max(max(lo_c[0], lo_c[1])) : INT32_MAX;
  const int w_in_hi = all_cols ? wave_min(min(hi_c[0], hi_c[1])) : -1;

  // Block ids of the tiles 64 at a time (lane i: tile jb + i), the next 64 prefetched.
  auto entry = [&](int J) { return J < ntiles ? row[(t0 + J) >> BS] : 0; };
  int jb = kTiles * k_lo;
  int ids_a = entry(jb + lane), ids_b = entry(jb + 64 + lane);

  const size_t tile = (size_t)B * D;  // one head's K (or V) tile of a block
  const size_t blk_stride = 2 * (size_t)P.num_kv_heads * tile;
  const E* pool = (const E*)P.pool_layer + (size_t)kvh * tile;
  const size_t v_rel = (size_t)P.num_kv_heads * tile;

  // Global -> registers for the step's two tiles (bad or absent tiles read
  // block 0; their keys are masked), registers -> LDS.
  uint4_v kreg[kTiles], vreg[kTiles];  // thread tid's chunk of each tile of the step
  unsigned bad = 0;  // bit t: tile t of the fetched step holds no keys (past the span, or no block)
  auto fetch = [&](int k) {
    const int J0 = kTiles * k;
    if (J0 - jb >= 64) {  // rotate the id window (uniform: every wave walks the same steps)
      ids_a = ids_b;
      jb += 64;
      ids_b = entry(jb + 64 + lane);
    }
    bad = 0;
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      const int J = J0 + t;
      int id = __builtin_amdgcn_readlane(J - jb < 64 ? ids_a : ids_b, (J - jb) & 63);
      const bool b = J >= ntiles || (unsigned)id >= (unsigned)P.num_blocks;
      bad |= (b ? 1u : 0u) << t;
      if (b) id = 0;
      // tile t's K rows and V quads: a uniform base, this thread's chunk
      const E* src = pool + (size_t)id * blk_stride + (size_t)((t0 + J) & ((1 << BS) - 1)) * kBlock * D;
      if (TCH % kThreads == 0 || threadIdx.x < TCH) {
        kreg[t] = *(const uint4_v*)(src + threadIdx.x * CH);          // key tid / (D / CH), chunk tid % (D / CH)
        vreg[t] = *(const uint4_v*)(src + v_rel + threadIdx.x * CH);  // elements 16 tid .. of [4][D][4]
      }
    }
  };
  auto stash = [&](int buf) {
    if (TCH % kThreads != 0 && threadIdx.x >= TCH) return;
    const int key = threadIdx.x / (D / CH), cc = threadIdx.x - key * (D / CH);
    // this thread's V chunk: CH / 4 dims x 4 keys of quad q
    const int e0 = threadIdx.x * CH, q = e0 / (4 * D), d = (e0 - q * 4 * D) >> 2;
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      uint16_t* dk = &k_s[buf][(16 * t + key) * KROW + cc * CH];
      if constexpr (FP8) {
        *(uint4_v*)dk = fp8_widen8(uint2_v{kreg[t].x, kreg[t].y});
        *(uint4_v*)(dk + 8) = fp8_widen8(uint2_v{kreg[t].z, kreg[t].w});
      } else {
        *(uint4_v*)dk = kreg[t];
      }
    }
    // per dim, its 4 keys of tile 2h beside those of tile 2h + 1 (this thread
    // holds the same quad and dims of both); even dim d of its 32-dim group
    // at row (d mod 32) / 2 of the group, odd dim d + 1 at row 16 + that
    const int d_even = (d & ~31) + ((d & 31) >> 1);
#pragma unroll
    for (int h = 0; h < kTiles / 2; ++h) {
      uint16_t* dst_e = &v_s[buf][h * 32 * D + (q * D + d_even) * 8];
      uint16_t* dst_o = dst_e + 16 * 8;
      const uint4_v a = vreg[2 * h], b = vreg[2 * h + 1];
      if constexpr (FP8) {
        // dims d .. d + 3 (four codes each): d and d + 2 in adjacent even
        // rows, d + 1 and d + 3 in odd rows, widened to bf16
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint2_v wa = fp8_widen4(a[j]), wb = fp8_widen4(b[j]);
          *(uint4_v*)((j & 1 ? dst_o : dst_e) + 8 * (j >> 1)) = uint4_v{wa.x, wa.y, wb.x, wb.y};
        }
      } else {
        *(uint4_v*)dst_e = uint4_v{a.x, a.y, b.x, b.y};
        *(uint4_v*)dst_o = uint4_v{a.z, a.w, b.z, b.w};
      }
    }
  };

  // Scores in base 2 are c * (K . q) with c > 0: a negative scale was folded
  // into the queries' signs (exact in bf16); scale 0 becomes a vanishing c,
  // which gives the same uniform weights.
  const float c = fmaxf(fabsf(P.scale_log2), 1e-30f);
  float m_run[2] = {-INFINITY, -INFINITY};
  float4_v acc[2][D / 16];
  float4_v acc_l[2];  // [nb][r]: weight sum of output row 4 q4 + r (an MFMA of P with a ones operand)
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    acc_l[nb] = float4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < D / 16; ++n) acc[nb][n] = float4_v{0.f, 0.f, 0.f, 0.f};
  }
  const bf16x8_v ones = __builtin_bit_cast(bf16x8_v, uint4_v{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});

  // One round of 32 keys (tiles 2h, 2h+1 of the step in LDS buffer buf).
  // EDGE rounds hold keys outside the span, in a bad tile, or outside some
  // column's range: they mask; the others run without a branch except the
  // (rare) rescale, so the compiler can interleave softmax and MFMAs.
  auto round = [&](auto edge, int u0, int buf, int h, bool vedge, bool bad0, bool bad1) {
    constexpr bool EDGE = decltype(edge)::value;
    const uint16_t* ks = k_s[buf] + 32 * h * KROW;
    const uint16_t* vs = v_s[buf] + 32 * h * D;
    // S^T per tile and column block, issued at a raised wave priority so
    // that of the two waves on a SIMD the one in its product phase issues
    // first and the other fills the gaps with its softmax
    float4_v sc[2][2];
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      uint4_v kf[D / 32];
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) kf[kk] = *(const uint4_v*)(ks + (t * 16 + col) * KROW + 32 * kk + 8 * q4);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float4_v a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, kf[kk]),
                                                      __builtin_bit_cast(bf16x8_v, qop[nb][kk]), a, 0, 0, 0);
        sc[t][nb] = a;
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // keys of the step outside the span (or in a bad tile) hold no data:
    // zero their V and mask their scores for every column
    unsigned vm[2][2] = {{~0u, ~0u}, {~0u, ~0u}};  // [tile][half]: keys 4q4 + {0,1} and {2,3} hold data
    if constexpr (EDGE) {
      if (vedge) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int u = u0 + t * 16 + 4 * q4 + 2 * hh;
            const bool tb = t ? bad1 : bad0;
            const bool a = !tb & (u >= so) & (u < send), b = !tb & (u + 1 >= so) & (u + 1 < send);
            vm[t][hh] = (a ? 0xffffu : 0u) | (b ? 0xffff0000u : 0u);
          }
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int u = u0 + t * 16 + 4 * q4 + r;
            const bool keep = ((vm[t][r >> 1] >> (16 * (r & 1))) & 1u) & (u >= lo_c[nb]) & (u <= hi_c[nb]);
            sc[t][nb][r] = keep ? sc[t][nb][r] : -INFINITY;
          }
    }
    // running max: raised (for both column blocks) only when a score passes
    // it by more than the slack; max(c s) = c max(s) as c > 0
    float mc[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float lmax = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) lmax = fmaxf(lmax, sc[t][nb][r]);
      mc[nb] = lmax * c;
    }
    if (__any((mc[0] > m_run[0] + kRescaleSlack) | (mc[1] > m_run[1] + kRescaleSlack))) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const float m_new = fmaxf(m_run[nb], rows_max(mc[nb]));
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run[nb] - m_use);
        m_run[nb] = m_new;
        // output rows here are columns 4 q4 + r; whole-vector products keep
        // each accumulator in its registers
        const float4_v ar = {__shfl(alpha, 4 * q4), __shfl(alpha, 4 * q4 + 1), __shfl(alpha, 4 * q4 + 2),
                             __shfl(alpha, 4 * q4 + 3)};
        acc_l[nb] *= ar;
#pragma unroll
        for (int n = 0; n < D / 16; ++n) acc[nb][n] *= ar;
      }
    }
    // V operands of the round (B rows 8 q4 .. +7 are keys 4 q4 .. +3 of
    // tile 0, then of tile 1)
    uint4_v vb[D / 32][2];
#pragma unroll
    for (int m = 0; m < D / 32; ++m) {
      vb[m][0] = *(const uint4_v*)(vs + (q4 * D + 32 * m + col) * 8);       // dim 32 m + 2 col
      vb[m][1] = *(const uint4_v*)(vs + (q4 * D + 32 * m + 16 + col) * 8);  // dim 32 m + 2 col + 1
      if constexpr (EDGE) {
        if (vedge) {
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            vb[m][i].x &= vm[0][0]; vb[m][i].y &= vm[0][1]; vb[m][i].z &= vm[1][0]; vb[m][i].w &= vm[1][1];
          }
        }
      }
    }
    // per column block: P = 2^(c s - m) as bf16 (and, in the shared-prefix
    // pass, the bf16 rest P - pa), then O += P V and the row sums; block 1's
    // softmax can run while block 0's products are in the matrix core
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float neg_m = m_run[nb] == -INFINITY ? 0.f : -m_run[nb];
      float pr[2][4];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) pr[t][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][nb][r], c, neg_m));
      const uint4_v pa = uint4_v{pack_bf16x2(pr[0][0], pr[0][1]), pack_bf16x2(pr[0][2], pr[0][3]),
                                 pack_bf16x2(pr[1][0], pr[1][1]), pack_bf16x2(pr[1][2], pr[1][3])};
      uint4_v pl;
      if constexpr (PREFIX) {
        // the decode kernels carry P as two bf16 terms; the cascade's prefix
        // pieces keep their precision, so cascade and plain decode agree
        pl = uint4_v{pack_bf16x2(pr[0][0] - bf16_lo(pa.x), pr[0][1] - bf16_hi(pa.x)),
                     pack_bf16x2(pr[0][2] - bf16_lo(pa.y), pr[0][3] - bf16_hi(pa.y)),
                     pack_bf16x2(pr[1][0] - bf16_lo(pa.z), pr[1][1] - bf16_hi(pa.z)),
                     pack_bf16x2(pr[1][2] - bf16_lo(pa.w), pr[1][3] - bf16_hi(pa.w))};
      }
#pragma unroll
      for (int m = 0; m < D / 32; ++m)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          acc[nb][2 * m + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_v, pa), __builtin_bit_cast(bf16x8_v, vb[m][i]), acc[nb][2 * m + i], 0, 0, 0);
          if constexpr (PREFIX)
            acc[nb][2 * m + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_v, pl), __builtin_bit_cast(bf16x8_v, vb[m][i]), acc[nb][2 * m + i], 0, 0, 0);
        }
      // row sums of the same rounded weights the outputs use
      acc_l[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, pa), ones, acc_l[nb], 0, 0, 0);
      if constexpr (PREFIX)
        acc_l[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, pl), ones, acc_l[nb], 0, 0, 0);
    }
  };

  // Steps k .. k_end in one form (EDGE: every round masks what it must and
  // skips what no column of the wave attends), each with the next step's
  // loads in flight; the unmasked form stops at a step holding a bad tile.
  // Every wave runs every step once whatever its split into these loops,
  // so the workgroup's barriers match.
  unsigned bad_c = 0;
  auto steps = [&](auto edge, int k, int k_end) {
    constexpr bool EDGE = decltype(edge)::value;
    for (; k <= k_end; ++k) {
      if constexpr (!EDGE) {
        if (bad_c) break;
      }
      const int buf = (k - k_lo) & 1;
      const bool more = k < k_hi;
      if (more) {  // the next step's loads go out at a raised priority, ahead of the other waves' softmax
        __builtin_amdgcn_s_setprio(1);
        fetch(k + 1);
        __builtin_amdgcn_s_setprio(0);
      }
#pragma unroll
      for (int h = 0; h < kTiles / 2; ++h) {
        const int u0 = k * kStep + 32 * h;  // span slot of the round's first key
        if constexpr (EDGE) {
          if (u0 + 31 < w_lo || u0 > w_hi) continue;  // no column of this wave attends these keys
          const bool bad0 = (bad_c >> (2 * h)) & 1u, bad1 = (bad_c >> (2 * h + 1)) & 1u;
          round(edge, u0, buf, h, bad0 || bad1 || u0 < so || u0 + 32 > send, bad0, bad1);
        } else {
          round(edge, u0, buf, h, false, false, false);
        }
      }
      if (more) stash(buf ^ 1);
      __syncthreads();
      bad_c = bad;
    }
    return k;
  };

  if (k_hi >= k_lo) {
    fetch(k_lo);
    bad_c = bad;
    stash(0);
    __syncthreads();
    // interior steps: every key in the span and every column of the wave
    // attending all of them (w_in_lo = INT32_MAX when a column attends none)
    const int in_lo = max(so, w_in_lo), in_hi = min(send - 1, w_in_hi);
    int k_a = in_lo == INT32_MAX ? k_hi + 1 : max(k_lo, (in_lo + kStep - 1) / kStep);
    int k_b = in_hi < 0 ? k_lo - 1 : min(k_hi, (in_hi + 1) / kStep - 1);
    if (k_a > k_b) {
      k_a = k_hi + 1;
      k_b = k_hi;
    }
    int k = steps(std::true_type{}, k_lo, k_a - 1);
    k = steps(std::false_type{}, k, k_b);
    steps(std::true_type{}, k, k_hi);
  }

  // output row 4 q4 + r of block nb is column 4 q4 + r
  if constexpr (PREFIX) {
    // (max, sum, unnormalised output) of query (s, h) over chunk kc, for
    // the merge with the other chunks and the tails
    const size_t piece = (size_t)kc * P.num_seqs * P.num_q_heads;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      // the sum of column col lives in register col % 4 of the lanes with q4 = col / 4
      const int j = lane & 3;
      const float lsel = j == 0 ? acc_l[nb][0] : j == 1 ? acc_l[nb][1] : j == 2 ? acc_l[nb][2] : acc_l[nb][3];
      const float l_tot = __shfl(lsel, 16 * (col >> 2) + (col & 3));
      if (lane < 16 && hrow[nb] >= 0) {
        const int sq = hrow[nb] / G, g = hrow[nb] - sq * G;
        const size_t qh = piece + (size_t)sq * P.num_q_heads + kvh * G + g;
        *(float2*)(P.pre_ml + qh * 2) = make_float2(m_run[nb], l_tot);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int hr = __shfl(hrow[nb], 4 * q4 + r);
        if (hr >= 0) {
          const int sq = hr / G, g = hr - sq * G;
          float2* o = (float2*)(P.pre_o + (piece + (size_t)sq * P.num_q_heads + kvh * G + g) * D);
#pragma unroll
          for (int m = 0; m < D / 32; ++m) o[16 * m + col] = make_float2(acc[nb][2 * m][r], acc[nb][2 * m + 1][r]);
        }
      }
    }
    return;
  }
  // normalise and store
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int g = 4 * q4 + r;
      const float lg = acc_l[nb][r];
      const int hr = __shfl(hrow[nb], g);
      const float inv = lg > 0.f ? P.v_scale / lg : 0.f;
      if (hr >= 0) {
        const int i = hr / G, h = hr - (hr / G) * G;
        unsigned* o = (unsigned*)((uint16_t*)P.out + ((size_t)(c0 + i) * P.num_q_heads + kvh * G + h) * D);
#pragma unroll
        for (int m = 0; m < D / 32; ++m)
          o[16 * m + col] = pack_bf16x2(acc[nb][2 * m][r] * inv, acc[nb][2 * m + 1][r] * inv);
      }
    }
  }
}

template <int D, bool FP8, bool PREFIX>
hipError_t launch_pf(const PrefillParams& p, unsigned grid, hipStream_t stream) {
  if (p.bshift)
    hipLaunchKernelGGL((prefill_kernel<D, FP8, 1, PREFIX>), dim3(grid), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((prefill_kernel<D, FP8, 0, PREFIX>), dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <bool PREFIX>
hipError_t launch_any(const PrefillParams& p, long long grid, int head_dim, bool fp8, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const unsigned g = (unsigned)grid;
  if (head_dim == 128) return fp8 ? launch_pf<128, true, PREFIX>(p, g, stream) : launch_pf<128, false, PREFIX>(p, g, stream);
  if (head_dim == 64) return fp8 ? launch_pf<64, true, PREFIX>(p, g, stream) : launch_pf<64, false, PREFIX>(p, g, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int head_dim, bool fp8, hipStream_t stream) {
  return launch_any<false>(p, (long long)p.num_seqs * p.num_kv_heads * p.qtiles, head_dim, fp8, stream);
}

hipError_t launch_prefix_pass(const PrefillParams& p, int head_dim, bool fp8, hipStream_t stream) {
  return launch_any<true>(p, (long long)p.num_kv_heads * p.qtiles * p.prefix_pieces, head_dim, fp8, stream);
}

}  // namespace kvp
