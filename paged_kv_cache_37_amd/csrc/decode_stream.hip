// Paged decode attention on the CDNA4 matrix cores (bf16 or FP8 pools), streaming
// form: a persistent grid of exactly the resident waves splits the batch's
// work evenly, whatever the mix of sequence lengths.
//
// The work is the list of tiles (head group, sequence, tile): row (hg, s)
// has one tile per 16 tokens of sequence s's blocks (one per block-table
// entry, two with 32-token blocks), each tile being 16 tokens of K/V for
// that KV head ("PagedAttention: Virtual
// Memory for LLMs" in "Optimizing KV Cache Memory Management in vLLM with
// PagedAttention and Dynamic Block Allocation": the kernel walks the
// sequence's block table to find each block).  Wave w streams the
// contiguous tile range [w T / W, (w+1) T / W).  Its loads run DEPTH tiles
// ahead of its compute across row boundaries: every in-flight tile carries
// its row context, and the next row's table entries and queries are fetched
// while the current row streams.  A row that lies wholly inside a wave's
// range is normalised and stored by that wave; the (at most two) rows cut by
// a range boundary leave a partial result (running max, sum, unnormalised
// output) that a second kernel merges.
//
// Ranges are contiguous per XCD (workgroup i runs on XCD i mod 8): the
// tiles of one head group, which share physical blocks across sequences
// with a common prefix, stay in one XCD's L2.  Tiles are read with
// non-temporal loads (NT) when no block is listed by two rows, each line
// then being read once, and with cached loads when rows share blocks.
#include "mfma_tile.h"

namespace kvp {
namespace {

#ifndef KVP_STREAM_WAVES_PER_EU
#define KVP_STREAM_WAVES_PER_EU 2
#endif

// Index of this workgroup when the grid is ordered XCD by XCD.
__device__ __forceinline__ int xcd_major_index(int wg, int nwg) {
  const int x = wg & 7, k = wg >> 3;
  return x * (nwg >> 3) + min(x, nwg & 7) + k;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  return v;
}

// floor(num / den) for 0 <= num < 2^53, 0 < den: the double quotient of two
// exactly represented integers is either that integer or at least 1/den
// away from it, far more than its rounding error, so the floor is exact
// (and avoids the GPU's software 64-bit integer division).
__device__ __forceinline__ long long floor_div(long long num, long long den) {
  return (long long)__builtin_floor((double)num / (double)den);
}

// Pieces of a cut row, merged in wave order kMergeChunk at a time: each
// round takes the round's largest max, rescales what was merged so far once,
// then adds the round's pieces (max m, sum l, unnormalised o; an absent
// piece is m = -inf, l = 0, o = 0).  The merge kernel folds the shared
// prefix's chunk pieces and a row's wave pieces with it.
constexpr int kMergeChunk = 8;

template <int PER, int CH>
__device__ __forceinline__ void merge_round(float& M, float& den, float (&num)[PER], const float (&m)[CH],
                                            const float (&l)[CH], const float (&v)[CH][PER]) {
  float Mc = M;
#pragma unroll
  for (int u = 0; u < CH; ++u) Mc = fmaxf(Mc, m[u]);
  if (Mc == -INFINITY) return;
  const float ao = __builtin_amdgcn_exp2f(M - Mc);
  den *= ao;
#pragma unroll
  for (int e = 0; e < PER; ++e) num[e] *= ao;
#pragma unroll
  for (int u = 0; u < CH; ++u) {
    const float f = __builtin_amdgcn_exp2f(m[u] - Mc);
    den += f * l[u];
#pragma unroll
    for (int e = 0; e < PER; ++e) num[e] += f * v[u][e];
  }
  M = Mc;
}

// The pieces of a cut row [a, a + nb) of the work list (T tiles over W
// waves), in wave order.  With T >= W every range holds a tile, so they are
// waves w_first .. w_last: the first holds the row as its last row (slot 1)
// unless its range starts at the row, every later one as its first (slot 0).
// With T < W a range holds at most one tile, and each of the row's tiles is
// a piece of its own (slot 0).  Only the first piece needs a division.
struct CutPieces {
  long long a, T, W, w_first, w_last;
  int n, slot_first;
  __device__ __forceinline__ CutPieces(long long a_, int nb, long long T_, long long W_) : a(a_), T(T_), W(W_) {
    w_first = floor_div((a + 1) * W - 1, T);
    w_last = floor_div((a + nb) * W - 1, T);
    n = T >= W ? (int)(w_last - w_first + 1) : nb;
    slot_first = T >= W && floor_div(w_first * T, W) < a ? 1 : 0;
  }
  // partial slot (wave * 2 + slot) of piece k < n
  __device__ __forceinline__ long long slot(int k) const {
    if (T >= W) return (w_first + k) * 2 + (k == 0 ? slot_first : 0);
    return floor_div((a + k + 1) * W - 1, T) * 2;
  }
};

// A row of the work list and what the waves need to know about it.
struct RowCtx {
  int hg, s;      // head group, sequence
  int nb;         // table entries (tiles) of the row
  long long a;    // first tile of the row in the work list
};

// Tile ring entry: loads in flight plus the tile's place in its row.
template <int D, bool FP8>
struct StreamTile {
  MfmaTiles<D, FP8> t;
  int j;       // table entry within the row
  int row_id;  // rows of this wave counted from 0
};

// FUSED: the step also stores each sequence's new token (k_new/v_new at
// slot_mapping[s], the decode-phase append of [Optimizing] The Block Manager
// and Dynamic Allocation Lifecycle) and attends with it at position
// seq_lens[s] - 1: the wave that computes a row's last block takes the new
// key/value from registers instead of the pool, and the wave of the KV
// head's first head group writes them to the pool.  No wave reads a slot
// another wave writes in the same launch (the slot lies in the sequence's
// own last block), so no ordering between waves is needed.  Into an FP8
// pool the new token goes as its codes (the same rounding as cache_write),
// and the attention uses those codes.
// NT: the tiles are read with non-temporal loads (no block of the batch is
// listed by two rows), else with cached ones.
template <int D, int DEPTH, bool FUSED, bool FP8, int BS, bool NT>  // BS = log2(block size / 16)
__global__ __launch_bounds__(kThreads, KVP_STREAM_WAVES_PER_EU) void decode_stream_kernel(const DecodeParams P) {
  constexpr int NBUF = DEPTH + 1;
  __shared__ int pre[kMaxStreamSeqs + 1];  // pre[s] = tiles of sequences < s
  __shared__ uint8_t t0s[BS ? kMaxStreamSeqs : 1];  // the first attended tile's place in its block
  __shared__ int wsum[kWaves];
  __shared__ int ctxs[kMaxStreamSeqs];  // seq_lens, read once: the rows' spans come from here
  const int ptiles = P.prefix_blocks << BS;  // tiles of the shared prefix (cascade)
  const int S = P.num_seqs;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // Tiles per sequence and their prefix sums: each thread a contiguous run
  // of sequences, a wave scan of the runs, then the waves' totals.
  {
    const int per = (S + kThreads - 1) / kThreads;
    const int s0 = threadIdx.x * per;
    int local = 0;
    for (int i = 0; i < per; ++i) {
      const int s = s0 + i;
      if (s < S) {
        const int ctx = P.seq_lens[s];
        ctxs[s] = ctx;
        const RowSpan rs = row_span(ctx, P.window, P.max_blocks, BS);
        const int nb = max(rs.nblocks - ptiles, 0);
        pre[s + 1] = nb;
        if constexpr (BS != 0) t0s[s] = (uint8_t)rs.t0;
        local += nb;
      }
    }
    const int incl = wave_scan(local, lane);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int run = incl - local;
    for (int w = 0; w < wave; ++w) run += wsum[w];
    if (threadIdx.x == 0) pre[0] = 0;
    for (int i = 0; i < per; ++i) {
      const int s = s0 + i;
      if (s < S) {
        run += pre[s + 1];
        pre[s + 1] = run;
      }
    }
    __syncthreads();
  }
  const int per_row = pre[S];
  const int HG = P.num_kv_heads * P.qgroups;
  const long long T = (long long)per_row * HG;

  if (blockIdx.x == 0) {
    // publish the prefix sums for the merge pass; zero the rows of empty
    // sequences (with a shared prefix the merge pass writes every row)
    for (int i = threadIdx.x; i <= S; i += kThreads) P.prefix[i] = pre[i];
    if (P.prefix_blocks == 0)  // each thread the empty rows among sequences t, t + 256, ...
      for (int s = threadIdx.x; s < S; s += kThreads)
        if (pre[s + 1] == pre[s]) {
          uint4_v* o = (uint4_v*)((uint16_t*)P.out + (size_t)s * P.num_q_heads * D);
          for (int i = 0; i < P.num_q_heads * D / 8; ++i) o[i] = uint4_v{0, 0, 0, 0};
        }
  }

  const long long W = (long long)gridDim.x * kWaves;
  const long long widx = (long long)xcd_major_index(blockIdx.x, gridDim.x) * kWaves + wave;
  const long long t_begin = floor_div(widx * T, W), t_end = floor_div((widx + 1) * T, W);
  const int n_tiles = (int)(t_end - t_begin);
  if (n_tiles <= 0) return;

  const void* pool = P.pool_layer;
  const uint16_t* q = (const uint16_t*)P.q;

  auto row_at = [&](long long t) {  // row holding tile t
    RowCtx r;
    r.hg = (int)(t / per_row);
    const int rr = (int)(t - (long long)r.hg * per_row);
    int lo = 0, hi = S;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pre[mid] <= rr) lo = mid; else hi = mid;
    }
    r.s = lo;
    r.nb = pre[lo + 1] - pre[lo];
    r.a = (long long)r.hg * per_row + pre[lo];
    return r;
  };
  auto row_after = [&](const RowCtx& r) {  // next non-empty row of the work list
    return row_at(r.a + r.nb < T ? r.a + r.nb : T - 1);
  };
  auto head0 = [&](int hg) {
    const int kvh = hg / P.qgroups;
    return kvh * P.group + (hg - kvh * P.qgroups) * P.heads_per_wg;
  };
  auto heads = [&](int hg) {
    const int kvh = hg / P.qgroups;
    return min(P.heads_per_wg, P.group - (hg - kvh * P.qgroups) * P.heads_per_wg);
  };

  // Table entry holding tile j (counted after the shared prefix) of sequence
  // s's row; t0 is the row's first tile in its block.
  auto tid = [&](int s, int t0, int j) { return P.block_tables[(size_t)s * P.max_blocks + ((t0 + ptiles + j) >> BS)]; };
  auto t0_of = [&](int s) { return BS ? (int)t0s[s] : 0; };

  // ---- issue side: walks the range DEPTH tiles ahead of the compute ----
  RowCtx ir = row_at(t_begin);  // row of the next tile to issue
  int ij = (int)(t_begin - ir.a);
  int irow_id = 0;
  int it0 = t0_of(ir.s);
  int ids_a = ij + lane < ir.nb ? tid(ir.s, it0, ij + lane) : 0;            // blocks of tiles ij .. ij+63
  int ids_b = ij + 64 + lane < ir.nb ? tid(ir.s, it0, ij + 64 + lane) : 0;  // tiles ij+64 .. ij+127
  int ids_base = ij;                                                         // tile held by lane 0 of ids_a
  RowCtx nr = row_after(ir);                                                 // the row after, prefetched
  int nt0 = t0_of(nr.s);
  int ids_n = lane < nr.nb ? tid(nr.s, nt0, lane) : 0;
  constexpr int SUB = (1 << BS) - 1;
  MfmaLanes ila = mfma_lanes<D, BS, FP8>(P.num_kv_heads, ir.hg / P.qgroups, lane);
  int issued = 0;

  auto issue = [&](StreamTile<D, FP8>& x) {
    if (issued >= n_tiles) {  // past the range: loads of a line just read (the current row's queries)
      mfma_issue_hot(x.t, q + ((size_t)ir.s * P.num_q_heads + head0(ir.hg)) * D);
      x.j = -1;
      return;
    }
    if (ij == ir.nb) {  // row change: the prefetched row becomes current
      ir = nr;
      ij = 0;
      ++irow_id;
      it0 = nt0;
      ids_a = ids_n;
      ids_b = 64 + lane < ir.nb ? tid(ir.s, it0, 64 + lane) : 0;
      ids_base = 0;
      nr = row_after(ir);
      nt0 = t0_of(nr.s);
      ids_n = lane < nr.nb ? tid(nr.s, nt0, lane) : 0;
      ila = mfma_lanes<D, BS, FP8>(P.num_kv_heads, ir.hg / P.qgroups, lane);
    } else if (ij - ids_base == 64) {  // next chunk of 64 tiles: rotate, fetch the one after
      ids_a = ids_b;
      ids_base += 64;
      ids_b = ids_base + 64 + lane < ir.nb ? tid(ir.s, it0, ids_base + 64 + lane) : 0;
    }
    mfma_issue<BS, NT>(x.t, pool, ila, __builtin_amdgcn_readlane(ids_a, ij - ids_base), (it0 + ptiles + ij) & SUB,
                       P.num_blocks);
    x.j = ij;
    x.row_id = irow_id;
    ++ij;
    ++issued;
  };

  // ---- compute side ----
  RowCtx cr = row_at(t_begin);
  int crow_id = 0;
  int c_h0 = head0(cr.hg), c_nh = heads(cr.hg);
  RowSpan crs = row_span(ctxs[cr.s], P.window, P.max_blocks, BS);
  MfmaRow<D> st;
  st.template load_q<FP8>(q, (size_t)cr.s * P.num_q_heads + c_h0, c_nh, lane);
  st.reset();
  // queries and length of the next row, fetched ahead
  RowCtx qn = row_after(cr);
  int ctx_next = ctxs[qn.s];
  uint4_v q_next[D / 32];
  {
    const int g = lane & 15, nh_n = heads(qn.hg);
    const uint16_t* qp = q + ((size_t)qn.s * P.num_q_heads + head0(qn.hg) + g) * D;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      q_next[kk] = g < nh_n ? *(const uint4_v*)(qp + qk_dim<FP8>(kk, lane >> 4)) : uint4_v{0, 0, 0, 0};
  }

  auto finish_row = [&]() {
    const float l_tot = rows_sum(st.l_run);
    const int q4 = lane >> 4;
    const long long ra = cr.a, rb = cr.a + cr.nb;
    if (ra >= t_begin && rb <= t_end && P.prefix_blocks > 0) {
      // a whole tail of a row with a shared prefix: its partial goes to the
      // row's own slot, for the merge with the prefix pass
      const size_t pbase = ((size_t)cr.hg * S + cr.s) * P.heads_per_wg;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int g = 4 * q4 + r4;
        if (g < c_nh) st.template store_partial<FP8>(P.row_o + (pbase + g) * D, r4, lane);
      }
      if (lane < c_nh) {
        P.row_ml[(pbase + lane) * 2 + 0] = st.m_run;
        P.row_ml[(pbase + lane) * 2 + 1] = l_tot;
      }
    } else if (ra >= t_begin && rb <= t_end) {
      // the whole row is here: normalise and store
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int g = 4 * q4 + r4;
        const float lg = __shfl(l_tot, g);
        const float inv = lg > 0.f ? P.v_scale / lg : 0.f;
        if (g < c_nh)
          st.template store_out<FP8>((uint16_t*)P.out + ((size_t)cr.s * P.num_q_heads + c_h0 + g) * D, r4, inv, lane);
      }
    } else {
      const int slot = ra <= t_begin ? 0 : 1;
      const size_t pbase = (size_t)(widx * 2 + slot) * P.heads_per_wg;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int g = 4 * q4 + r4;
        if (g < c_nh) st.template store_partial<FP8>(P.part_o + (pbase + g) * D, r4, lane);
      }
      if (lane < c_nh) *(float2*)(P.part_ml + (pbase + lane) * 2) = make_float2(st.m_run, l_tot);
    }
  };

  // The new token of the current and of the next row (FUSED only): lanes
  // 0..D/8-1 hold its key (8 dims each), lanes 0..D/2-1 its value (2 dims
  // each), every lane its slot as loaded.  Nothing reads them before the
  // row's last tile, so the loads never hold up the tile loads behind them.
  uint4_v kn = {0, 0, 0, 0}, kn_next = {0, 0, 0, 0};
  unsigned vn = 0, vn_next = 0;
  int slot_c = -1, slot_next = -1;
  auto load_new = [&](const RowCtx& r, uint4_v& kd, unsigned& vd, int& sd) {
    if constexpr (FUSED) {
      sd = P.slot_mapping[r.s];
      const size_t tok = ((size_t)r.s * P.num_kv_heads + r.hg / P.qgroups) * D;
      kd = lane < D / 8 ? ((const uint4_v*)((const uint16_t*)P.k_new + tok))[lane] : uint4_v{0, 0, 0, 0};
      vd = lane < D / 2 ? ((const unsigned*)((const uint16_t*)P.v_new + tok))[lane] : 0u;
    }
  };
  load_new(cr, kn, vn, slot_c);
  load_new(qn, kn_next, vn_next, slot_next);

  // The row's last block holds the new token at table slot send - 1: put
  // its key and value into this wave's operands (layouts of mfma_tile.h),
  // and store them into the pool once per KV head.
  auto put_new = [&](MfmaTiles<D, FP8>& t, int slot) {
    const int o = (crs.start_off + crs.n - 1) & (kBlock - 1);
    const int q4 = lane >> 4, j = lane & 15;
    constexpr int B = kBlock << BS;  // tokens per block
    const int kvh = cr.hg / P.qgroups, b = slot >> (4 + BS), off = slot & (B - 1);
    const bool writer = cr.hg % P.qgroups == 0;
    const size_t blk = (size_t)b * 2 * P.num_kv_heads * B * D;
    const size_t kt = blk + (size_t)kvh * B * D, vt = blk + (size_t)(P.num_kv_heads + kvh) * B * D;
    const int e = ((off >> 2) * D + 2 * lane) * 4 + (off & 3);  // this lane's first V element
    if constexpr (FP8) {
      const uint2_v kc = fp8_quant8(kn, P.inv_k_scale);  // codes of dims 8 lane .. +7
      const unsigned vc = fp8_quant2(vn, P.inv_v_scale);  // codes of dims 2 lane, +1
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        const int src = qk_dim<true>(kk, q4) >> 3;  // lane holding the codes of MFMA kk's dims
        const uint2_v v = {(unsigned)__shfl((int)kc.x, src), (unsigned)__shfl((int)kc.y, src)};
        if (j == o) t.k[kk] = v;
      }
      const int sh = 8 * (o & 3);
      const unsigned keep = ~(0xffu << sh);
      // word e of t.v[h] holds dim 64 h + 4 j + e (its four tokens' codes)
#pragma unroll
      for (int h = 0; h < D / 64; ++h) {
        const unsigned na = (unsigned)__shfl((int)vc, 32 * h + 2 * j);      // dims 64 h + 4 j (byte 0), +1 (byte 1)
        const unsigned nb = (unsigned)__shfl((int)vc, 32 * h + 2 * j + 1);  // dims 64 h + 4 j + 2, +3
        if (q4 == (o >> 2)) {
          t.v[h].x = (t.v[h].x & keep) | ((na & 0xffu) << sh);
          t.v[h].y = (t.v[h].y & keep) | (((na >> 8) & 0xffu) << sh);
          t.v[h].z = (t.v[h].z & keep) | ((nb & 0xffu) << sh);
          t.v[h].w = (t.v[h].w & keep) | (((nb >> 8) & 0xffu) << sh);
        }
      }
      if (writer) {
        uint8_t* pl = (uint8_t*)P.pool_layer;
        if (lane < D / 8) *(uint2_v*)(pl + kt + off * D + 8 * lane) = kc;
        if (lane < D / 2) {
          pl[vt + e] = (uint8_t)(vc & 0xffu);
          pl[vt + e + 4] = (uint8_t)((vc >> 8) & 0xffu);
        }
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        const int src = qk_dim<false>(kk, q4) >> 3;  // lane holding dims 32 kk + 8 q4 .. +7
        const uint4_v v = {(unsigned)__shfl((int)kn.x, src), (unsigned)__shfl((int)kn.y, src),
                           (unsigned)__shfl((int)kn.z, src), (unsigned)__shfl((int)kn.w, src)};
        if (j == o) t.k[kk] = v;
      }
      const bool hi = (o & 1) != 0;
      const unsigned keep = hi ? 0x0000ffffu : 0xffff0000u;
      const int sh = hi ? 16 : 0;
#pragma unroll
      for (int m = 0; m < D / 32; ++m) {
        const unsigned nv = (unsigned)__shfl((int)vn, 16 * m + j);  // dims 32 m + 2 j (low half), +1
        if (q4 == (o >> 2)) {
          const unsigned d0 = (nv & 0xffffu) << sh, d1 = (nv >> 16) << sh;
          if ((o & 2) == 0) {
            t.v[m].x = (t.v[m].x & keep) | d0;
            t.v[m].z = (t.v[m].z & keep) | d1;
          } else {
            t.v[m].y = (t.v[m].y & keep) | d0;
            t.v[m].w = (t.v[m].w & keep) | d1;
          }
        }
      }
      if (writer) {
        uint16_t* pl = (uint16_t*)P.pool_layer;
        if (lane < D / 8) *(uint4_v*)(pl + kt + off * D + 8 * lane) = kn;
        if (lane < D / 2) {
          pl[vt + e] = (uint16_t)(vn & 0xffffu);
          pl[vt + e + 4] = (uint16_t)(vn >> 16);
        }
      }
    }
  };

  auto compute = [&](StreamTile<D, FP8>& x) {
    if (x.row_id != crow_id) {  // first tile of the next row
      finish_row();
      cr = qn;
      if constexpr (FUSED) {
        kn = kn_next;
        vn = vn_next;
        slot_c = slot_next;
      }
      ++crow_id;
      c_h0 = head0(cr.hg);
      c_nh = heads(cr.hg);
      crs = row_span(ctx_next, P.window, P.max_blocks, BS);
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) st.qop[kk] = q_next[kk];
      st.reset();
      qn = row_after(cr);
      ctx_next = ctxs[qn.s];
      const int g = lane & 15, nh_n = heads(qn.hg);
      const uint16_t* qp = q + ((size_t)qn.s * P.num_q_heads + head0(qn.hg) + g) * D;
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)
        q_next[kk] = g < nh_n ? *(const uint4_v*)(qp + qk_dim<FP8>(kk, lane >> 4)) : uint4_v{0, 0, 0, 0};
      load_new(qn, kn_next, vn_next, slot_next);
    }
    const int J = ptiles + x.j;  // the tile's place in the row span
    if constexpr (FUSED) {
      if (J == crs.nblocks - 1) {
        // a slot outside the pool (or negative: no new token) writes nothing
        const int sl = __builtin_amdgcn_readfirstlane(slot_c);
        if (sl >= 0 && sl < (P.num_blocks << (4 + BS))) put_new(x.t, sl);
      }
    }
    st.step(x.t, J, crs.start_off, crs.start_off + crs.n, crs.nblocks, P.scale_log2, lane);
  };

  StreamTile<D, FP8> buf[NBUF];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    issue(buf[d]);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int k0 = 0; k0 < n_tiles; k0 += NBUF) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      if (k0 + u >= n_tiles) break;
      __builtin_amdgcn_s_setprio(1);  // the next tile's loads go out ahead of the other wave's compute
      issue(buf[(u + DEPTH) % NBUF]);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      compute(buf[u]);
    }
  }
  finish_row();
}

// Merge of the rows cut by range boundaries.  One wave per (sequence,
// query head): the row's tiles [a, b) were covered by the waves w_first ..
// w_last; each left its partial in slot 0 (the row held the wave's first
// tile) or slot 1 (the row was the wave's last).  Rows inside one wave were
// stored by the first pass.  The partials' loads go out eight at a time.
// With a shared prefix every row is merged here: the prefix pass's piece,
// then either the row's own slot (a tail inside one wave) or the wave
// slots (a tail cut by range boundaries); a row with no tail is the prefix
// piece alone.
template <int D>
__global__ __launch_bounds__(256) void decode_stream_reduce_kernel(const DecodeParams P) {
  const int s = blockIdx.y;
  const int h = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (h >= P.num_q_heads) return;
  const int lane = threadIdx.x & 63;
  const int S = P.num_seqs;
  const bool cascade = P.prefix_blocks > 0;
  const int kvh = h / P.group, g_in = h - kvh * P.group;
  const int qg = g_in / P.heads_per_wg, hh = g_in - qg * P.heads_per_wg;
  const int hg = kvh * P.qgroups + qg;

  constexpr int PER = D / 64;
  float M = -INFINITY, den = 0.f, num[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) num[e] = 0.f;
  // With a shared prefix, the prefix pass's piece and the row's own slot
  // do not depend on the prefix sums: their loads go out with them.
  float rm = -INFINITY, rl = 0.f, ro[PER];
  if (cascade) {
    // the prefix pass's pieces (one per key chunk, in chunk order)
    static_assert(kMaxPrefixPieces <= kMergeChunk, "one merge round takes every prefix piece");
    const size_t qh = (size_t)s * P.num_q_heads + h, pstride = (size_t)S * P.num_q_heads;
    float m[kMergeChunk], l[kMergeChunk], v[kMergeChunk][PER];
#pragma unroll
    for (int u = 0; u < kMergeChunk; ++u) {
      const bool use = u < P.prefix_pieces;
      const size_t pq = qh + (use ? u : 0) * pstride;
      const float2 ml = *(const float2*)(P.pre_ml + pq * 2);
      m[u] = use ? ml.x : -INFINITY;
      l[u] = use ? ml.y : 0.f;
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const float x = P.pre_o[pq * D + lane + 64 * e];
        v[u][e] = use ? x : 0.f;
      }
    }
    const size_t rb = ((size_t)hg * S + s) * P.heads_per_wg + hh;
    rm = P.row_ml[rb * 2];
    rl = P.row_ml[rb * 2 + 1];
#pragma unroll
    for (int e = 0; e < PER; ++e) ro[e] = P.row_o[rb * D + lane + 64 * e];
    merge_round(M, den, num, m, l, v);
  }
  const int pre_s = P.prefix[s], nb = P.prefix[s + 1] - pre_s, per_row = P.prefix[S];
  if (nb == 0 && !cascade) return;
  // merge one more piece (max m, sum l, unnormalised o)
  auto add = [&](float m, float l, const float* o) {
    const float Mc = fmaxf(M, m);
    if (Mc == -INFINITY) return;
    const float a = __builtin_amdgcn_exp2f(M - Mc), b = __builtin_amdgcn_exp2f(m - Mc);
    den = den * a + l * b;
#pragma unroll
    for (int e = 0; e < PER; ++e) num[e] = num[e] * a + o[e] * b;
    M = Mc;
  };

  if (nb > 0) {
    const long long T = (long long)per_row * P.num_kv_heads * P.qgroups;
    const long long W = (long long)P.stream_wgs * kWaves;
    const long long a = (long long)hg * per_row + pre_s;
    const CutPieces pc(a, nb, T, W);
    if (pc.n == 1) {
      if (!cascade) return;  // stored by the first pass
      add(rm, rl, ro);       // the tail one wave held whole
    } else {
      constexpr int CH = kMergeChunk;
      for (int k0 = 0; k0 < pc.n; k0 += CH) {
        float m[CH], l[CH], v[CH][PER];
#pragma unroll
        for (int u = 0; u < CH; ++u) {
          const bool use = k0 + u < pc.n;
          const size_t pb = (size_t)pc.slot(use ? k0 + u : pc.n - 1) * P.heads_per_wg + hh;
          const float2 ml = *(const float2*)(P.part_ml + pb * 2);
          m[u] = use ? ml.x : -INFINITY;
          l[u] = use ? ml.y : 0.f;
#pragma unroll
          for (int e = 0; e < PER; ++e) {
            const float x = P.part_o[pb * D + lane + 64 * e];
            v[u][e] = use ? x : 0.f;
          }
        }
        merge_round(M, den, num, m, l, v);
      }
    }
  }
  const float inv = den > 0.f ? P.v_scale / den : 0.f;
  uint16_t* out = (uint16_t*)P.out + ((size_t)s * P.num_q_heads + h) * D;
#pragma unroll
  for (int e = 0; e < PER; ++e) out[lane + 64 * e] = bf16_rne(num[e] * inv);
}

// The shared-prefix pass on the prefill kernel: all S * G decode queries of
// a KV head against the prefix, key chunk by key chunk.
hipError_t launch_prefix(const DecodeParams& p, int head_dim, hipStream_t stream) {
  PrefillParams f{};
  f.pool_layer = p.pool_layer;
  f.q = p.q;
  f.block_tables = p.block_tables;
  f.max_blocks = p.max_blocks;
  f.num_seqs = p.num_seqs;
  f.num_q_heads = p.num_q_heads;
  f.num_kv_heads = p.num_kv_heads;
  f.num_blocks = p.num_blocks;
  f.bshift = p.bshift;
  f.group = p.group;
  f.window = 0;
  f.qtiles = (p.num_seqs * p.group + 127) / 128;
  f.scale_log2 = p.scale_log2;
  f.v_scale = p.v_scale;
  f.prefix_blocks = p.prefix_blocks;
  f.prefix_pieces = p.prefix_pieces;
  f.prefix_chunk = p.prefix_chunk;
  f.pre_o = p.pre_o;
  f.pre_ml = p.pre_ml;
  return launch_prefix_pass(f, head_dim, p.kv_fp8 != 0, stream);
}

template <int D, int DEPTH, bool FP8, int BS, bool NT>
void launch_sk(const DecodeParams& p, hipStream_t stream) {
  if (p.slot_mapping) {
    // the fused step runs at ring depth 1: the new token takes the registers of a deeper ring
    hipLaunchKernelGGL((decode_stream_kernel<D, 1, true, FP8, BS, NT>), dim3(p.stream_wgs), dim3(kThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL((decode_stream_kernel<D, DEPTH, false, FP8, BS, NT>), dim3(p.stream_wgs), dim3(kThreads), 0, stream,
                       p);
  }
}

template <int D, int DEPTH, bool FP8, int BS>
hipError_t launch_sd(const DecodeParams& p, hipStream_t stream) {
  if (p.slot_mapping && DEPTH != 1) return hipErrorInvalidValue;
  if (p.prefix_blocks > 0) {
    const hipError_t e = launch_prefix(p, D, stream);
    if (e != hipSuccess) return e;
  }
  if (p.nt_loads) launch_sk<D, DEPTH, FP8, BS, true>(p, stream);
  else launch_sk<D, DEPTH, FP8, BS, false>(p, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((p.num_q_heads + 3) / 4, p.num_seqs);
  hipLaunchKernelGGL((decode_stream_reduce_kernel<D>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool FP8, int BS>
hipError_t launch_s(const DecodeParams& p, hipStream_t stream) {
  switch (p.depth) {
    case 1: return launch_sd<D, 1, FP8, BS>(p, stream);
    case 2: return launch_sd<D, 2, FP8, BS>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t launch_st(const DecodeParams& p, hipStream_t stream) {
  if (p.kv_fp8) return p.bshift ? launch_s<D, true, 1>(p, stream) : launch_s<D, true, 0>(p, stream);
  return p.bshift ? launch_s<D, false, 1>(p, stream) : launch_s<D, false, 0>(p, stream);
}

template <int D, bool FP8, int BS, bool NT>
const void* symbol_of(int depth, bool fused) {
  if (fused) return depth == 1 ? (const void*)decode_stream_kernel<D, 1, true, FP8, BS, NT> : nullptr;
  return depth == 1 ? (const void*)decode_stream_kernel<D, 1, false, FP8, BS, NT>
                    : (const void*)decode_stream_kernel<D, 2, false, FP8, BS, NT>;
}

template <int D, bool NT>
const void* symbol_d(int depth, bool fused, bool fp8, int bshift) {
  if (fp8) return bshift ? symbol_of<D, true, 1, NT>(depth, fused) : symbol_of<D, true, 0, NT>(depth, fused);
  return bshift ? symbol_of<D, false, 1, NT>(depth, fused) : symbol_of<D, false, 0, NT>(depth, fused);
}

}  // namespace

const void* stream_kernel_symbol(int head_dim, int depth, bool fused, bool fp8, int bshift, bool nt) {
  if (nt) return head_dim == 128 ? symbol_d<128, true>(depth, fused, fp8, bshift) : symbol_d<64, true>(depth, fused, fp8, bshift);
  return head_dim == 128 ? symbol_d<128, false>(depth, fused, fp8, bshift) : symbol_d<64, false>(depth, fused, fp8, bshift);
}

hipError_t launch_decode_stream(const DecodeParams& p, int head_dim, hipStream_t stream) {
  if (head_dim == 128) return launch_st<128>(p, stream);
  if (head_dim == 64) return launch_st<64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace kvp
