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
#include "prefill_common.h"

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

// The products and sums are written out (explicit fma, no contraction left
// to the compiler), so every kernel that merges pieces gets the same bits.
template <int PER, int CH>
__device__ __forceinline__ void merge_round(float& M, float& den, float (&num)[PER], const float (&m)[CH],
                                            const float (&l)[CH], const float (&v)[CH][PER]) {
#pragma clang fp contract(off)
  float Mc = M;
#pragma unroll
  for (int u = 0; u < CH; ++u) Mc = fmaxf(Mc, m[u]);
  if (Mc == -INFINITY) return;
  const float ao = __builtin_amdgcn_exp2f(M - Mc);
  den = den * ao;
#pragma unroll
  for (int e = 0; e < PER; ++e) num[e] = num[e] * ao;
#pragma unroll
  for (int u = 0; u < CH; ++u) {
    const float f = __builtin_amdgcn_exp2f(m[u] - Mc);
    den = __builtin_fmaf(f, l[u], den);
#pragma unroll
    for (int e = 0; e < PER; ++e) num[e] = __builtin_fmaf(f, v[u][e], num[e]);
  }
  M = Mc;
}

// One more piece (max m, sum l, unnormalised o) into the merge, the
// products and sums written out like merge_round's.
template <int PER>
__device__ __forceinline__ void merge_one(float& M, float& den, float (&num)[PER], float m, float l,
                                          const float (&o)[PER]) {
#pragma clang fp contract(off)
  const float Mc = fmaxf(M, m);
  if (Mc == -INFINITY) return;
  const float a = __builtin_amdgcn_exp2f(M - Mc), b = __builtin_amdgcn_exp2f(m - Mc);
  den = __builtin_fmaf(l, b, den * a);
#pragma unroll
  for (int e = 0; e < PER; ++e) num[e] = __builtin_fmaf(o[e], b, num[e] * a);
  M = Mc;
}

// The pieces of a cut row [a, a + nb) of the work list (T tiles over W
// waves), in wave order, found from the split alone (the merge uses it
// when T < W; otherwise the first pass records where each row's pieces are).  With T >= W every range holds a tile, so they are
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
  int kvh;        // KV head of the head group
  int h0, nh;     // its first query head and how many it serves
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
// LDS of one streaming workgroup.
template <int BS>
struct StreamLds {
  int pre[kMaxStreamSeqs + 1];               // pre[s] = tiles of sequences < s
  uint8_t t0s[BS ? kMaxStreamSeqs : 1];      // the first attended tile's place in its block
  int wsum[kWaves];
  int ctxs[kMaxStreamSeqs];                  // seq_lens, read once: the rows' spans come from here
};

// Loads of another wave's partial results, through the L2 of this XCD
// (agent-scope loads miss the compute unit's L1).
__device__ __forceinline__ float l2_load(const float* p) {
  return __builtin_bit_cast(float, __hip_atomic_load((const unsigned*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ uint64_t l2_load(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kMergePolls = 1 << 18;  // a bound on each wait for a piece (~0.1 s), far past any wait of a call

// The merge of the cut rows inside the streaming launch (P.merge_wgs > 0),
// for batches whose rows never cross an XCD: the KV heads split evenly over
// the 8 XCDs (Hkv % 8 == 0, one head group per KV head) and the streaming
// grid a multiple of 8 workgroups, so the waves of XCD x (workgroups x, x
// + 8, ...) stream exactly KV heads [x Hkv / 8, (x + 1) Hkv / 8).  Merge
// workgroup m runs on XCD m mod 8 (launched after every streaming
// workgroup, it starts on a compute unit one of them has left) and takes
// four query heads of that XCD for one sequence.  A wave stores its
// partials, waits for its stores, then writes this call's mark (P.epoch)
// beside each (slot, head); the merging wave waits for the marks of the
// row's pieces, reads them through the shared L2, merges them as the merge
// kernel does (the same rounds, so the same bits), stores the output and
// clears the marks.  The streaming workgroups are all dispatched before any
// merge workgroup (in-order dispatch), so every wait ends.
template <int D, int BS>
__device__ __forceinline__ void merge_in_launch(const DecodeParams& P, int m, StreamLds<BS>& L) {
  const int S = P.num_seqs;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // prefix sums of the rows' tiles, as the streaming workgroups compute them
  {
    const int per = (S + kThreads - 1) / kThreads;
    const int s0 = threadIdx.x * per;
    int local = 0;
    for (int i = 0; i < per; ++i) {
      const int s = s0 + i;
      if (s < S) {
        const RowSpan rs = row_span(P.seq_lens[s], P.window, P.max_blocks, BS);
        L.pre[s + 1] = rs.nblocks;
        local += rs.nblocks;
      }
    }
    const int incl = wave_scan(local, lane);
    if (lane == 63) L.wsum[wave] = incl;
    __syncthreads();
    int run = incl - local;
    for (int w = 0; w < wave; ++w) run += L.wsum[w];
    if (threadIdx.x == 0) L.pre[0] = 0;
    for (int i = 0; i < per; ++i) {
      const int s = s0 + i;
      if (s < S) {
        run += L.pre[s + 1];
        L.pre[s + 1] = run;
      }
    }
    __syncthreads();
  }
  // this wave's (sequence, query head)
  const int hpx = P.num_q_heads / 8;  // query heads of one XCD
  const int wps = (hpx + 3) / 4;      // merge workgroups per (XCD, sequence)
  const int x = m & 7, k = m >> 3;
  const int s = k / wps, j = 4 * (k - s * wps) + wave;
  if (s >= S || j >= hpx) return;
  const int h = x * hpx + j;
  const int kvh = h / P.group, hh = h - kvh * P.group;  // one head group per KV head here
  const int per_row = L.pre[S], nb = L.pre[s + 1] - L.pre[s];
  if (nb == 0) return;  // an empty row: zeroed by the first streaming workgroup
  const long long T = (long long)per_row * P.num_kv_heads, W = (long long)P.stream_wgs * kWaves;
  const CutPieces pc((long long)kvh * per_row + L.pre[s], nb, T, W);
  const int n = pc.n;
  if (n == 1) return;  // the row lay inside one wave's range: stored there
  const unsigned hpw = (unsigned)P.heads_per_wg;
  // wait for the pieces' marks, 64 at a time
  for (int k0 = 0; k0 < n; k0 += 64) {
    const int kk = k0 + lane;
    const unsigned pb = kk < n ? (unsigned)pc.slot(kk) * hpw + hh : 0u;
    bool ready = kk >= n;
    for (int it = 0; it < kMergePolls; ++it) {
      if (!ready) ready = l2_load(P.flags + pb) == P.epoch;
      if (__all(ready)) break;
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  constexpr int PER = D / 64;
  float M = -INFINITY, den = 0.f, num[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) num[e] = 0.f;
  constexpr int CH = kMergeChunk;
  for (int k0 = 0; k0 < n; k0 += CH) {
    float mm[CH], l[CH], v[CH][PER];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const bool use = k0 + u < n;
      const unsigned pb = (unsigned)pc.slot(use ? k0 + u : n - 1) * hpw + hh;
      const float a = l2_load(P.part_ml + pb * 2u), b = l2_load(P.part_ml + pb * 2u + 1u);
      mm[u] = use ? a : -INFINITY;
      l[u] = use ? b : 0.f;
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const float xv = l2_load(P.part_o + pb * (unsigned)D + lane + 64 * e);
        v[u][e] = use ? xv : 0.f;
      }
    }
    merge_round(M, den, num, mm, l, v);
  }
  const float inv = den > 0.f ? P.v_scale / den : 0.f;
  uint16_t* out = (uint16_t*)P.out + ((size_t)s * P.num_q_heads + h) * D;
#pragma unroll
  for (int e = 0; e < PER; ++e) out[lane + 64 * e] = bf16_rne(num[e] * inv);
  // clear the marks for the next call
  for (int k0 = 0; k0 < n; k0 += 64) {
    const int kk = k0 + lane;
    if (kk < n) P.flags[(unsigned)pc.slot(kk) * hpw + hh] = 0;
  }
}

template <int D, int DEPTH, bool FUSED, bool FP8, int BS, bool NT>  // BS = log2(block size / 16)
__global__ __launch_bounds__(kThreads, KVP_STREAM_WAVES_PER_EU) void decode_stream_kernel(const DecodeParams P) {
  __shared__ StreamLds<BS> lds;
  StreamLds<BS>& L = lds;
  if ((int)blockIdx.x >= P.stream_wgs) {  // a merge workgroup (P.merge_wgs > 0)
    merge_in_launch<D, BS>(P, (int)blockIdx.x - P.stream_wgs, L);
    return;
  }
  const int wg = blockIdx.x, nwg = P.stream_wgs;
  constexpr bool CASCADE = false;
#include "stream_body.inc"
}

// Cascade decode in one launch: the first P.stream_wgs workgroups stream the
// private tails (the body of decode_stream_kernel), the rest run the
// shared-prefix pass (the prefill body over the prefix's key chunks).  The
// host sizes the two parts to the resident workgroup slots: when the prefix
// pass fits in its share, all of it starts at once beside the streaming
// workgroups, the memory-bound tails and the MFMA-bound prefix pass sharing
// the chip; otherwise the streaming grid fills every slot and the prefix
// workgroups, which start in index order, take the compute units the
// streaming workgroups leave.  The two share one LDS allocation.
template <int D, int DEPTH, bool FUSED, bool FP8, int BS, bool NT>
__global__ __launch_bounds__(kThreads, KVP_STREAM_WAVES_PER_EU) void decode_cascade_kernel(const DecodeParams P,
                                                                                            const PrefillParams PF) {
  __shared__ union {
    StreamLds<BS> s;
    pf::PfLds<D> p;
  } lds;
  if ((int)blockIdx.x < P.stream_wgs) {
    StreamLds<BS>& L = lds.s;
    const int wg = blockIdx.x, nwg = P.stream_wgs;
    constexpr bool CASCADE = true;
#include "stream_body.inc"
  } else {
    using namespace pf;
    constexpr bool PREFIX = true;
    PfLds<D>& L = lds.p;
    const int wg = (int)blockIdx.x - P.stream_wgs;
#include "prefill_body.inc"
  }
}

// Merge of the rows cut by range boundaries.  One wave per (sequence,
// query head): the row's tiles [a, b) were covered by the waves w_first ..
// w_last (recorded by the first pass); each left its partial in slot 0 (the
// row held the wave's first tile) or slot 1 (the row was the wave's last).
// Rows inside one wave were stored by the first pass.  The partials' loads
// go out eight at a time.  At most 64 VGPRs (8 waves per SIMD): every wave
// of the largest merge here (256 sequences x 32 heads) is resident at once.
// With a shared prefix every row is merged here: the prefix pass's chunk
// pieces, then the row's tail: its first kRowSlots pieces were stored by
// row, so their loads go out with the first ones (one round trip for most
// rows), any further ones come from the wave slots; a row with no tail is
// the prefix pieces alone.
template <int D>
__global__ __launch_bounds__(256, 8) void decode_stream_reduce_kernel(const DecodeParams P) {
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
  constexpr int CH = kMergeChunk;

  // the row's place in the work list and its pieces (written by the first
  // pass), loaded first: with a shared prefix the first prefix round's and
  // the row's slots go out while they travel
  const int pre_s = P.prefix[s], nb = P.prefix[s + 1] - pre_s, per_row = P.prefix[S];
  const int2 cut = *(const int2*)(P.cuts + 2 * ((size_t)hg * S + s));

  float M = -INFINITY, den = 0.f, num[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) num[e] = 0.f;
  // the prefix pass's pieces (one per key chunk, in chunk order), in rounds
  // of PR: absent pieces change no bit of a round
  constexpr int PR = 4;
  static_assert(kMaxPrefixPieces <= 2 * PR && kRowSlots <= CH, "piece rounds");
  // (element offsets into the workspace fit 32 bits: the host sizes it)
  const unsigned qh = (unsigned)s * P.num_q_heads + h, pstride = (unsigned)S * P.num_q_heads;
  // load round r0 of the prefix pieces into m, l, v
  auto load_prefix = [&](int r0, float (&m)[PR], float (&l)[PR], float (&v)[PR][PER]) {
    unsigned pq = qh + r0 * pstride;  // stepped by additions (a 64-bit multiply-add here waited for a load)
#pragma unroll
    for (int u = 0; u < PR; ++u, pq += pstride) {
      m[u] = -INFINITY;
      l[u] = 0.f;
#pragma unroll
      for (int e = 0; e < PER; ++e) v[u][e] = 0.f;
      if (r0 + u < P.prefix_pieces) {  // uniform: the absent chunks' loads are skipped
        const float2 ml = *(const float2*)(P.pre_ml + pq * 2u);
        m[u] = ml.x;
        l[u] = ml.y;
#pragma unroll
        for (int e = 0; e < PER; ++e) v[u][e] = P.pre_o[pq * (unsigned)D + lane + 64 * e];
      }
    }
  };
  float rsm[kRowSlots], rsl[kRowSlots], rso[kRowSlots][PER];
  if (cascade) {
    float pm[PR], pl[PR], pv[PR][PER];
    load_prefix(0, pm, pl, pv);
    const unsigned rb = (((unsigned)hg * S + s) * P.heads_per_wg + hh) * kRowSlots;
#pragma unroll
    for (int k = 0; k < kRowSlots; ++k) {
      rsm[k] = P.row_ml[(rb + k) * 2u];
      rsl[k] = P.row_ml[(rb + k) * 2u + 1u];
#pragma unroll
      for (int e = 0; e < PER; ++e) rso[k][e] = P.row_o[(rb + k) * (unsigned)D + lane + 64 * e];
    }
    merge_round(M, den, num, pm, pl, pv);
    if (P.prefix_pieces > PR) {
      load_prefix(PR, pm, pl, pv);
      merge_round(M, den, num, pm, pl, pv);
    }
  } else if (nb == 0) {
    return;
  }

  if (nb > 0) {
    const long long T = (long long)per_row * P.num_kv_heads * P.qgroups;
    const long long W = (long long)P.stream_wgs * kWaves;
    const unsigned first = (unsigned)cut.x;
    // every wave holds a tile (T >= W): the pieces are the waves from the
    // one holding the row's first tile (its recorded piece) to the one
    // holding its last, every later one in slot 0; else each tile is a
    // piece of its own, located by CutPieces
    const int n = T >= W ? cut.y - (int)(first >> 1) + 1 : nb;
    if (n == 1) {
      if (!cascade) return;  // stored by the first pass
      merge_one(M, den, num, rsm[0], rsl[0], rso[0]);  // the tail one wave held whole
    } else {
      const CutPieces pc((long long)hg * per_row + pre_s, nb, T, W);
      auto slot = [&](int k) -> unsigned {
        if (T >= W) return k == 0 ? first : ((first >> 1) + (unsigned)k) * 2u;
        return (unsigned)pc.slot(k);
      };
      // pieces k0 .. n-1 in rounds of CH (unused places load the last piece
      // again: no branch around the loads); with a shared prefix the first
      // kRowSlots come from the row's slots, and a tail of at most that many
      // pieces needs no further load
      auto load_piece = [&](int k, bool use, float& m, float& l, float (&v)[PER]) {
        const unsigned pb = slot(use ? k : n - 1) * (unsigned)P.heads_per_wg + hh;
        const float2 ml = *(const float2*)(P.part_ml + pb * 2u);
        m = use ? ml.x : -INFINITY;
        l = use ? ml.y : 0.f;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const float x = P.part_o[pb * (unsigned)D + lane + 64 * e];
          v[e] = use ? x : 0.f;
        }
      };
      int k0 = 0;
      if (cascade) {
        float m[CH], l[CH], v[CH][PER];
#pragma unroll
        for (int u = 0; u < kRowSlots; ++u) {
          const bool use = u < n;
          m[u] = use ? rsm[u] : -INFINITY;
          l[u] = use ? rsl[u] : 0.f;
#pragma unroll
          for (int e = 0; e < PER; ++e) v[u][e] = use ? rso[u][e] : 0.f;
        }
        if (n <= kRowSlots) {
#pragma unroll
          for (int u = kRowSlots; u < CH; ++u) {
            m[u] = -INFINITY;
            l[u] = 0.f;
#pragma unroll
            for (int e = 0; e < PER; ++e) v[u][e] = 0.f;
          }
        } else {
#pragma unroll
          for (int u = kRowSlots; u < CH; ++u) load_piece(u, u < n, m[u], l[u], v[u]);
        }
        merge_round(M, den, num, m, l, v);
        k0 = CH;
      }
      for (; k0 < n; k0 += CH) {
        float m[CH], l[CH], v[CH][PER];
#pragma unroll
        for (int u = 0; u < CH; ++u) load_piece(k0 + u, k0 + u < n, m[u], l[u], v[u]);
        merge_round(M, den, num, m, l, v);
      }
    }
  }
  const float inv = den > 0.f ? P.v_scale / den : 0.f;
  uint16_t* out = (uint16_t*)P.out + ((size_t)s * P.num_q_heads + h) * D;
#pragma unroll
  for (int e = 0; e < PER; ++e) out[lane + 64 * e] = bf16_rne(num[e] * inv);
}

// Arguments of the shared-prefix pass: all S * G decode queries of a KV
// head against the prefix, key chunk by key chunk.
PrefillParams prefix_params(const DecodeParams& p) {
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
  return f;
}

template <int D, int DEPTH, bool FP8, int BS, bool NT>
void launch_sk(const DecodeParams& p, hipStream_t stream) {
  if (p.prefix_blocks > 0) {
    const PrefillParams f = prefix_params(p);
    const unsigned grid = (unsigned)p.stream_wgs + (unsigned)(f.num_kv_heads * f.qtiles * f.prefix_pieces);
    if (p.slot_mapping)
      hipLaunchKernelGGL((decode_cascade_kernel<D, 1, true, FP8, BS, NT>), dim3(grid), dim3(kThreads), 0, stream, p, f);
    else
      hipLaunchKernelGGL((decode_cascade_kernel<D, DEPTH, false, FP8, BS, NT>), dim3(grid), dim3(kThreads), 0, stream, p,
                         f);
  } else if (p.slot_mapping) {
    // the fused step runs at ring depth 1: the new token takes the registers of a deeper ring
    hipLaunchKernelGGL((decode_stream_kernel<D, 1, true, FP8, BS, NT>), dim3(p.stream_wgs + p.merge_wgs), dim3(kThreads),
                       0, stream, p);
  } else {
    hipLaunchKernelGGL((decode_stream_kernel<D, DEPTH, false, FP8, BS, NT>), dim3(p.stream_wgs + p.merge_wgs),
                       dim3(kThreads), 0, stream, p);
  }
}

template <int D, int DEPTH, bool FP8, int BS>
hipError_t launch_sd(const DecodeParams& p, hipStream_t stream) {
  if (p.slot_mapping && DEPTH != 1) return hipErrorInvalidValue;
  if (p.prefix_blocks > 0 && (long long)p.num_kv_heads * ((p.num_seqs * p.group + 127) / 128) * p.prefix_pieces +
                                     p.stream_wgs > 0x7fffffffLL)
    return hipErrorInvalidValue;
  if (p.nt_loads) launch_sk<D, DEPTH, FP8, BS, true>(p, stream);
  else launch_sk<D, DEPTH, FP8, BS, false>(p, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.merge_wgs > 0) return hipSuccess;  // merged inside the launch
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

template <int D, bool FP8, int BS, bool NT, bool CASCADE>
const void* symbol_of(int depth, bool fused) {
  if constexpr (CASCADE) {
    if (fused) return depth == 1 ? (const void*)decode_cascade_kernel<D, 1, true, FP8, BS, NT> : nullptr;
    return depth == 1 ? (const void*)decode_cascade_kernel<D, 1, false, FP8, BS, NT>
                      : (const void*)decode_cascade_kernel<D, 2, false, FP8, BS, NT>;
  } else {
    if (fused) return depth == 1 ? (const void*)decode_stream_kernel<D, 1, true, FP8, BS, NT> : nullptr;
    return depth == 1 ? (const void*)decode_stream_kernel<D, 1, false, FP8, BS, NT>
                      : (const void*)decode_stream_kernel<D, 2, false, FP8, BS, NT>;
  }
}

template <int D, bool NT, bool CASCADE>
const void* symbol_d(int depth, bool fused, bool fp8, int bshift) {
  if (fp8)
    return bshift ? symbol_of<D, true, 1, NT, CASCADE>(depth, fused) : symbol_of<D, true, 0, NT, CASCADE>(depth, fused);
  return bshift ? symbol_of<D, false, 1, NT, CASCADE>(depth, fused) : symbol_of<D, false, 0, NT, CASCADE>(depth, fused);
}

template <bool CASCADE>
const void* symbol_c(int head_dim, int depth, bool fused, bool fp8, int bshift, bool nt) {
  if (nt)
    return head_dim == 128 ? symbol_d<128, true, CASCADE>(depth, fused, fp8, bshift)
                           : symbol_d<64, true, CASCADE>(depth, fused, fp8, bshift);
  return head_dim == 128 ? symbol_d<128, false, CASCADE>(depth, fused, fp8, bshift)
                         : symbol_d<64, false, CASCADE>(depth, fused, fp8, bshift);
}

}  // namespace

const void* stream_kernel_symbol(int head_dim, int depth, bool fused, bool fp8, int bshift, bool nt, bool cascade) {
  return cascade ? symbol_c<true>(head_dim, depth, fused, fp8, bshift, nt)
                 : symbol_c<false>(head_dim, depth, fused, fp8, bshift, nt);
}

hipError_t launch_decode_stream(const DecodeParams& p, int head_dim, hipStream_t stream) {
  if (head_dim == 128) return launch_st<128>(p, stream);
  if (head_dim == 64) return launch_st<64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace kvp
