// Multi-token (prefill / chunked-prefill) paged attention on the CDNA4
// matrix cores: constants, helpers and LDS of the prefill workgroup (its
// body, prefill_body.inc, is included by the prefill kernel and by the
// cascade decode kernel, whose shared-prefix workgroups run it).
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
#pragma once

#include "mfma_tile.h"

namespace kvp {
namespace pf {

constexpr int kPfRows = 128;         // query rows per workgroup (32 per wave)
constexpr int kLptMaxPairs = 256;    // (sequence, query tile) pairs ranked by work in every workgroup
constexpr int kTiles = 4;            // 16-token tiles per step
constexpr int kStep = 16 * kTiles;   // keys per step (loaded together; computed 32 at a time)

template <bool FP8>
using Elt = std::conditional_t<FP8, uint8_t, uint16_t>;

// Position of 16-byte chunk c (dims 8c .. 8c + 7) within LDS K row r: the
// chunk index XOR the row's low bits.  A QK operand read has lane l take
// chunk 4 kk + l / 16 of row l % 16; unswizzled rows of 256 bytes put all
// 16 rows on the same banks, and rows padded to 272 bytes still read at
// half of the LDS rate on gfx950 (measured: 128 of ~250 bytes per clock),
// while this layout reads at the full rate, and so do the row-wise stores
// that fill it.
template <int D>
__device__ __forceinline__ int k_chunk(int r, int c) {
  return c ^ (r & (D / 8 - 1));
}


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

// LDS of one workgroup.  It holds bf16 whatever the pool's type: FP8 codes
// are widened once, when a step is staged, not by each of the four waves
// that read them.
template <int D>
struct PfLds {
  __align__(16) uint16_t k_s[2][kStep * D];        // K rows, 16-byte chunks swizzled (k_chunk)
  __align__(16) uint16_t v_s[2][kStep * D];        // per 32-key round: [4 quads][D][2 tiles][4 keys]
  int lpt_cost[kLptMaxPairs];
  int lpt_pick;
};

// PREFIX: the shared-prefix pass of cascade decode instead: the rows are
// the decode queries of all sequences, the keys one chunk of the shared
// prefix blocks (no causal mask), and a partial result goes out.
}  // namespace pf
}  // namespace kvp
