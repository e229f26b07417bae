// Internal declarations shared by the kernels and the C-ABI layer of
// libkvpool.  Not part of the public interface (see include/kvpool.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvp {

constexpr int kBlock = 16;      // tokens per tile: the unit every kernel streams.  A pool's
                                // block holds 16 tokens (the pages' default) or 32 (two tiles)
constexpr int kWaves = 4;       // waves per decode workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxStreamSeqs = 4096;  // sequences one streaming launch can take (LDS prefix sums)
constexpr int kMaxPrefixPieces = 8;    // key chunks of the shared-prefix pass
constexpr int kRowSlots = 3;         // cascade: a row's first pieces stored by row (the merge's first loads)

// Geometry and arguments of one decode launch, resolved on the host.
struct DecodeParams {
  const void* pool_layer;       // first element of this layer's blocks
  const void* q;                // [S][Hq][D]
  void* out;                    // [S][Hq][D]
  const int32_t* block_tables;  // [S][max_blocks]
  const int32_t* seq_lens;      // [S]
  float* part_o;                // [S][Hq][num_parts][D]      (split only)
  float* part_ml;               // [S][Hq][num_parts][2]      (split only)
  int32_t max_blocks;           // row stride of block_tables
  int32_t window;               // 0 = full context
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t num_blocks;           // physical blocks per layer (bounds check)
  int32_t bshift;               // log2(block_size / 16): a block (table entry) holds 1 << bshift tiles
  int32_t group;                // query heads per KV head (G)
  int32_t heads_per_wg;         // query heads one workgroup serves (<= 16)
  int32_t qgroups;              // workgroups per KV head = ceil(G / heads_per_wg)
  int32_t part_blocks;          // tiles per partition
  int32_t num_parts;            // partitions of the longest possible row
  float scale_log2;             // scale * log2(e): scores are kept in base 2
  int32_t depth;                // blocks of K/V a wave keeps in flight ahead of the one it computes
  int32_t* prefix;              // [S + 1] tiles before each sequence's row     (streaming only)
  int32_t* cuts;                // [HG][S][2] per row: first piece (wave * 2 + slot), last wave  (streaming only)
  int32_t merge_wgs;            // > 0: the streaming launch merges the cut rows itself, in these
                                // workgroups after the streaming ones (streaming only)
  uint64_t epoch;               // this call's ready mark for the in-launch merge (never 0)
  uint64_t* flags;              // [waves * 2][heads_per_wg] a piece's ready mark, cleared by its merge
  int32_t stream_wgs;           // persistent workgroups of a streaming launch   (streaming only)
  const void* k_new;            // [S][Hkv][D] new token per sequence        (fused write only)
  const void* v_new;            // [S][Hkv][D]                               (fused write only)
  const int32_t* slot_mapping;  // [S]; NULL: attention only                 (fused write only)
  int32_t prefix_blocks;        // table entries every row shares (cascade); 0: none   (streaming only)
  int32_t prefix_pieces;        // key chunks of the prefix pass (cascade only)
  int32_t prefix_chunk;         // tiles per chunk, a multiple of 4 (cascade only)
  float* pre_o;                 // [pieces][S][Hq][D] prefix pass: unnormalised output (cascade only)
  float* pre_ml;                // [pieces][S][Hq][2] prefix pass: (max, sum)          (cascade only)
  float* row_o;                 // [rows][heads_per_wg][kRowSlots][D] a tail's first pieces  (cascade only)
  float* row_ml;                // [rows][heads_per_wg][kRowSlots][2]                      (cascade only)
  int32_t nt_loads;             // tiles read with non-temporal loads (no block read by two rows)  (matrix-core kernels)
  int32_t kv_fp8;               // the pool holds E4M3 codes (K scale folded into scale_log2)
  float v_scale;                // multiplies every output (FP8 V codes); 1 otherwise
  float inv_k_scale;            // 1 / k_scale, 1 / v_scale: quantizing the fused write's new token
  float inv_v_scale;
};

// Geometry and arguments of one prefill (multi-token) launch.
struct PrefillParams {
  const void* pool_layer;       // first element of this layer's blocks
  const void* q;                // [T][Hq][D] bf16
  void* out;                    // [T][Hq][D] bf16
  const int32_t* cu_q_lens;     // [S + 1] chunk offsets into q / out
  const int32_t* seq_lens;      // [S] context after the chunk
  const int32_t* block_tables;  // [S][max_blocks]
  int32_t max_blocks;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t bshift;
  int32_t group;                // G
  int32_t window;
  int32_t qtiles;               // 128-row query tiles per (sequence, KV head) for the longest chunk
  int32_t max_q_len;            // chunk rows past it are not computed
  int32_t total_q;              // rows of q / out (reads and writes stay inside)
  float scale_log2;             // scale * log2(e) (* k_scale for FP8)
  float v_scale;
  // The shared-prefix pass of cascade decode runs on the same kernel: every
  // sequence's decode query against the first prefix_blocks entries of the
  // table's first row, the prefix's tiles split into prefix_pieces chunks
  // of prefix_chunk tiles (a multiple of the 4-tile step), each chunk
  // leaving (max, sum, unnormalised output) per (sequence, query head).
  int32_t prefix_blocks;
  int32_t prefix_pieces;
  int32_t prefix_chunk;
  float* pre_o;                 // [pieces][S][Hq][D]
  float* pre_ml;                // [pieces][S][Hq][2]
};

// Span of one block-table row in 16-token tiles.  The row's first block
// starts at a multiple of the block size; under a sliding window the first
// attended position may lie past its first tile (t0 = 1 in a 32-token
// block) and past slots of the tile it lies in (start_off).  Tile J of the
// span is tile t0 + J of the row: tile (t0 + J) & ((1 << bshift) - 1) of
// the block in entry (t0 + J) >> bshift.  Kernels load entries as stored
// and check them against the pool only when they use them, so that a table
// load never has to complete before the tile loads issued after it.
struct RowSpan {
  int start_off;  // unattended leading slots of the first tile
  int n;          // attended keys
  int nblocks;    // tiles holding them
  int t0;         // tiles of the first block before the first attended one
};

__device__ __forceinline__ RowSpan row_span(int ctx, int window, int max_blocks, int bshift) {
  RowSpan r{0, 0, 0, 0};
  if (ctx <= 0) return r;
  const int B = kBlock << bshift;
  const int first = (window > 0 && ctx > window) ? ctx - window : 0;
  const int off = first & (B - 1);
  r.t0 = off >> 4;
  r.start_off = off & (kBlock - 1);
  r.n = ctx - first;
  if (((unsigned)off + (unsigned)r.n + B - 1) / B > (unsigned)max_blocks)  // row longer than the table:
    r.n = max_blocks * B - off;                                             // attend what the table holds
  r.nblocks = (r.start_off + r.n + kBlock - 1) / kBlock;
  return r;
}


// Launchers (each defined next to its kernel).
hipError_t launch_cache_write(void* pool_layer, int dtype, int num_blocks, int bshift, int num_kv_heads,
                              int head_dim, const void* k_new, const void* v_new,
                              const int32_t* slots, int num_tokens, float inv_k_scale, float inv_v_scale,
                              hipStream_t stream);
hipError_t launch_copy_blocks(void* pool_base, int num_layers, int num_blocks, size_t block_bytes, const int32_t* src,
                              const int32_t* dst, int num_pairs, hipStream_t stream);
hipError_t launch_decode_valu(const DecodeParams& p, int dtype, int head_dim, hipStream_t stream);
hipError_t launch_decode_mfma(const DecodeParams& p, int head_dim, hipStream_t stream);
hipError_t launch_decode_reduce(const DecodeParams& p, int dtype, int head_dim, hipStream_t stream);
hipError_t launch_decode_stream(const DecodeParams& p, int head_dim, hipStream_t stream);
hipError_t launch_prefill(const PrefillParams& p, int head_dim, bool fp8, hipStream_t stream);
// The streaming kernel instance a launch would use (for occupancy queries;
// cascade: the one that also runs the shared-prefix pass); nullptr for one
// that is never launched (the fused step runs at depth 1).
const void* stream_kernel_symbol(int head_dim, int depth, bool fused, bool fp8, int bshift, bool nt, bool cascade);

}  // namespace kvp
