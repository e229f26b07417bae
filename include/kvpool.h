/*
 * kvpool.h -- C ABI of the MI355X (gfx950) paged KV-cache library.
 *
 * One hot path: decode attention over a KV cache held in a pool of fixed
 * 16-token (or 32-token) blocks, and the cache write that stores each new
 * token's K and V into its slot.  Sources (page titles as printed):
 *
 *  [Optimizing] "Optimizing KV Cache Memory Management in vLLM with
 *     PagedAttention and Dynamic Block Allocation"
 *       - section "PagedAttention: Virtual Memory for LLMs": logical block
 *         index floor(i / B), offset i mod B, the kernel looks the physical
 *         block up in the sequence's block table and computes the address;
 *       - section "The Block Manager and Dynamic Allocation Lifecycle"
 *         (Prefill / Decode phases): prompt and decode K/V are written into
 *         the physical blocks; decode appends into the last block;
 *       - section "The Math of the KV Cache Bottleneck": GQA/MQA, fewer KV
 *         heads than query heads;
 *       - section "Trade-offs of Block Size Tuning": block size 16 is the
 *         default, 32 is offered for very long contexts.
 *  [Paged] the paged-attention post on zhangchitc.github.io
 *       - section "What a physical block looks like": the pool is split per
 *         layer into num_blocks blocks of [2, block_size, num_kv_heads,
 *         head_dim]; a block id names the same block in every layer.
 *  [Memory] "The memory behind the next token"
 *       - section "Why the next token needs yesterday's state": exact layouts
 *         depend on the attention backend; a sliding window drops the blocks
 *         it no longer needs.
 *  [Pool] "How the block pool manages KV memory"
 *       - section "Hybrid models get groups": a sliding-window layer keeps
 *         only the blocks inside the last window.
 *
 * The pages give no formula for attention itself; the library computes the
 * standard decode attention out_h = softmax(q_h K^T * scale) V for every
 * query head h, with KV head h / G (G = num_q_heads / num_kv_heads).
 *
 * Conventions
 *  - Every device pointer is caller-owned memory (e.g. a torch tensor); the
 *    library allocates no device memory and keeps no pointer past a call,
 *    except the pool handle, which borrows its base pointer.
 *  - All work is enqueued asynchronously on the given hipStream_t (NULL = the
 *    default stream); the calls return after the launch.
 *  - Status codes are int32_t (kvp_status).  Arguments are checked before any
 *    launch; on error nothing is launched and kvp_last_error() returns a
 *    thread-local message.
 *  - Device data are not validated on the fast path, but kernels never
 *    read or write outside the pool, the table row, or the output: a slot or
 *    block id outside [0, num_blocks*block_size) / [0, num_blocks) is
 *    skipped.
 */
#ifndef KVPOOL_H
#define KVPOOL_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVP_OK = 0,
  KVP_ERR_INVALID_ARG = -1,      /* a pointer, size or index is out of range */
  KVP_ERR_UNSUPPORTED = -2,      /* a valid but unimplemented shape or dtype */
  KVP_ERR_WORKSPACE_TOO_SMALL = -3,
  KVP_ERR_HIP = -4               /* the HIP runtime refused a launch */
} kvp_status;

/*
 * Pool element types.  KVP_FP8_E4M3 stores each K/V value as one byte in
 * the E4M3 format (sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, S.1111.111 = NaN, largest magnitude 448); a stored K code c
 * means c * k_scale and a V code c means c * v_scale, one (k_scale,
 * v_scale) per layer (kv_pool_set_fp8_scales).  [Optimizing] "The Math of
 * the KV Cache Bottleneck": FP8 halves the bytes per element of BF16.
 * Queries, outputs and new tokens stay BF16 with an FP8 pool.
 */
typedef enum { KVP_F32 = 0, KVP_BF16 = 1, KVP_FP8_E4M3 = 2 } kvp_dtype;

/* Kernel variant for paged_decode_attention. */
typedef enum {
  KVP_VARIANT_AUTO = 0,   /* bf16/fp8: STREAM (MFMA with partition_tokens > 0
                             or more than 4096 sequences); fp32: VALU         */
  KVP_VARIANT_VALU = 1,   /* vector ALU dot products, partitioned rows
                             (fp32 and bf16 pools)                            */
  KVP_VARIANT_MFMA = 2,   /* matrix cores for QK^T and PV, partitioned rows
                             (bf16 and fp8 pools)                             */
  KVP_VARIANT_STREAM = 3  /* matrix cores, persistent waves that split the
                             batch's blocks evenly (bf16 and fp8 pools, <=
                             4096 sequences)                                  */
} kvp_variant;

/*
 * Pool geometry.  block_size 16 (the pages' default block) or 32 ([Optimizing]
 * "Trade-offs of Block Size Tuning").  head_dim 64 or 128.  dtype a
 * kvp_dtype.  num_blocks * block_size must fit in int32.
 */
typedef struct {
  int32_t num_layers;
  int32_t num_blocks;     /* physical blocks per layer */
  int32_t block_size;     /* 16 or 32 */
  int32_t num_kv_heads;
  int32_t head_dim;       /* 64 or 128 */
  int32_t dtype;          /* kvp_dtype */
} kvp_pool_desc;

typedef struct kvp_pool_s* kvp_pool;  /* opaque, immutable after create */

/*
 * Device layout of the pool (elements of the pool dtype).  For layer l,
 * physical block b, KV head h, slot t (0..B-1, B = block_size) and
 * dimension d:
 *
 *   blk   = (l * num_blocks + b) * 2 * num_kv_heads * B * head_dim
 *   K(t,d) = blk + (              h) * B * head_dim + t * head_dim + d
 *   V(t,d) = blk + (num_kv_heads + h) * B * head_dim
 *                + ((t / 4) * head_dim + d) * 4 + (t % 4)
 *
 * i.e. per block all K tiles, then all V tiles; a (block, head) K tile is
 * one contiguous row-major [B][head_dim] array and a V tile is
 * [B/4][head_dim][4]: for each group of four slots, the four slots' values
 * of one dimension sit next to each other.  This is the pages' block shape
 * [2, block_size, num_kv_heads, head_dim] with heads moved outside slots
 * (one contiguous tile per head) and V's slots interleaved in fours, which
 * the attention backend is free to choose ([Memory], "Why the next token
 * needs yesterday's state").
 */

/* Bytes a pool of this geometry occupies; 0 if the geometry is invalid. */
size_t kv_pool_bytes(const kvp_pool_desc* desc);

/*
 * Create a handle over caller-owned device memory `dev_base` of `bytes`
 * bytes (>= kv_pool_bytes(desc), 256-byte aligned).  The memory is not
 * touched.  The handle borrows dev_base and must not outlive it.
 * Errors: KVP_ERR_INVALID_ARG (null pointers, misalignment, too small),
 * KVP_ERR_UNSUPPORTED (block_size not 16/32, head_dim not 64/128, dtype).
 */
int32_t kv_pool_create(const kvp_pool_desc* desc, void* dev_base, size_t bytes, kvp_pool* out);

/* Release the handle (not the memory).  NULL is accepted. */
int32_t kv_pool_destroy(kvp_pool pool);

/* Copy the geometry of a handle into *desc. */
int32_t kv_pool_describe(kvp_pool pool, kvp_pool_desc* desc);

/*
 * Scales of one layer of an FP8 pool: a K code c stands for c * k_scale, a
 * V code for c * v_scale (both finite and > 0; 1.0 until set).  Writes
 * quantize with them (cache_write, paged_decode_step), attention
 * dequantizes with them; they apply to calls enqueued after this one.
 * Errors: KVP_ERR_INVALID_ARG (layer, non-positive or non-finite scale),
 * KVP_ERR_UNSUPPORTED (the pool is not FP8).
 */
int32_t kv_pool_set_fp8_scales(kvp_pool pool, int32_t layer, float k_scale, float v_scale);

/*
 * Element offset (from dev_base) of K (kv = 0) or V (kv = 1) of
 * (layer, block, head, slot, dim), per the layout above; -1 if any index is
 * out of range.  Host-side helper for loaders and tests.
 */
int64_t kv_pool_offset(kvp_pool pool, int32_t layer, int32_t block, int32_t kv, int32_t head,
                       int32_t slot, int32_t dim);

/*
 * cache_write -- store new tokens' K and V into their slots of one layer.
 *   [Optimizing] "The Block Manager and Dynamic Allocation Lifecycle": in
 *   prefill the kernel writes the prompt's K/V into the allocated blocks; in
 *   decode the new token's K/V go to the free slot of the last block.
 *
 *   k_new, v_new : device, [num_tokens][num_kv_heads][head_dim], pool dtype
 *                  (BF16 for an FP8 pool), contiguous.
 *   slot_mapping : device int32 [num_tokens]; slot = block * B + offset
 *                  ([Optimizing] "PagedAttention": floor(i/B), i mod B).
 *                  A negative slot (padding) writes nothing; a slot
 *                  >= num_blocks*B writes nothing.  Two tokens naming the
 *                  same slot in one call leave that slot undefined.
 *   The copy is bit-exact.  An FP8 pool stores codes instead: each value x
 *   becomes the E4M3 code nearest to x * (1 / scale) (reciprocal and product
 *   in float32, ties to the even code, magnitudes above 448 saturate to
 *   448), with the layer's k_scale / v_scale.  num_tokens == 0 launches
 *   nothing.
 */
int32_t cache_write(kvp_pool pool, int32_t layer, const void* k_new, const void* v_new,
                    const int32_t* slot_mapping, int32_t num_tokens, hipStream_t stream);

/* Arguments of paged_decode_attention (all device pointers caller-owned). */
typedef struct {
  int32_t layer;
  const void* q;                /* [num_seqs][num_q_heads][head_dim], pool dtype
                                   (BF16 for an FP8 pool)                       */
  void* out;                    /* same shape and dtype as q                    */
  const int32_t* block_tables;  /* [num_seqs][max_blocks_per_seq]               */
  int32_t max_blocks_per_seq;   /* row stride of block_tables (>= 1)            */
  const int32_t* seq_lens;      /* [num_seqs], absolute context lengths (>= 0)  */
  int32_t sliding_window;       /* 0 = attend to the whole context              */
  int32_t num_seqs;
  int32_t num_q_heads;          /* multiple of the pool's num_kv_heads          */
  float scale;                  /* softmax scale, e.g. 1/sqrt(head_dim)         */
  int32_t partition_tokens;     /* 0 = auto; else a multiple of 16 <= 1024      */
  int32_t variant;              /* kvp_variant                                  */
  void* workspace;              /* device scratch, may be NULL if not needed    */
  size_t workspace_bytes;
  int32_t shared_prefix_blocks; /* 0, or: the first this-many entries of every
                                   row are the same full blocks (a shared
                                   prompt prefix); see paged_decode_attention */
  int32_t shared_blocks;        /* nonzero: some block past the shared prefix
                                   is listed by more than one row; a hint that
                                   changes no result (see paged_decode_attention) */
} kvp_decode_args;

/*
 * Bytes of workspace paged_decode_attention needs for these sizes (0 when a
 * single pass suffices, i.e. every row fits in one partition).
 */
size_t paged_decode_workspace_bytes(kvp_pool pool, int32_t num_seqs, int32_t num_q_heads,
                                    int32_t max_blocks_per_seq, int32_t partition_tokens);

/*
 * paged_decode_attention -- one decode step of one layer.
 *   [Optimizing] "PagedAttention: Virtual Memory for LLMs": for each
 *   sequence the kernel walks its block table (row s of block_tables,
 *   [Paged] "Two lookup structures": req_to_blocks is the ordered
 *   logical-to-physical list) and reads each key and value where the table
 *   says it lives.
 *
 *   Rows.  With sliding_window == 0, row s lists logical blocks
 *   0 .. (ctx-1)/B and all ctx = seq_lens[s] tokens are attended (B =
 *   block_size).  With a window W > 0 ([Pool] "Hybrid models get groups")
 *   row s lists only the blocks covering positions max(0, ctx-W) .. ctx-1:
 *   logical blocks max(0,ctx-W)/B .. (ctx-1)/B; the first
 *   max(0,ctx-W) % B slots of its first block are not attended.  Entries past the row's length are
 *   never read.  A row with ctx == 0 yields zeros.
 *
 *   out[s][h] = sum_i p_i V_i with p = softmax(K q[s][h] * scale) over the
 *   attended keys of KV head h / G; fp32 accumulation, output rounded to
 *   the query dtype (round to nearest even for bf16).  With an FP8 pool,
 *   K and V are the stored codes times the layer's k_scale and v_scale
 *   (variants STREAM and MFMA).
 *
 *   Long rows are split into partitions of partition_tokens table slots;
 *   each partition leaves its partial result (running max, sum and
 *   unnormalised output) in `workspace` (paged_decode_workspace_bytes()
 *   bytes, contents need no initialisation) and a second kernel on the
 *   same stream merges them.  The STREAM variant splits the batch's tiles
 *   evenly over its waves; the rows cut between waves are merged the same
 *   way, or, when no row crosses an XCD (num_kv_heads a multiple of 8, at
 *   most 16 query heads per KV head, no shared prefix), inside the same
 *   launch by workgroups that start as the streaming ones finish; those
 *   keep per-call marks in the workspace, written and cleared within each
 *   call (left zero; marks of other contents are practically never taken
 *   for a call's own, so no initialisation is needed either).  Calls that
 *   share one workspace must not overlap.
 *
 *   Environment: KVP_LAUNCH_MERGE=0 (read at each call) keeps the separate
 *   merge kernel.
 *
 *   Environment: KVP_DECODE_DEPTH (1..3 for the MFMA variant, 1..2 for
 *   the others) overrides how many blocks each wave keeps in flight ahead
 *   of the one it computes (a tuning knob, read once per process).
 *
 *   Errors: KVP_ERR_INVALID_ARG (nulls, layer, heads, partition size),
 *   KVP_ERR_UNSUPPORTED (variant/dtype/head group combination),
 *   KVP_ERR_WORKSPACE_TOO_SMALL, KVP_ERR_HIP.
 */
int32_t paged_decode_attention(kvp_pool pool, const kvp_decode_args* args, hipStream_t stream);
/*
 *   Shared prefix (cascade).  shared_prefix_blocks = P > 0 promises that the
 *   first P entries of every row are the same physical blocks, all full and
 *   all attended (seq_lens[s] >= B P): a prompt prefix that every sequence
 *   of the batch reuses ([Pool] "Finding a prefix again"; [Memory] "How
 *   vLLM recognizes a reusable prefix": only full blocks are shared).  The
 *   STREAM variant then attends the prefix once per KV head for all
 *   sequences (a dense pass: 128 query rows of any sequences per workgroup
 *   share the prefix's K/V tiles in LDS, and the prefix's keys are split
 *   into up to 8 chunks, each leaving its own partial result), streams only
 *   the private tails, and merges the two; the result is the same
 *   attention up to fp32 rounding.  Both passes run in one launch: when the
 *   prefix pass's workgroups fit in a share of the resident workgroup
 *   slots (a quarter; three eighths for an FP8 pool) they run beside the
 *   tails' streaming workgroups from the start, else after them
 *   (KVP_PREFIX_PIECES=1..8 sets the number of chunks, read at each
 *   call).  Other variants, and
 *   rows with a sliding window, ignore the hint.  P must be <=
 *   max_blocks_per_seq (KVP_ERR_INVALID_ARG otherwise); if the promise does
 *   not hold the outputs are unspecified (memory is still only read inside
 *   the pool and the table rows).
 *
 *   Blocks read by several rows.  By default the STREAM and MFMA variants
 *   read the K/V tiles with non-temporal loads: when every block of the batch is
 *   listed by one row only (the case without sharing, and the private
 *   tails of a cascade), each line is read once and streaming it past the
 *   caches is faster.  Rows may also share blocks outside the prefix
 *   passed as shared_prefix_blocks ([Optimizing] "Copy-on-Write (CoW) for
 *   Parallel Sampling and Prefix Caching": sequences of one prompt list the
 *   same physical blocks until they write to them; the host's reference
 *   counts show it).  shared_blocks != 0 says so: tiles are then read with
 *   ordinary cached loads, and rows that share a block find it in the L2
 *   cache.  The hint changes no output bit, only speed; the VALU variant
 *   always uses cached loads.
 */

/*
 * paged_decode_step -- one decode step of one layer: store each sequence's
 * new token, then attend with it.
 *   [Optimizing] "The Block Manager and Dynamic Allocation Lifecycle" (The
 *   Decode Phase): the new token's K/V go into the next free slot of the
 *   sequence's last block, and decode attention runs over the context that
 *   now includes it.
 *
 *   args         : as for paged_decode_attention; seq_lens[s] counts the
 *                  new token.
 *   k_new, v_new : device, [num_seqs][num_kv_heads][head_dim], pool dtype,
 *                  one token per sequence, 16-byte aligned.
 *   slot_mapping : device int32 [num_seqs]: slot of sequence s's new token,
 *                  which must be the slot of position seq_lens[s]-1 of row s
 *                  (in the row's last block, a block no other sequence
 *                  uses: copy-on-write happens first).  Negative: s has no
 *                  new token (attention only); >= num_blocks*B: nothing
 *                  is written.
 *
 *   Result: the pool and out are bit-identical to cache_write(num_seqs
 *   tokens) followed by paged_decode_attention.  The STREAM variant does
 *   both in one pass (the wave that computes a row's last block takes the
 *   new K/V from registers and stores them to the pool); other variants
 *   launch the write first.  If a slot breaks the rule above, the values
 *   written and the outputs are unspecified, but nothing outside the pool,
 *   the table rows and the outputs is accessed.  Errors as for
 *   paged_decode_attention, plus KVP_ERR_INVALID_ARG for NULL or misaligned
 *   k_new, v_new or slot_mapping.
 */
int32_t paged_decode_step(kvp_pool pool, const kvp_decode_args* args, const void* k_new,
                          const void* v_new, const int32_t* slot_mapping, hipStream_t stream);

/*
 * paged_decode_step_noalloc -- paged_decode_step for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It allocates nothing (no
 * hipMalloc, hipFree or allocating library call): its workspace is a
 * static array of KVP_NOALLOC_SCRATCH_BYTES in the library, one per GPU,
 * held from the first use of the library's code on that GPU to the end of
 * the process.  The caller still passes every input and output.
 *
 *   Arguments, results and errors as for paged_decode_step (same kernels,
 *   bit-identical outputs and pool), except that args->workspace and
 *   args->workspace_bytes are ignored.  A call whose workspace would exceed
 *   KVP_NOALLOC_SCRATCH_BYTES (paged_decode_workspace_bytes() bounds it) is
 *   refused with KVP_ERR_WORKSPACE_TOO_SMALL before anything is launched.
 *   The array needs no clearing: a call writes every byte of it that it
 *   reads.  All calls on one GPU share the array, so calls that overlap
 *   on one GPU (on different streams, or from several threads without an
 *   order between their streams) race and give unspecified results.  The
 *   first call on a GPU looks the array's address up (hipGetSymbolAddress,
 *   with the stream's device current); KVP_ERR_HIP if that fails.
 */
#define KVP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int32_t paged_decode_step_noalloc(kvp_pool pool, const kvp_decode_args* args, const void* k_new,
                                  const void* v_new, const int32_t* slot_mapping, hipStream_t stream);

/*
 * kv_pool_copy_blocks -- the device side of copy-on-write, every layer.
 *   [Optimizing] "Copy-on-Write (CoW) for Parallel Sampling and Prefix
 *   Caching": before a sequence writes into a block it shares, it is given a
 *   new physical block holding a copy of the shared one (the host
 *   bookkeeping allocates it, moves the reference and repoints the table).
 *
 *   src, dst  : device int32 [num_pairs] physical block ids; every layer's
 *               K and V of block src[i] are copied into block dst[i].  A
 *               pair with an id outside [0, num_blocks) or src == dst is
 *               skipped.  No dst may repeat or appear as a src in the same
 *               call (the copies of one call run in no particular order).
 *   Bit-exact.  num_pairs == 0 launches nothing.  Errors:
 *   KVP_ERR_INVALID_ARG (NULL or misaligned ids, num_pairs < 0),
 *   KVP_ERR_HIP.
 */
int32_t kv_pool_copy_blocks(kvp_pool pool, const int32_t* src, const int32_t* dst,
                            int32_t num_pairs, hipStream_t stream);

/*
 * Arguments of one multi-token (prefill / chunked-prefill) attention call.
 */
typedef struct {
  int32_t layer;
  const void* q;                /* device [total_q][num_q_heads][head_dim], BF16,
                                   16-byte aligned; chunk s is rows
                                   cu_q_lens[s] .. cu_q_lens[s+1]-1          */
  void* out;                    /* device, same shape and dtype as q           */
  const int32_t* cu_q_lens;     /* device int32 [num_seqs + 1], cu_q_lens[0] = 0,
                                   nondecreasing, cu_q_lens[num_seqs] = total_q */
  const int32_t* seq_lens;      /* device int32 [num_seqs]: context length after
                                   the chunk (the chunk's tokens included)      */
  const int32_t* block_tables;  /* device int32 [num_seqs][max_blocks_per_seq] */
  int32_t max_blocks_per_seq;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t total_q;              /* rows of q and out                            */
  int32_t max_q_len;            /* >= every chunk length: sizes the launch; rows
                                   of a longer chunk past it are not written    */
  int32_t sliding_window;       /* 0 = full context, else W > 0                 */
  float scale;                  /* softmax scale, usually 1/sqrt(head_dim)     */
} kvp_prefill_args;

/*
 * paged_prefill_attention -- attention of a batch of multi-token chunks
 * (one layer), over keys already in the pool.
 *   [Optimizing] "The Block Manager and Dynamic Allocation Lifecycle" (The
 *   Prefill Phase: a prompt's K/V are computed in one parallel step and
 *   written into its blocks) and "Production Tuning: Ratios, Failure Modes,
 *   and Mitigations" (Failure Mode 2: chunked prefill splits a long prompt
 *   into chunks that are processed step by step).
 *
 *   The chunk of sequence s is its last q_len = cu_q_lens[s+1] - cu_q_lens[s]
 *   positions, ctx - q_len .. ctx - 1 (ctx = seq_lens[s]); their K/V must be
 *   in the pool (cache_write, or paged_prefill_step).  The query at
 *   position p attends the keys at positions lo(p) .. p (causal), with
 *   lo(p) = 0, or max(0, p + 1 - W) under a sliding window W; for q_len = 1
 *   this is decode attention at context p + 1.  Row s of block_tables
 *   lists the blocks covering positions first .. ctx - 1, first =
 *   lo(ctx - q_len) (logical blocks first / B .. (ctx - 1) / B).
 *   out[row][h] = softmax over those keys of (K q * scale) times V, KV head
 *   h / G; fp32 accumulation, BF16 output (round to nearest even).  With
 *   an FP8 pool K and V are the codes times the layer's scales.  A chunk
 *   longer than its context leaves zeros in its rows without a position.
 *
 *   Errors: KVP_ERR_INVALID_ARG (nulls, misalignment, layer, heads, sizes),
 *   KVP_ERR_UNSUPPORTED (fp32 pools), KVP_ERR_HIP.
 */
int32_t paged_prefill_attention(kvp_pool pool, const kvp_prefill_args* args, hipStream_t stream);

/*
 * paged_prefill_step -- store the chunks' K/V, then attend: cache_write of
 * total_q tokens (k_new, v_new [total_q][num_kv_heads][head_dim] BF16, 16-byte
 * aligned; slot_mapping [total_q], the slot of each chunk token's position)
 * followed by paged_prefill_attention on the same stream.  Same results as
 * the two calls.  Errors as for both.
 */
int32_t paged_prefill_step(kvp_pool pool, const kvp_prefill_args* args, const void* k_new, const void* v_new,
                           const int32_t* slot_mapping, hipStream_t stream);

/* Static text of a status code. */
const char* kvp_status_str(int32_t status);

/* Detail of the last error on the calling thread ("" if none). */
const char* kvp_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVPOOL_H */
