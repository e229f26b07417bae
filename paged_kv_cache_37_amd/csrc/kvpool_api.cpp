// C-ABI of libkvpool: argument checks, geometry, variant and partition
// choice, launches.  Declared in include/kvpool.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include <unistd.h>

#include "internal.h"
#include "kvpool.h"

struct kvp_pool_s {
  kvp_pool_desc desc;
  void* base;
  size_t bytes;
  std::vector<float> k_scale, v_scale;  // per layer (FP8 pools)
};

namespace {

thread_local char g_err[512] = "";

int32_t fail(int32_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int32_t ok() {
  g_err[0] = '\0';
  return KVP_OK;
}

size_t elt_bytes(int32_t dtype) { return dtype == KVP_F32 ? 4 : dtype == KVP_BF16 ? 2 : 1; }

// log2(block_size / 16): the 16-token tiles per block, as a shift.
int32_t bshift_of(const kvp_pool_desc& d) { return d.block_size == 32 ? 1 : 0; }

// Elements of one layer: num_blocks * 2 * Hkv * block_size * D.
size_t layer_elems(const kvp_pool_desc& d) {
  return (size_t)d.num_blocks * 2 * (size_t)d.num_kv_heads * d.block_size * (size_t)d.head_dim;
}

int32_t check_desc(const kvp_pool_desc* d) {
  if (!d) return fail(KVP_ERR_INVALID_ARG, "desc is NULL");
  if (d->num_layers < 1 || d->num_blocks < 1 || d->num_kv_heads < 1)
    return fail(KVP_ERR_INVALID_ARG, "num_layers, num_blocks and num_kv_heads must be >= 1");
  if (d->block_size != 16 && d->block_size != 32)
    return fail(KVP_ERR_UNSUPPORTED, "block_size must be 16 or 32 (got %d)", d->block_size);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(KVP_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", d->head_dim);
  if (d->dtype != KVP_F32 && d->dtype != KVP_BF16 && d->dtype != KVP_FP8_E4M3)
    return fail(KVP_ERR_UNSUPPORTED, "dtype must be F32, BF16 or FP8_E4M3");
  if ((size_t)d->num_blocks * d->block_size > (size_t)INT32_MAX)
    return fail(KVP_ERR_INVALID_ARG, "num_blocks * block_size must fit in int32 slot numbers");
  return KVP_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Partition size in 16-token tiles.
int32_t resolve_part_blocks(int32_t partition_tokens, int32_t num_seqs, int32_t wg_per_seq_head_part,
                            int32_t max_tiles) {
  if (partition_tokens > 0) return partition_tokens / kvp::kBlock;
  // Auto: 512-token partitions; shorter when the grid would not fill the chip.
  int32_t pb = 32;
  const long wgs = (long)num_seqs * wg_per_seq_head_part * ((max_tiles + pb - 1) / pb);
  if (wgs < 2048) pb = 16;
  return pb;
}

}  // namespace

extern "C" {

size_t kv_pool_bytes(const kvp_pool_desc* desc) {
  if (check_desc(desc) != KVP_OK) return 0;
  return (size_t)desc->num_layers * layer_elems(*desc) * elt_bytes(desc->dtype);
}

int32_t kv_pool_create(const kvp_pool_desc* desc, void* dev_base, size_t bytes, kvp_pool* out) {
  if (!out) return fail(KVP_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  const int32_t st = check_desc(desc);
  if (st != KVP_OK) return st;
  if (!dev_base) return fail(KVP_ERR_INVALID_ARG, "dev_base is NULL");
  if (!aligned(dev_base, 256)) return fail(KVP_ERR_INVALID_ARG, "dev_base must be 256-byte aligned");
  const size_t need = kv_pool_bytes(desc);
  if (bytes < need) return fail(KVP_ERR_INVALID_ARG, "pool memory too small: %zu < %zu bytes", bytes, need);
  kvp_pool_s* p = new (std::nothrow) kvp_pool_s{*desc, dev_base, bytes, {}, {}};
  if (!p) return fail(KVP_ERR_INVALID_ARG, "out of host memory");
  p->k_scale.assign(desc->num_layers, 1.0f);
  p->v_scale.assign(desc->num_layers, 1.0f);
  *out = p;
  return ok();
}

int32_t kv_pool_destroy(kvp_pool pool) {
  delete pool;
  return ok();
}

int32_t kv_pool_describe(kvp_pool pool, kvp_pool_desc* desc) {
  if (!pool || !desc) return fail(KVP_ERR_INVALID_ARG, "NULL argument");
  *desc = pool->desc;
  return ok();
}

int32_t kv_pool_set_fp8_scales(kvp_pool pool, int32_t layer, float k_scale, float v_scale) {
  if (!pool) return fail(KVP_ERR_INVALID_ARG, "pool is NULL");
  if (pool->desc.dtype != KVP_FP8_E4M3) return fail(KVP_ERR_UNSUPPORTED, "the pool is not FP8");
  if (layer < 0 || layer >= pool->desc.num_layers) return fail(KVP_ERR_INVALID_ARG, "layer %d out of range", layer);
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(KVP_ERR_INVALID_ARG, "scales must be finite and > 0");
  pool->k_scale[layer] = k_scale;
  pool->v_scale[layer] = v_scale;
  return ok();
}

int64_t kv_pool_offset(kvp_pool pool, int32_t layer, int32_t block, int32_t kv, int32_t head, int32_t slot,
                       int32_t dim) {
  if (!pool) return -1;
  const kvp_pool_desc& d = pool->desc;
  if (layer < 0 || layer >= d.num_layers || block < 0 || block >= d.num_blocks || kv < 0 || kv > 1 || head < 0 ||
      head >= d.num_kv_heads || slot < 0 || slot >= d.block_size || dim < 0 || dim >= d.head_dim)
    return -1;
  const int64_t tile = (int64_t)d.block_size * d.head_dim;
  const int64_t blk = ((int64_t)layer * d.num_blocks + block) * 2 * d.num_kv_heads * tile;
  if (kv == 0) return blk + (int64_t)head * tile + (int64_t)slot * d.head_dim + dim;
  return blk + (int64_t)(d.num_kv_heads + head) * tile + ((int64_t)(slot / 4) * d.head_dim + dim) * 4 + slot % 4;
}

int32_t cache_write(kvp_pool pool, int32_t layer, const void* k_new, const void* v_new,
                    const int32_t* slot_mapping, int32_t num_tokens, hipStream_t stream) {
  if (!pool) return fail(KVP_ERR_INVALID_ARG, "pool is NULL");
  const kvp_pool_desc& d = pool->desc;
  if (layer < 0 || layer >= d.num_layers) return fail(KVP_ERR_INVALID_ARG, "layer %d out of range", layer);
  if (num_tokens < 0) return fail(KVP_ERR_INVALID_ARG, "num_tokens < 0");
  if (num_tokens == 0) return ok();
  if (!k_new || !v_new || !slot_mapping) return fail(KVP_ERR_INVALID_ARG, "NULL k_new, v_new or slot_mapping");
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(slot_mapping, 4))
    return fail(KVP_ERR_INVALID_ARG, "k_new/v_new must be 16-byte aligned");
  char* base = (char*)pool->base + (size_t)layer * layer_elems(d) * elt_bytes(d.dtype);
  const hipError_t e = kvp::launch_cache_write(base, d.dtype, d.num_blocks, bshift_of(d), d.num_kv_heads, d.head_dim, k_new,
                                               v_new, slot_mapping, num_tokens, 1.0f / pool->k_scale[layer],
                                               1.0f / pool->v_scale[layer], stream);
  if (e != hipSuccess) return fail(KVP_ERR_HIP, "cache_write launch: %s", hipGetErrorString(e));
  return ok();
}

// Resident workgroups of the streaming kernel on the current device:
// compute units x workgroups per compute unit at the kernel's occupancy
// (cascade: the kernel that also runs the shared-prefix pass).  0 if there
// is no device to ask.
static int32_t stream_workgroups(int32_t head_dim, int32_t depth, bool fused, bool fp8, int32_t bshift,
                                 bool cascade = false) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  static thread_local int cached_dev = -1, cached_d = 0, cached_depth = 0, cached_wgs = 0, cached_bs = 0;
  static thread_local bool cached_fused = false, cached_fp8 = false, cached_cascade = false;
  if (dev == cached_dev && head_dim == cached_d && depth == cached_depth && fused == cached_fused &&
      fp8 == cached_fp8 && bshift == cached_bs && cascade == cached_cascade)
    return cached_wgs;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 0;
  // the cached-load and non-temporal instances launch the same grid (the
  // smaller of their occupancies), so one workspace size serves both
  per_cu = 1 << 30;
  for (bool nt : {true, false}) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, kvp::stream_kernel_symbol(head_dim, depth, fused, fp8, bshift, nt, cascade), kvp::kThreads, 0) !=
            hipSuccess ||
        n <= 0)
      return 0;
    per_cu = std::min(per_cu, n);
  }
  cached_dev = dev;
  cached_d = head_dim;
  cached_depth = depth;
  cached_fused = fused;
  cached_fp8 = fp8;
  cached_bs = bshift;
  cached_cascade = cascade;
  cached_wgs = cus * per_cu;
  return cached_wgs;
}

// The streaming kernel keeps its tile counts in 32-bit prefix sums and its
// split (tile * waves / tiles) exact in double arithmetic: both hold when
// these bounds do.
static bool stream_fits(int32_t num_seqs, int32_t max_tiles, int32_t head_groups, int32_t wgs) {
  const double entries = (double)num_seqs * max_tiles;
  const double waves = (double)wgs * kvp::kWaves;
  return num_seqs <= kvp::kMaxStreamSeqs && entries < 2147483647.0 &&
         entries * head_groups * (waves + 1.0) < 4503599627370496.0;  // 2^52
}

enum { PATH_VALU = 0, PATH_MFMA = 1, PATH_STREAM = 2 };

// Blocks of K/V each wave keeps in flight ahead of the one it computes:
// KVP_DECODE_DEPTH if set and valid for the path, else the measured best
// (the streaming kernel keeps every wave busy across rows, so one suffices).
static int32_t decode_depth(int32_t path, bool fp8) {
  static const int env = [] {
    const char* e = getenv("KVP_DECODE_DEPTH");
    return e ? atoi(e) : 0;
  }();
  const int max_depth = path == PATH_MFMA ? 3 : 2;
  if (env >= 1 && env <= max_depth) return env;
  (void)fp8;  // FP8 tiles carry half the bytes, yet a second one in flight measured no faster
  return path == PATH_MFMA ? 2 : 1;
}

static int32_t plan(kvp_pool pool, int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks, int32_t partition_tokens,
                    int32_t variant, kvp::DecodeParams* p, int32_t* path) {
  const kvp_pool_desc& d = pool->desc;
  if (num_seqs < 0 || num_seqs > 65535) return fail(KVP_ERR_INVALID_ARG, "num_seqs must be in [0, 65535]");
  if (num_q_heads < 1 || num_q_heads % d.num_kv_heads != 0)
    return fail(KVP_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                num_q_heads, d.num_kv_heads);
  if (max_blocks < 1) return fail(KVP_ERR_INVALID_ARG, "max_blocks_per_seq must be >= 1");
  if ((int64_t)max_blocks * d.block_size > INT32_MAX)
    return fail(KVP_ERR_INVALID_ARG, "max_blocks_per_seq * block_size must fit in int32");
  const int32_t bs = bshift_of(d);
  const int32_t max_tiles = max_blocks << bs;  // 16-token tiles a row can hold
  if (partition_tokens != 0 &&
      (partition_tokens % kvp::kBlock != 0 || partition_tokens < kvp::kBlock || partition_tokens > 64 * kvp::kBlock))
    return fail(KVP_ERR_INVALID_ARG, "partition_tokens must be 0 or a multiple of 16 in [16, 1024]");
  const int32_t G = num_q_heads / d.num_kv_heads;
  const bool bf16 = d.dtype != KVP_F32;  // bf16 or fp8 storage: the matrix-core kernels
  const bool fp8 = d.dtype == KVP_FP8_E4M3;
  const int32_t mfma_groups = d.num_kv_heads * ((G + 15) / 16);  // head groups of the MFMA kernels
  int32_t pth;
  switch (variant) {
    case KVP_VARIANT_AUTO:
      if (!bf16) {
        pth = PATH_VALU;
      } else {
        const int32_t wgs =
            partition_tokens == 0 ? stream_workgroups(d.head_dim, decode_depth(PATH_STREAM, fp8), false, fp8, bs) : 0;
        pth = wgs > 0 && stream_fits(num_seqs, max_tiles, mfma_groups, wgs) ? PATH_STREAM : PATH_MFMA;
      }
      break;
    case KVP_VARIANT_VALU:
      if (d.dtype == KVP_FP8_E4M3) return fail(KVP_ERR_UNSUPPORTED, "the VALU variant takes fp32 and bf16 pools");
      pth = PATH_VALU;
      break;
    case KVP_VARIANT_MFMA:
      if (!bf16) return fail(KVP_ERR_UNSUPPORTED, "the MFMA variant needs a bf16 or fp8 pool");
      pth = PATH_MFMA;
      break;
    case KVP_VARIANT_STREAM:
      if (!bf16) return fail(KVP_ERR_UNSUPPORTED, "the STREAM variant needs a bf16 or fp8 pool");
      if (num_seqs > kvp::kMaxStreamSeqs)
        return fail(KVP_ERR_UNSUPPORTED, "the STREAM variant takes at most %d sequences", kvp::kMaxStreamSeqs);
      pth = PATH_STREAM;
      break;
    default: return fail(KVP_ERR_INVALID_ARG, "unknown variant %d", variant);
  }
  int32_t hpw;
  if (pth != PATH_VALU) {
    hpw = G < 16 ? G : 16;
  } else {
    // fp32 at head_dim 128 holds 8 heads' accumulators only by spilling
    const int32_t cap = d.dtype == KVP_F32 && d.head_dim == 128 ? 4 : 8;
    hpw = 1;
    while (hpw < G && hpw < cap) hpw *= 2;
  }
  const int32_t qgroups = (G + hpw - 1) / hpw;
  if ((long)d.num_kv_heads * qgroups > 65535) return fail(KVP_ERR_UNSUPPORTED, "too many head groups");
  // the partition size depends on the row geometry only, never on the variant,
  // so paged_decode_workspace_bytes() is valid for every variant
  const int32_t pb = resolve_part_blocks(partition_tokens, num_seqs, d.num_kv_heads, max_tiles);
  std::memset(p, 0, sizeof(*p));
  p->max_blocks = max_blocks;
  p->num_seqs = num_seqs;
  p->num_q_heads = num_q_heads;
  p->num_kv_heads = d.num_kv_heads;
  p->num_blocks = d.num_blocks;
  p->group = G;
  p->heads_per_wg = hpw;
  p->qgroups = qgroups;
  p->part_blocks = pb;
  p->num_parts = (max_tiles + pb - 1) / pb;
  p->bshift = bs;
  p->depth = decode_depth(pth, fp8);
  if (pth == PATH_STREAM) {
    p->stream_wgs = stream_workgroups(d.head_dim, p->depth, false, fp8, bs);
    if (p->stream_wgs <= 0) return fail(KVP_ERR_HIP, "cannot size the streaming grid (no device?)");
    if (!stream_fits(num_seqs, max_tiles, d.num_kv_heads * qgroups, p->stream_wgs))
      return fail(KVP_ERR_UNSUPPORTED, "num_seqs * max_blocks_per_seq too large for the STREAM variant");
  }
  *path = pth;
  return KVP_OK;
}

static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Workspace of the partitioned kernels: unnormalised partial outputs and
// their (max, sum) pairs per (sequence, query head, partition).
static size_t grid_workspace(const kvp::DecodeParams& p, int32_t head_dim, size_t* o_off, size_t* ml_off) {
  if (p.num_parts <= 1) {
    *o_off = *ml_off = 0;
    return 0;
  }
  const size_t rows = (size_t)p.num_seqs * p.num_q_heads * p.num_parts;
  *o_off = 0;
  *ml_off = align256(rows * head_dim * sizeof(float));
  return *ml_off + rows * 2 * sizeof(float);
}

// Workspace of the streaming kernel: prefix sums, the rows' piece ranges
// (first piece, last wave), the in-launch merge's ready marks (one per
// partial slot and head: zero outside a call), then
// two partial slots per wave for up to heads_per_wg heads ((max, sum) pairs
// and outputs), then, for a call with a shared prefix (cascade), the
// prefix pass's pieces: one per (key chunk, sequence, query head), and one
// per (row, head) for tails a single wave holds.
struct StreamLayout {
  size_t prefix, cuts, flags, ml, o, pre_ml, pre_o, row_ml, row_o, total;
};

// The cascade's one launch: its streaming grid and the key chunks of its
// shared-prefix pass, for `resident` workgroup slots.  The prefix pass has
// units = KV heads x 128-row tiles workgroups per chunk.  When whole chunks
// of units fit in the prefix pass's share of the slots (a quarter for bf16
// pools, three eighths for FP8 ones, whose tails stream half the bytes), the
// chunks take that share and the streaming grid the slots left, so the
// memory-bound tails and the matrix-bound prefix pass run side by side from
// the start (and the merge reads fewer pieces); else the streaming grid
// takes every slot and the prefix pass gets about as many workgroups,
// started on the slots the streaming workgroups free.  At most
// kMaxPrefixPieces chunks; KVP_PREFIX_PIECES (1..8, read at each call)
// overrides the count.  Returns the chunks wanted (those actually used can
// be fewer: a chunk is whole 4-tile steps).
static int32_t cascade_grid(kvp::DecodeParams& p, int32_t resident, bool fp8) {
  const long long units = (long long)p.num_kv_heads * ((p.num_seqs * p.group + 127) / 128);
  const long long share = (long long)resident * (fp8 ? 3 : 2) / 8;
  long long want;
  const long long split = units > 0 ? share / units : 0;
  const long long left = (resident - split * units) / 8 * 8;  // a multiple of 8 (the streaming grid's XCD order)
  if (split >= 1 && left >= 8) {
    p.stream_wgs = (int32_t)left;
    want = split;
  } else {
    p.stream_wgs = resident;
    want = units > 0 ? (resident + units - 1) / units : 1;
  }
  const char* ev = getenv("KVP_PREFIX_PIECES");
  if (ev && atoi(ev) >= 1) want = atoi(ev);
  return (int32_t)std::max(1LL, std::min<long long>(want, kvp::kMaxPrefixPieces));
}

// pieces: the cascade's prefix chunks (cascade_grid), else unused.
static StreamLayout stream_workspace(const kvp::DecodeParams& p, int32_t head_dim, bool cascade, int32_t pieces = 0) {
  StreamLayout L;
  const size_t slots = (size_t)p.stream_wgs * kvp::kWaves * 2 * p.heads_per_wg;
  const size_t qh = (size_t)p.num_seqs * p.num_q_heads;
  const size_t rows = (size_t)p.num_kv_heads * p.qgroups * p.num_seqs * p.heads_per_wg;
  L.prefix = 0;
  L.cuts = L.prefix + align256((size_t)(p.num_seqs + 1) * sizeof(int32_t));
  L.flags = L.cuts + align256((size_t)p.num_kv_heads * p.qgroups * p.num_seqs * 2 * sizeof(int32_t));
  L.ml = L.flags + align256(slots * sizeof(uint64_t));
  L.o = L.ml + align256(slots * 2 * sizeof(float));
  if (!cascade) {
    L.pre_ml = L.pre_o = L.row_ml = L.row_o = 0;
    L.total = L.o + slots * head_dim * sizeof(float);
    return L;
  }
  L.pre_ml = L.o + align256(slots * head_dim * sizeof(float));
  L.pre_o = L.pre_ml + align256((size_t)pieces * qh * 2 * sizeof(float));
  L.row_ml = L.pre_o + align256((size_t)pieces * qh * head_dim * sizeof(float));
  // a row's first kvp::kRowSlots tail pieces, by row
  L.row_o = L.row_ml + align256(rows * kvp::kRowSlots * 2 * sizeof(float));
  L.total = L.row_o + rows * kvp::kRowSlots * head_dim * sizeof(float);
  return L;
}

size_t paged_decode_workspace_bytes(kvp_pool pool, int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                    int32_t partition_tokens) {
  if (!pool) return 0;
  // enough for every variant that could run with these sizes
  size_t need = 0, a;
  for (int32_t v : {KVP_VARIANT_VALU, KVP_VARIANT_MFMA, KVP_VARIANT_STREAM}) {
    kvp::DecodeParams p;
    int32_t path;
    if (plan(pool, num_seqs, num_q_heads, max_blocks_per_seq, partition_tokens, v, &p, &path) != KVP_OK) continue;
    size_t n = path == PATH_STREAM ? stream_workspace(p, pool->desc.head_dim, false).total
                                   : grid_workspace(p, pool->desc.head_dim, &a, &a);
    if (path == PATH_STREAM) {  // the grids of the fused step and of the cascade (their own occupancies) must fit too
      const bool fp8 = pool->desc.dtype == KVP_FP8_E4M3;
      for (int fused = 0; fused < 2; ++fused)
        for (int cascade = 0; cascade < 2; ++cascade) {
          p.stream_wgs = stream_workgroups(pool->desc.head_dim, fused ? 1 : p.depth, fused != 0, fp8, p.bshift,
                                           cascade != 0);
          const int32_t pieces = cascade ? cascade_grid(p, p.stream_wgs, fp8) : 0;
          const size_t nf = stream_workspace(p, pool->desc.head_dim, cascade != 0, pieces).total;
          if (nf > n) n = nf;
        }
    }
    if (n > need) need = n;
  }
  g_err[0] = '\0';
  return need;
}

// Marks of successive calls: splitmix64 of a process-wide counter (nonzero)
// that starts from the clock and the process id, so that a mark left by
// another call or another process is practically never this call's.
static uint64_t next_epoch() {
  static std::atomic<uint64_t> counter{(uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() *
                                           0x2545f4914f6cdd1dull ^
                                       ((uint64_t)getpid() << 32)};
  uint64_t z = counter.fetch_add(0x9e3779b97f4a7c15ull) + 0x9e3779b97f4a7c15ull;
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  z ^= z >> 31;
  return z ? z : 1;
}

// Decode attention, optionally preceded by each sequence's new-token write
// (slots != NULL): fused into the streaming kernel, else a cache_write launch
// first.  scratch: the workspace is the library's own array (too small a
// call is then refused with a message naming its limit).
static int32_t decode(kvp_pool pool, const kvp_decode_args* a, const void* k_new, const void* v_new,
                      const int32_t* slots, hipStream_t stream, bool scratch = false) {
  if (!pool || !a) return fail(KVP_ERR_INVALID_ARG, "NULL pool or args");
  const kvp_pool_desc& d = pool->desc;
  if (a->layer < 0 || a->layer >= d.num_layers) return fail(KVP_ERR_INVALID_ARG, "layer %d out of range", a->layer);
  if (a->sliding_window < 0) return fail(KVP_ERR_INVALID_ARG, "sliding_window < 0");
  if (!std::isfinite(a->scale)) return fail(KVP_ERR_INVALID_ARG, "scale is not finite");
  kvp::DecodeParams p;
  int32_t path = PATH_VALU;
  int32_t st = plan(pool, a->num_seqs, a->num_q_heads, a->max_blocks_per_seq, a->partition_tokens, a->variant, &p, &path);
  if (st != KVP_OK) return st;
  if (a->num_seqs == 0) return ok();
  if (!a->q || !a->out || !a->block_tables || !a->seq_lens)
    return fail(KVP_ERR_INVALID_ARG, "NULL q, out, block_tables or seq_lens");
  if (!aligned(a->q, 16) || !aligned(a->out, 16) || !aligned(a->block_tables, 4) || !aligned(a->seq_lens, 4))
    return fail(KVP_ERR_INVALID_ARG, "q/out must be 16-byte aligned, tables and lengths 4-byte aligned");
  const bool write = slots != nullptr || k_new != nullptr || v_new != nullptr;
  if (write) {
    if (!k_new || !v_new || !slots) return fail(KVP_ERR_INVALID_ARG, "NULL k_new, v_new or slot_mapping");
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(slots, 4))
      return fail(KVP_ERR_INVALID_ARG, "k_new/v_new must be 16-byte aligned, slot_mapping 4-byte aligned");
  }
  if (write && path == PATH_STREAM) {
    // the fused kernel holds the new token in registers: ring depth 1
    const bool fp8 = d.dtype == KVP_FP8_E4M3;
    p.depth = 1;
    p.stream_wgs = stream_workgroups(d.head_dim, 1, true, fp8, p.bshift);
    if (p.stream_wgs <= 0) return fail(KVP_ERR_HIP, "cannot size the streaming grid (no device?)");
    p.k_new = k_new;
    p.v_new = v_new;
    p.slot_mapping = slots;
  }
  int32_t want_pieces = 0;  // the cascade's prefix chunks (workspace layout)
  if (a->shared_prefix_blocks < 0 || a->shared_prefix_blocks > a->max_blocks_per_seq)
    return fail(KVP_ERR_INVALID_ARG, "shared_prefix_blocks must be in [0, max_blocks_per_seq]");
  // the shared-prefix pass is a STREAM feature for full-context rows; elsewhere the hint is ignored
  if (path == PATH_STREAM && a->sliding_window == 0) p.prefix_blocks = a->shared_prefix_blocks;
  if (p.prefix_blocks > 0) {
    // one launch runs the tails and the prefix pass: the slots of that kernel
    const int32_t resident = stream_workgroups(d.head_dim, p.depth, p.slot_mapping != nullptr,
                                               d.dtype == KVP_FP8_E4M3, p.bshift, true);
    if (resident <= 0) return fail(KVP_ERR_HIP, "cannot size the streaming grid (no device?)");
    // split the prefix's keys into chunks of whole 4-tile steps (the
    // workspace holds as many pieces as cascade_grid wants)
    const int32_t tiles = p.prefix_blocks << p.bshift;
    want_pieces = cascade_grid(p, resident, d.dtype == KVP_FP8_E4M3);
    const int32_t want = want_pieces;
    const int32_t per = (tiles + want - 1) / want;
    p.prefix_chunk = (per + 3) / 4 * 4;
    p.prefix_pieces = (tiles + p.prefix_chunk - 1) / p.prefix_chunk;
  }
  // The streaming launch merges the cut rows itself when no row crosses an
  // XCD (KV heads split evenly over the 8 XCDs, one head group each, the
  // grid a multiple of 8 workgroups); KVP_LAUNCH_MERGE=0 (read at each
  // call) keeps the separate merge kernel.
  if (path == PATH_STREAM && p.prefix_blocks == 0 && p.qgroups == 1 && d.num_kv_heads % 8 == 0 &&
      p.stream_wgs % 8 == 0) {
    const char* ev = getenv("KVP_LAUNCH_MERGE");
    if (!(ev && atoi(ev) == 0)) {
      const long long wps = (a->num_q_heads / 8 + 3) / 4;
      const long long mw = 8LL * a->num_seqs * wps;
      if (mw + p.stream_wgs <= 0x7fffffffLL) p.merge_wgs = (int32_t)mw;
    }
  }
  if (p.merge_wgs > 0) p.epoch = next_epoch();
  size_t o_off = 0, ml_off = 0;
  const StreamLayout SL =
      path == PATH_STREAM ? stream_workspace(p, d.head_dim, p.prefix_blocks > 0, want_pieces) : StreamLayout{};
  const size_t ws = path == PATH_STREAM ? SL.total : grid_workspace(p, d.head_dim, &o_off, &ml_off);
  if (path == PATH_STREAM && ws / sizeof(float) >= 0xffffffffull)  // the merge kernel's 32-bit element offsets
    return fail(KVP_ERR_UNSUPPORTED, "the STREAM variant's workspace would exceed 2^32 floats");
  if (ws > 0) {
    if (scratch && a->workspace_bytes < ws)
      return fail(KVP_ERR_WORKSPACE_TOO_SMALL,
                  "this call needs %zu bytes of scratch; the no-allocation entry point holds %zu", ws,
                  a->workspace_bytes);
    if (!a->workspace || a->workspace_bytes < ws)
      return fail(KVP_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes needed (%zu given)", ws,
                  a->workspace ? a->workspace_bytes : (size_t)0);
    if (!aligned(a->workspace, 256)) return fail(KVP_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    char* w = (char*)a->workspace;
    if (path == PATH_STREAM) {
      p.prefix = (int32_t*)(w + SL.prefix);
      p.cuts = (int32_t*)(w + SL.cuts);
      p.flags = (uint64_t*)(w + SL.flags);
      p.part_ml = (float*)(w + SL.ml);
      p.part_o = (float*)(w + SL.o);
      p.pre_ml = (float*)(w + SL.pre_ml);
      p.pre_o = (float*)(w + SL.pre_o);
      p.row_ml = (float*)(w + SL.row_ml);
      p.row_o = (float*)(w + SL.row_o);
    } else {
      p.part_o = (float*)(w + o_off);
      p.part_ml = (float*)(w + ml_off);
    }
  }
  p.pool_layer = (const char*)pool->base + (size_t)a->layer * layer_elems(d) * elt_bytes(d.dtype);
  p.q = a->q;
  p.out = a->out;
  p.block_tables = a->block_tables;
  p.seq_lens = a->seq_lens;
  p.window = a->sliding_window;
  p.nt_loads = path != PATH_VALU && a->shared_blocks == 0;
  // FP8 codes: K's scale joins the softmax scale, V's the final normalisation
  const bool fp8 = d.dtype == KVP_FP8_E4M3;
  p.kv_fp8 = fp8;
  p.scale_log2 = a->scale * 1.4426950408889634f * (fp8 ? pool->k_scale[a->layer] : 1.0f);
  p.v_scale = fp8 ? pool->v_scale[a->layer] : 1.0f;
  p.inv_k_scale = 1.0f / pool->k_scale[a->layer];
  p.inv_v_scale = 1.0f / pool->v_scale[a->layer];
  hipError_t e;
  if (write && path != PATH_STREAM) {
    e = kvp::launch_cache_write(const_cast<void*>(p.pool_layer), d.dtype, d.num_blocks, p.bshift, d.num_kv_heads, d.head_dim,
                                k_new, v_new, slots, a->num_seqs, p.inv_k_scale, p.inv_v_scale, stream);
    if (e != hipSuccess) return fail(KVP_ERR_HIP, "cache_write launch: %s", hipGetErrorString(e));
  }
  if (path == PATH_STREAM) {
    e = kvp::launch_decode_stream(p, d.head_dim, stream);
    if (e != hipSuccess) return fail(KVP_ERR_HIP, "stream decode launch: %s", hipGetErrorString(e));
    return ok();
  }
  e = path == PATH_MFMA ? kvp::launch_decode_mfma(p, d.head_dim, stream)
                        : kvp::launch_decode_valu(p, d.dtype, d.head_dim, stream);
  if (e != hipSuccess) return fail(KVP_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  if (p.num_parts > 1) {
    e = kvp::launch_decode_reduce(p, d.dtype, d.head_dim, stream);
    if (e != hipSuccess) return fail(KVP_ERR_HIP, "reduce launch: %s", hipGetErrorString(e));
  }
  return ok();
}

int32_t paged_decode_attention(kvp_pool pool, const kvp_decode_args* a, hipStream_t stream) {
  return decode(pool, a, nullptr, nullptr, nullptr, stream);
}

int32_t paged_decode_step(kvp_pool pool, const kvp_decode_args* a, const void* k_new, const void* v_new,
                          const int32_t* slot_mapping, hipStream_t stream) {
  if (!k_new || !v_new || !slot_mapping) return fail(KVP_ERR_INVALID_ARG, "NULL k_new, v_new or slot_mapping");
  return decode(pool, a, k_new, v_new, slot_mapping, stream);
}

}  // extern "C"

// ---- the decode step for callers that cannot allocate ----
//
// Its workspace is this array: one copy per GPU, resident from the load of
// the library's code on that GPU to the end of the process.  Host code
// never passes the array's name to a kernel (on the host it stands for a
// host-side symbol, not a device address); it asks the runtime for the
// array's address on each device once and passes that.
static __device__ __align__(256) unsigned char scratch[KVP_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device `stream` runs on, looked up
// the first time with that device current.
int32_t scratch_for(hipStream_t stream, void** out) {
  int dev = -1, cur = -1;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return fail(KVP_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(KVP_ERR_UNSUPPORTED, "device %d past the library's table", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return fail(KVP_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(KVP_ERR_HIP, "hipSetDevice(%d): %s", dev, hipGetErrorString(e));
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess || !ptr)
      return fail(KVP_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    if (back != hipSuccess) return fail(KVP_ERR_HIP, "hipSetDevice(%d): %s", cur, hipGetErrorString(back));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KVP_OK;
}

}  // namespace

extern "C" {

int32_t paged_decode_step_noalloc(kvp_pool pool, const kvp_decode_args* a, const void* k_new, const void* v_new,
                                  const int32_t* slot_mapping, hipStream_t stream) {
  if (!pool || !a) return fail(KVP_ERR_INVALID_ARG, "NULL pool or args");
  if (!k_new || !v_new || !slot_mapping) return fail(KVP_ERR_INVALID_ARG, "NULL k_new, v_new or slot_mapping");
  void* ws = nullptr;
  const int32_t st = scratch_for(stream, &ws);
  if (st != KVP_OK) return st;
  kvp_decode_args b = *a;  // the caller's workspace fields are ignored
  b.workspace = ws;
  b.workspace_bytes = KVP_NOALLOC_SCRATCH_BYTES;
  return decode(pool, &b, k_new, v_new, slot_mapping, stream, true);
}

}  // extern "C"

// Checks of a prefill call and its launch parameters; *launch is false when
// there is nothing to do.
static int32_t plan_prefill(kvp_pool pool, const kvp_prefill_args* a, kvp::PrefillParams* p, bool* launch) {
  *launch = false;
  if (!pool || !a) return fail(KVP_ERR_INVALID_ARG, "NULL pool or args");
  const kvp_pool_desc& d = pool->desc;
  if (a->layer < 0 || a->layer >= d.num_layers) return fail(KVP_ERR_INVALID_ARG, "layer %d out of range", a->layer);
  if (d.dtype == KVP_F32) return fail(KVP_ERR_UNSUPPORTED, "prefill attention takes bf16 and fp8 pools");
  if (a->num_seqs < 0 || a->total_q < 0 || a->max_q_len < 0)
    return fail(KVP_ERR_INVALID_ARG, "num_seqs, total_q and max_q_len must be >= 0");
  if (a->num_q_heads < 1 || a->num_q_heads % d.num_kv_heads != 0)
    return fail(KVP_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                a->num_q_heads, d.num_kv_heads);
  if (a->max_blocks_per_seq < 1) return fail(KVP_ERR_INVALID_ARG, "max_blocks_per_seq must be >= 1");
  if ((int64_t)a->max_blocks_per_seq * d.block_size > INT32_MAX)
    return fail(KVP_ERR_INVALID_ARG, "max_blocks_per_seq * block_size must fit in int32");
  if (a->sliding_window < 0) return fail(KVP_ERR_INVALID_ARG, "sliding_window < 0");
  if (!std::isfinite(a->scale)) return fail(KVP_ERR_INVALID_ARG, "scale is not finite");
  if (a->num_seqs == 0 || a->total_q == 0 || a->max_q_len == 0) return ok();
  if (!a->q || !a->out || !a->cu_q_lens || !a->seq_lens || !a->block_tables)
    return fail(KVP_ERR_INVALID_ARG, "NULL q, out, cu_q_lens, seq_lens or block_tables");
  if (!aligned(a->q, 16) || !aligned(a->out, 16) || !aligned(a->cu_q_lens, 4) || !aligned(a->seq_lens, 4) ||
      !aligned(a->block_tables, 4))
    return fail(KVP_ERR_INVALID_ARG, "q/out must be 16-byte aligned, index arrays 4-byte aligned");
  const int32_t G = a->num_q_heads / d.num_kv_heads;
  const int64_t qtiles = ((int64_t)a->max_q_len * G + 127) / 128;
  if ((int64_t)a->num_seqs * d.num_kv_heads * qtiles > INT32_MAX || (int64_t)a->max_q_len * G > INT32_MAX)
    return fail(KVP_ERR_UNSUPPORTED, "too many query rows for one launch");
  const bool fp8 = d.dtype == KVP_FP8_E4M3;
  std::memset(p, 0, sizeof(*p));
  p->pool_layer = (const char*)pool->base + (size_t)a->layer * layer_elems(d) * elt_bytes(d.dtype);
  p->q = a->q;
  p->out = a->out;
  p->cu_q_lens = a->cu_q_lens;
  p->seq_lens = a->seq_lens;
  p->block_tables = a->block_tables;
  p->max_blocks = a->max_blocks_per_seq;
  p->num_seqs = a->num_seqs;
  p->num_q_heads = a->num_q_heads;
  p->num_kv_heads = d.num_kv_heads;
  p->num_blocks = d.num_blocks;
  p->bshift = bshift_of(d);
  p->group = G;
  p->window = a->sliding_window;
  p->qtiles = (int32_t)qtiles;
  p->max_q_len = a->max_q_len;
  p->total_q = a->total_q;
  p->scale_log2 = a->scale * 1.4426950408889634f * (fp8 ? pool->k_scale[a->layer] : 1.0f);
  p->v_scale = fp8 ? pool->v_scale[a->layer] : 1.0f;
  *launch = true;
  return KVP_OK;
}

extern "C" {

int32_t paged_prefill_attention(kvp_pool pool, const kvp_prefill_args* a, hipStream_t stream) {
  kvp::PrefillParams p;
  bool launch = false;
  const int32_t st = plan_prefill(pool, a, &p, &launch);
  if (st != KVP_OK || !launch) return st;
  const hipError_t e = kvp::launch_prefill(p, pool->desc.head_dim, pool->desc.dtype == KVP_FP8_E4M3, stream);
  if (e != hipSuccess) return fail(KVP_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return ok();
}

int32_t paged_prefill_step(kvp_pool pool, const kvp_prefill_args* a, const void* k_new, const void* v_new,
                           const int32_t* slot_mapping, hipStream_t stream) {
  kvp::PrefillParams p;
  bool launch = false;
  int32_t st = plan_prefill(pool, a, &p, &launch);  // every check before anything is launched
  if (st != KVP_OK) return st;
  if (a->total_q > 0) {
    if (!k_new || !v_new || !slot_mapping) return fail(KVP_ERR_INVALID_ARG, "NULL k_new, v_new or slot_mapping");
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(slot_mapping, 4))
      return fail(KVP_ERR_INVALID_ARG, "k_new/v_new must be 16-byte aligned, slot_mapping 4-byte aligned");
  }
  st = cache_write(pool, a->layer, k_new, v_new, slot_mapping, a->total_q, stream);
  if (st != KVP_OK || !launch) return st;
  const hipError_t e = kvp::launch_prefill(p, pool->desc.head_dim, pool->desc.dtype == KVP_FP8_E4M3, stream);
  if (e != hipSuccess) return fail(KVP_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return ok();
}

int32_t kv_pool_copy_blocks(kvp_pool pool, const int32_t* src, const int32_t* dst, int32_t num_pairs,
                            hipStream_t stream) {
  if (!pool) return fail(KVP_ERR_INVALID_ARG, "pool is NULL");
  if (num_pairs < 0) return fail(KVP_ERR_INVALID_ARG, "num_pairs < 0");
  if (num_pairs == 0) return ok();
  if (!src || !dst) return fail(KVP_ERR_INVALID_ARG, "NULL src or dst");
  if (!aligned(src, 4) || !aligned(dst, 4)) return fail(KVP_ERR_INVALID_ARG, "src/dst must be 4-byte aligned");
  const kvp_pool_desc& d = pool->desc;
  const size_t block_bytes = 2 * (size_t)d.num_kv_heads * d.block_size * d.head_dim * elt_bytes(d.dtype);
  const hipError_t e = kvp::launch_copy_blocks(pool->base, d.num_layers, d.num_blocks, block_bytes, src, dst,
                                               num_pairs, stream);
  if (e != hipSuccess) return fail(KVP_ERR_HIP, "copy_blocks launch: %s", hipGetErrorString(e));
  return ok();
}

const char* kvp_status_str(int32_t status) {
  switch (status) {
    case KVP_OK: return "ok";
    case KVP_ERR_INVALID_ARG: return "invalid argument";
    case KVP_ERR_UNSUPPORTED: return "unsupported";
    case KVP_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case KVP_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* kvp_last_error(void) { return g_err; }

}  // extern "C"
