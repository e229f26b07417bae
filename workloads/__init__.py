"""Seeded synthetic inputs for paged decode attention and the paged cache write.

This module only *draws* inputs: random values, the order in which physical
blocks are handed out, context lengths and the block tables that follow from
them.  It holds no attention arithmetic and no scatter; both the CPU oracle
(``oracle/``) and the GPU library's tests and bench consume what it returns.

Layout of the returned pool (the *logical* layout, the block shape the
PagedAttention write-ups print: per layer and block, ``[2, block_size,
num_kv_heads, head_dim]`` with index 0 = K and 1 = V)::

    pool[layer, block, kv, slot, kv_head, dim]

bf16 data is held as its raw 16-bit patterns (``np.uint16``) so that the
oracle and the device see identical bytes; fp32 data is ``np.float32``.
An "fp8" workload holds its pool as 8-bit E4M3 codes (``np.uint8``, drawn
directly as codes: sign, exponent field 1..9 and mantissa uniform, i.e.
magnitudes 2^-6 .. 7.5 before the per-layer scales k_scale and v_scale),
and its queries and new tokens in bf16.
Slots no sequence owns (unused blocks, the slots after a sequence's last
token, and the slots before a sliding window's first position) hold NaN so
that any read of them would show up in the results.

The five workloads (sizes as in the write-ups' Llama-3 serving examples):

1. tiny fp32 decode: 4 sequences of context {5, 16, 17, 40}, 8 query / 2 KV
   heads, head_dim 64, a 32-block pool, plus one next-token write per
   sequence;
2. Llama-3-8B-shaped bf16 layer: 64 sequences, 32/8 heads, head_dim 128,
   contexts uniform in [512, 4096], pool sized 1.25x the blocks in use;
3. Llama-3-70B-shaped bf16 layer: 128 sequences at context 8192, 64/8 heads;
4. shared-prefix decode: 256 sequences whose first 2048 tokens (128 full
   blocks) are the same physical blocks, each with a private tail of 1..512
   tokens whose last block is partial;
5. sliding-window layer: 32 sequences with contexts in [4096, 32768] and a
   4096-token window; tables hold only the blocks covering the window;
6. long contexts: 16 Llama-3-8B-shaped sequences of 32768..40960 tokens (the
   case for which a 32-token block size is offered).

``prefill_batch`` draws multi-token (chunked-prefill) batches: per sequence
a prior context already cached and a chunk of q_len new tokens whose K/V
are in the pool too; queries are packed [T, Hq, D] with offsets cu_q_lens.
``prefill_config`` is the Llama-3-8B-shaped chunked-prefill step: 8
sequences x 512-token chunks (4096 batched tokens) over prior contexts
uniform in [0, 8192].

Blocks hold 16 tokens unless a generator is asked for block_size=32 (same
lengths and shapes; tables in 32-token blocks).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BLOCK_SIZE = 16
BF16_NAN = np.uint16(0x7FC0)
FP8_NAN = np.uint8(0x7F)  # the E4M3 NaN code

_CONFIG_NAMES = {
    1: "tiny-fp32-S4-H8/2-D64",
    2: "llama3-8b-S64-H32/8-D128-ctx512..4096",
    3: "llama3-70b-S128-H64/8-D128-ctx8192",
    4: "shared-prefix-S256-H32/8-D128-prefix2048+tail1..512",
    5: "sliding-window4096-S32-H32/8-D128-ctx4096..32768",
    6: "llama3-8b-long-S16-H32/8-D128-ctx32768..40960",
    7: "chunked-prefill-S8x512-H32/8-D128-prior0..8192",
}


@dataclass
class Workload:
    config: int
    seed: int
    dtype: str                 # pool storage: "f32", "bf16" or "fp8" (E4M3 codes)
    num_layers: int
    num_blocks: int
    block_size: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    window: int                # 0 = full attention
    scale: float               # softmax scale, a float32-representable value
    seq_lens: np.ndarray       # int32 [S], absolute context length
    block_tables: np.ndarray   # int32 [S, W]; entries past row_blocks[s] are filler
    row_blocks: np.ndarray     # int32 [S], used entries of each row
    pool: np.ndarray           # [L, NB, 2, B, Hkv, D]; uint16 (bf16 bits), float32 or uint8 (fp8 codes)
    q: np.ndarray              # [S, Hq, D]; float32 for f32 pools, else bf16 bits
    # one next-token write per sequence (position seq_lens[s]); filled by with_next_token()
    k_new: Optional[np.ndarray] = None          # [T, Hkv, D]
    v_new: Optional[np.ndarray] = None          # [T, Hkv, D]
    slot_mapping: Optional[np.ndarray] = None   # int32 [T]
    block_tables_after: Optional[np.ndarray] = None
    row_blocks_after: Optional[np.ndarray] = None
    seq_lens_after: Optional[np.ndarray] = None
    unused_blocks: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))
    owned_slots: int = 0       # distinct physical slots some sequence attends to
    name: str = ""
    k_scale: float = 1.0       # fp8 pools: stored K code c means c * k_scale (float32-representable)
    v_scale: float = 1.0       # fp8 pools: stored V code c means c * v_scale

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def elt_bytes(self) -> int:
        """Bytes of one pool element."""
        return {"f32": 4, "bf16": 2, "fp8": 1}[self.dtype]

    @property
    def act_dtype(self) -> str:
        """Storage of queries, outputs and new tokens: fp32 or bf16."""
        return "f32" if self.dtype == "f32" else "bf16"

    def valid_tokens(self) -> np.ndarray:
        """Keys each sequence attends to (the whole context, or the window)."""
        if self.window > 0:
            return np.minimum(self.seq_lens, self.window).astype(np.int64)
        return self.seq_lens.astype(np.int64)

    def kv_bytes(self) -> int:
        """K+V bytes of the valid tokens of one layer (the algorithmic read)."""
        return int(self.valid_tokens().sum()) * 2 * self.num_kv_heads * self.head_dim * self.elt_bytes

    def unique_kv_bytes(self) -> int:
        """Like kv_bytes() but counting a physical slot read by several
        sequences once (the shared-prefix workload reads its prefix once
        per sequence but stores it once)."""
        return self.owned_slots * 2 * self.num_kv_heads * self.head_dim * self.elt_bytes

    def _first_pos(self, s: int) -> int:
        ctx = int(self.seq_lens[s])
        return max(0, ctx - self.window) if self.window > 0 else 0


# ---------------------------------------------------------------------------
# value drawing


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal_f32(seed: int, tag: int, shape) -> np.ndarray:
    rng = np.random.default_rng(np.random.SeedSequence([seed, tag]))
    return rng.standard_normal(size=shape, dtype=np.float32)


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest even) and return the raw bits."""
    import torch  # CPU conversion only

    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return x.astype(np.float32) if dtype == "f32" else _to_bf16_bits(x)


def _nan(dtype: str):
    return {"f32": np.float32("nan"), "bf16": BF16_NAN, "fp8": FP8_NAN}[dtype]


def _draw_codes(seed: int, tag: int, shape) -> np.ndarray:
    """E4M3 codes: sign, exponent field 1..9 and mantissa drawn uniformly."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, tag]))
    sign = rng.integers(0, 2, size=shape, dtype=np.uint8)
    expo = rng.integers(1, 10, size=shape, dtype=np.uint8)
    mant = rng.integers(0, 8, size=shape, dtype=np.uint8)
    return (sign << 7) | (expo << 3) | mant


_POOL_CHUNK = 64  # physical blocks drawn per independent random stream


def _draw_pool(seed: int, dtype: str, L: int, NB: int, Hkv: int, D: int, B: int) -> np.ndarray:
    """N(0,1) values for every slot of the pool, drawn in fixed chunks of
    physical blocks so the result does not depend on the thread count."""
    storage = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[dtype]
    pool = np.empty((L, NB, 2, B, Hkv, D), dtype=storage)
    nchunks = (NB + _POOL_CHUNK - 1) // _POOL_CHUNK

    def work(job):
        layer, c = job
        b0 = c * _POOL_CHUNK
        b1 = min(NB, b0 + _POOL_CHUNK)
        tag, shape = 1_000_003 * (layer + 1) + c, (b1 - b0, 2, B, Hkv, D)
        pool[layer, b0:b1] = _draw_codes(seed, tag, shape) if dtype == "fp8" else _store(_normal_f32(seed, tag, shape), dtype)

    jobs = [(layer, c) for layer in range(L) for c in range(nchunks)]
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, jobs))
    return pool


# ---------------------------------------------------------------------------
# block assignment


def _row_span(ctx: int, window: int, B: int):
    """(first logical block, number of table entries, leading masked slots)
    of one sequence: the whole context, or with a window only the blocks
    covering the last `window` positions."""
    first = max(0, ctx - window) if window > 0 else 0
    first_block = first // B
    last_block = (ctx - 1) // B
    return first_block, last_block - first_block + 1, first - first_block * B


def _poison_unowned(w: Workload) -> None:
    """NaN into every slot that no sequence owns."""
    B = w.block_size
    owned = np.zeros((w.num_blocks, B), dtype=bool)
    for s in range(w.num_seqs):
        ctx = int(w.seq_lens[s])
        _, nrow, start_off = _row_span(ctx, w.window, B)
        n = min(ctx, w.window) if w.window > 0 else ctx
        for j in range(nrow):
            lo = start_off if j == 0 else 0
            hi = min(B, start_off + n - j * B)
            owned[w.block_tables[s, j], lo:hi] = True
    nan = _nan(w.dtype)
    blk, slot = np.nonzero(~owned)
    w.pool[:, blk, :, slot] = nan
    w.unused_blocks = np.nonzero(~owned.any(axis=1))[0].astype(np.int32)
    w.owned_slots = int(owned.sum())


def _fill_tables(rows, width: int, filler: int) -> np.ndarray:
    bt = np.full((len(rows), width), filler, dtype=np.int32)
    for s, r in enumerate(rows):
        bt[s, : len(r)] = r
    return bt


def _finish(w: Workload, rows, extra_cols: int = 1) -> Workload:
    """Tables from per-sequence block lists; entries past a row's length
    point at an unowned (NaN) block so a stray read would poison the result
    without leaving the pool."""
    width = max(len(r) for r in rows) + extra_cols
    w.block_tables = _fill_tables(rows, width, 0)
    w.row_blocks = np.array([len(r) for r in rows], dtype=np.int32)
    _poison_unowned(w)
    if len(w.unused_blocks) == 0:
        raise ValueError("pool has no unowned block to use as table filler")
    for s, r in enumerate(rows):
        w.block_tables[s, len(r):] = w.unused_blocks[s % len(w.unused_blocks)]
    return w


def _base(config, seed, dtype, L, NB, Hq, Hkv, D, window, seq_lens, block_size=BLOCK_SIZE) -> Workload:
    w = Workload(
        config=config, seed=seed, dtype=dtype, num_layers=L, num_blocks=NB,
        block_size=block_size, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
        window=window, scale=float(np.float32(1.0 / math.sqrt(D))),
        seq_lens=np.asarray(seq_lens, dtype=np.int32),
        block_tables=np.zeros((0, 0), np.int32), row_blocks=np.zeros(0, np.int32),
        pool=np.zeros(0), q=np.zeros(0), name=_CONFIG_NAMES.get(config, f"custom-{config}"),
    )
    if dtype == "fp8":
        w.name += "-fp8"
        w.k_scale, w.v_scale = float(np.float32(0.37)), float(np.float32(0.61))
    if block_size != BLOCK_SIZE:
        w.name += f"-B{block_size}"
    return w


def _draw_q(w: Workload) -> None:
    w.q = _store(_normal_f32(w.seed, 7, (w.num_seqs, w.num_q_heads, w.head_dim)), w.act_dtype)


# ---------------------------------------------------------------------------
# the five workloads


def config1(seed: int = 1) -> Workload:
    """Tiny fp32 decode with a next-token write per sequence."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(32).astype(np.int32)
    ctx = [5, 16, 17, 40]
    w = _base(1, seed, "f32", 1, 32, 8, 2, 64, 0, ctx)
    rows, k = [], 0
    for c in ctx:
        nb = (c + BLOCK_SIZE - 1) // BLOCK_SIZE
        rows.append(list(perm[k:k + nb]))
        k += nb
    w.pool = _draw_pool(seed, w.dtype, 1, 32, 2, 64, BLOCK_SIZE)
    _finish(w, rows)
    _draw_q(w)
    return with_next_token(w, list(perm[k:]))


def config2(seed: int = 2, num_layers: int = 1, dtype: str = "bf16", block_size: int = BLOCK_SIZE) -> Workload:
    rng = np.random.default_rng(seed)
    ctx = rng.integers(512, 4096, size=64, endpoint=True)
    return _scattered(2, seed, rng, ctx, 32, 8, 128, 0, num_layers, dtype, block_size)


def config3(seed: int = 3, num_layers: int = 1, dtype: str = "bf16", block_size: int = BLOCK_SIZE) -> Workload:
    rng = np.random.default_rng(seed)
    ctx = np.full(128, 8192)
    return _scattered(3, seed, rng, ctx, 64, 8, 128, 0, num_layers, dtype, block_size)


def config5(seed: int = 5, num_layers: int = 1, dtype: str = "bf16", block_size: int = BLOCK_SIZE) -> Workload:
    rng = np.random.default_rng(seed)
    ctx = rng.integers(4096, 32768, size=32, endpoint=True)
    return _scattered(5, seed, rng, ctx, 32, 8, 128, 4096, num_layers, dtype, block_size)


def config6(seed: int = 6, num_layers: int = 1, dtype: str = "bf16", block_size: int = BLOCK_SIZE) -> Workload:
    """Long contexts, the case the block-size trade-off is about ([Optimizing]
    Trade-offs of Block Size Tuning: 32-token blocks for 32k+ contexts with a
    Llama-3-8B-shaped model): 16 sequences of U[32768, 40960] tokens."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(32768, 40960, size=16, endpoint=True)
    return _scattered(6, seed, rng, ctx, 32, 8, 128, 0, num_layers, dtype, block_size)


def _scattered(config, seed, rng, ctx, Hq, Hkv, D, window, L, dtype="bf16", block_size=BLOCK_SIZE) -> Workload:
    spans = [_row_span(int(c), window, block_size) for c in ctx]
    need = sum(nrow for _, nrow, _ in spans)
    NB = math.ceil(1.25 * need)
    perm = rng.permutation(NB).astype(np.int32)
    rows, k = [], 0
    for _, nrow, _ in spans:
        rows.append(list(perm[k:k + nrow]))
        k += nrow
    w = _base(config, seed, dtype, L, NB, Hq, Hkv, D, window, ctx, block_size)
    w.pool = _draw_pool(seed, w.dtype, L, NB, Hkv, D, block_size)
    _finish(w, rows)
    _draw_q(w)
    return w


def shared_prefix(seed: int, prefix_tokens: int, tails, num_q_heads: int = 32, num_kv_heads: int = 8,
                  head_dim: int = 128, num_layers: int = 1, config: int = 0, rng=None,
                  dtype: str = "bf16", block_size: int = BLOCK_SIZE) -> Workload:
    """Batch whose rows all start with the same prefix_tokens / block_size
    full blocks (the same physical ids in every row) followed by a private
    tail of tails[s] tokens (0 = the prefix alone); physical ids are a
    seeded permutation of a pool 1.25x the unique blocks."""
    B = block_size
    if prefix_tokens % B:
        raise ValueError("the shared prefix is a whole number of blocks")
    rng = np.random.default_rng(seed) if rng is None else rng
    tails = np.asarray(tails, dtype=np.int64)
    prefix_blocks = prefix_tokens // B
    tail_blocks = [(int(t) + B - 1) // B for t in tails]
    unique = prefix_blocks + sum(tail_blocks)
    NB = math.ceil(1.25 * unique)
    perm = rng.permutation(NB).astype(np.int32)
    prefix = list(perm[:prefix_blocks])
    rows, k = [], prefix_blocks
    for nb in tail_blocks:
        rows.append(prefix + list(perm[k:k + nb]))
        k += nb
    ctx = prefix_tokens + tails
    w = _base(config, seed, dtype, num_layers, NB, num_q_heads, num_kv_heads, head_dim, 0, ctx, B)
    w.pool = _draw_pool(seed, w.dtype, num_layers, NB, num_kv_heads, head_dim, B)
    _finish(w, rows)
    _draw_q(w)
    return w


def config4(seed: int = 4, num_layers: int = 1, num_seqs: int = 256, dtype: str = "bf16",
            block_size: int = BLOCK_SIZE) -> Workload:
    """Shared 2048-token prefix (128 blocks of 16, same physical ids in every
    row) plus a private tail per sequence whose last 16-token block is
    partial."""
    rng = np.random.default_rng(seed)
    tails_allowed = np.array([t for t in range(1, 513) if t % BLOCK_SIZE != 0])
    tails = rng.choice(tails_allowed, size=num_seqs)
    return shared_prefix(seed, 2048, tails, 32, 8, 128, num_layers, config=4, rng=rng, dtype=dtype,
                         block_size=block_size)


def make(config: int, seed: Optional[int] = None, num_layers: int = 1, dtype: str = "bf16",
         block_size: int = BLOCK_SIZE) -> Workload:
    """Workload `config` (1..6); configs 2..6 can hold their pool as fp8
    codes instead of bf16 (dtype="fp8") and use 32-token blocks
    (block_size=32), with the same shapes and lengths."""
    seed = config if seed is None else seed
    if config == 1:
        if num_layers != 1 or dtype != "bf16" or block_size != BLOCK_SIZE:
            raise ValueError("config 1 is one fp32 layer of 16-token blocks")
        return config1(seed)
    return {2: config2, 3: config3, 4: config4, 5: config5, 6: config6}[config](
        seed, num_layers=num_layers, dtype=dtype, block_size=block_size)


def custom(seed: int, ctx, num_q_heads: int, num_kv_heads: int, head_dim: int,
           dtype: str = "bf16", window: int = 0, num_layers: int = 1,
           pool_factor: float = 1.25, extra_blocks: int = 2, block_size: int = BLOCK_SIZE) -> Workload:
    """A small workload of the same structure with chosen shapes (parity
    sweeps over lengths, head groups, head_dim, window offsets and block
    size)."""
    rng = np.random.default_rng(seed)
    ctx = np.asarray(ctx, dtype=np.int64)
    spans = [_row_span(int(c), window, block_size) if c > 0 else (0, 0, 0) for c in ctx]
    need = sum(nrow for _, nrow, _ in spans)
    NB = max(math.ceil(pool_factor * need), need + extra_blocks)
    perm = rng.permutation(NB).astype(np.int32)
    rows, k = [], 0
    for _, nrow, _ in spans:
        rows.append(list(perm[k:k + nrow]))
        k += nrow
    w = _base(0, seed, dtype, num_layers, NB, num_q_heads, num_kv_heads, head_dim, window, ctx, block_size)
    w.pool = _draw_pool(seed, dtype, num_layers, NB, num_kv_heads, head_dim, block_size)
    width_rows = [r if r else [] for r in rows]
    width = max([len(r) for r in width_rows] + [1]) + 1
    w.block_tables = _fill_tables(width_rows, width, 0)
    w.row_blocks = np.array([len(r) for r in width_rows], dtype=np.int32)
    _poison_unowned(w)
    filler = w.unused_blocks if len(w.unused_blocks) else np.array([0], np.int32)
    for s, r in enumerate(width_rows):
        w.block_tables[s, len(r):] = filler[s % len(filler)]
    _draw_q(w)
    return w


def with_next_token(w: Workload, fresh_blocks) -> Workload:
    """Add one next-token K/V per sequence at position seq_lens[s]; a
    sequence whose last block is full takes the next block of `fresh_blocks`
    (the decode-append rule: a block boundary allocates).  Values, the slot
    of each token (physical block * block_size + offset) and the tables for
    context seq_lens + 1 are recorded (under a window the row then starts at
    the block holding position seq_lens + 1 - window); the pool itself is
    left untouched."""
    B = w.block_size
    fresh = list(fresh_blocks)
    T = w.num_seqs
    slots = np.empty(T, dtype=np.int32)
    rows = []
    for s in range(T):
        pos = int(w.seq_lens[s])
        row = list(w.block_tables[s, : w.row_blocks[s]])
        first_block = _row_span(pos, w.window, B)[0] if pos > 0 else 0
        lb = pos // B - first_block
        if lb == len(row):
            row.append(fresh.pop(0))
        slots[s] = row[lb] * B + pos % B
        new_first = _row_span(pos + 1, w.window, B)[0]
        rows.append(row[new_first - first_block:])
    w.k_new = _store(_normal_f32(w.seed, 11, (T, w.num_kv_heads, w.head_dim)), w.act_dtype)
    w.v_new = _store(_normal_f32(w.seed, 12, (T, w.num_kv_heads, w.head_dim)), w.act_dtype)
    w.slot_mapping = slots
    width = max(w.block_tables.shape[1], max(len(r) for r in rows))
    bt = np.full((T, width), w.block_tables[0, -1], dtype=np.int32)
    bt[:, : w.block_tables.shape[1]] = w.block_tables
    for s, r in enumerate(rows):
        bt[s, : len(r)] = r
    w.block_tables_after = bt
    w.row_blocks_after = np.array([len(r) for r in rows], dtype=np.int32)
    w.seq_lens_after = (w.seq_lens + 1).astype(np.int32)
    return w


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    return _to_bf16_bits(np.asarray(x, dtype=np.float32))


# ---------------------------------------------------------------------------
# multi-token (prefill / chunked-prefill) batches


def prefill_batch(seed: int, prior, q_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                  window: int = 0, dtype: str = "bf16", block_size: int = BLOCK_SIZE, num_layers: int = 1,
                  config: int = 0, pool_factor: float = 1.25) -> Workload:
    """Sequence s has prior[s] cached tokens and a chunk of q_lens[s] new
    tokens (positions prior .. prior + q_len - 1, their K/V already stored);
    seq_lens = prior + q_lens.  Table rows list the blocks covering every
    position some query of the chunk attends (from max(0, prior + 1 - W)
    under a window W, else 0); physical ids are a seeded permutation of a
    pool pool_factor x the blocks in use; unowned slots NaN.  q is
    [T, Hq, D] with sequence s's chunk at rows cu_q_lens[s] .. cu_q_lens[s+1]-1."""
    B = block_size
    rng = np.random.default_rng(seed)
    prior = np.asarray(prior, dtype=np.int64)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    ctx = prior + q_lens
    firsts = [max(0, int(p) + 1 - window) if window > 0 else 0 for p in prior]
    nbs = [((int(c) - 1) // B - f // B + 1) if c > 0 else 0 for c, f in zip(ctx, firsts)]
    need = sum(nbs)
    NB = max(math.ceil(pool_factor * need), need + 2)
    perm = rng.permutation(NB).astype(np.int32)
    rows, k = [], 0
    for nb in nbs:
        rows.append(list(perm[k:k + nb]))
        k += nb
    w = _base(config, seed, dtype, num_layers, NB, num_q_heads, num_kv_heads, head_dim, window, ctx, B)
    w.pool = _draw_pool(seed, dtype, num_layers, NB, num_kv_heads, head_dim, B)
    owned = np.zeros((NB, B), dtype=bool)
    for s, (c, f) in enumerate(zip(ctx, firsts)):
        for pos in range(f, int(c)):
            owned[rows[s][pos // B - f // B], pos % B] = True
    blk, slot = np.nonzero(~owned)
    w.pool[:, blk, :, slot] = _nan(dtype)
    w.unused_blocks = np.nonzero(~owned.any(axis=1))[0].astype(np.int32)
    w.owned_slots = int(owned.sum())
    width = max([len(r) for r in rows] + [1]) + 1
    w.block_tables = _fill_tables(rows, width, int(w.unused_blocks[0]))
    w.row_blocks = np.array([len(r) for r in rows], dtype=np.int32)
    w.prior = prior.astype(np.int32)
    w.q_lens = q_lens.astype(np.int32)
    w.cu_q_lens = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    T = int(w.cu_q_lens[-1])
    w.q = _store(_normal_f32(seed, 7, (T, num_q_heads, head_dim)), w.act_dtype)
    return w


def prefill_config(seed: int = 7, num_layers: int = 1, dtype: str = "bf16", block_size: int = BLOCK_SIZE,
                   num_seqs: int = 8, chunk: int = 512, max_prior: int = 8192) -> Workload:
    """The Llama-3-8B-shaped chunked-prefill step (config 7): num_seqs
    sequences, each a chunk of `chunk` tokens after a prior context uniform
    in [0, max_prior]."""
    rng = np.random.default_rng(seed)
    prior = rng.integers(0, max_prior, size=num_seqs, endpoint=True)
    return prefill_batch(seed, prior, np.full(num_seqs, chunk), 32, 8, 128, 0, dtype, block_size, num_layers,
                         config=7)
