"""Plain float64 statements of the paged cache write and paged decode attention.

TEST INFRASTRUCTURE (see the package docstring): imported only by tests, the
smoke check and the bench's CPU baseline.

Pool layout consumed here is the block shape the pages print ([Paged]
§What a physical block looks like), with the layer and block index in front:

    pool[layer, block, kv, slot, kv_head, dim]     kv: 0 = K, 1 = V

bf16 pools arrive as uint16 bit patterns, fp32 pools as float32, FP8 pools
as uint8 E4M3 codes with one (k_scale, v_scale) pair for the layer
(``oracle.fp8``).
"""
from __future__ import annotations

import math

import numpy as np

from .fp8 import e4m3_decode, quantize


# ---------------------------------------------------------------------------
# representation


def to_f64(x: np.ndarray) -> np.ndarray:
    """Exact widening to float64: uint16 arrays are bf16 bit patterns (a bf16
    value is the upper half of the float32 with the same bits), uint8 arrays
    E4M3 codes (unscaled), float32 is widened directly."""
    x = np.asarray(x)
    if x.dtype == np.uint8:
        return e4m3_decode(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError(f"unsupported storage dtype {x.dtype}")


# ---------------------------------------------------------------------------
# which table entries and slots a sequence owns


def row_span(ctx: int, window: int, block_size: int):
    """(start_off, n, nblocks) of one sequence's block-table row.

    Without a window the row lists logical blocks 0 .. floor((ctx-1)/B) and
    all ctx tokens are attended ([Optimizing] §PagedAttention: logical block
    of position i is floor(i / B)).  With a window W > 0 the row lists only
    the blocks covering positions ctx-W .. ctx-1 ([Pool] §Hybrid models get
    groups; [Memory] §Why the next token needs yesterday's state); the
    first listed block may start with start_off = (ctx-W) mod B slots that
    lie before the window.  n is the number of attended keys and nblocks the
    number of table entries the row uses.
    """
    if ctx <= 0:
        return 0, 0, 0
    first = max(0, ctx - window) if window > 0 else 0
    start_off = first % block_size
    n = ctx - first
    nblocks = -(-(start_off + n) // block_size)
    return start_off, n, nblocks


def check_tables(block_tables, seq_lens, window: int, block_size: int, num_blocks: int,
                 row_blocks=None) -> None:
    """Raise ValueError unless every row is well formed: its used entries are
    in range and distinct, it uses exactly ceil((start_off + n) / B)
    entries, so that only its last block can be short of tokens (and, under
    a window, its first) -- [Paged] §Borrowing paging from the operating
    system (the only waste is inside a request's last block) and
    [Optimizing] §PagedAttention (at most B-1 wasted slots per request)."""
    bt = np.asarray(block_tables)
    for s, ctx in enumerate(np.asarray(seq_lens)):
        start_off, n, nb = row_span(int(ctx), window, block_size)
        if row_blocks is not None and int(row_blocks[s]) != nb:
            raise ValueError(f"row {s}: {int(row_blocks[s])} entries, expected {nb}")
        if nb > bt.shape[1]:
            raise ValueError(f"row {s}: needs {nb} entries, table has {bt.shape[1]}")
        ids = [int(b) for b in bt[s, :nb]]
        if any(b < 0 or b >= num_blocks for b in ids):
            raise ValueError(f"row {s}: block id out of range")
        if len(set(ids)) != len(ids):
            raise ValueError(f"row {s}: a block appears twice")
        # slots used in each listed block; only the first and last may be short
        for j in range(nb):
            lo = start_off if j == 0 else 0
            hi = min(block_size, start_off + n - j * block_size)
            if hi - lo < block_size and 0 < j < nb - 1:
                raise ValueError(f"row {s}: interior block {j} is partial")
            if hi <= lo:
                raise ValueError(f"row {s}: block {j} holds no attended token")
        if window == 0 and start_off != 0:
            raise ValueError(f"row {s}: only a windowed row may start mid-block")


# ---------------------------------------------------------------------------
# cache write


def cache_write(pool: np.ndarray, layer: int, k_new: np.ndarray, v_new: np.ndarray,
                slot_mapping: np.ndarray, k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """Return a copy of `pool` with token t's K and V stored at slot
    slot_mapping[t] of `layer`: physical block slot // B, offset slot % B
    ([Optimizing] §The Block Manager and Dynamic Allocation Lifecycle: the
    kernel writes each token's key and value vectors into the physical
    block's free slot).  A negative slot is skipped (padding).  The copy is
    bit for bit: no arithmetic touches the values, except for an FP8 pool,
    whose codes are the new values quantized with the layer's scales
    (``oracle.fp8.quantize``)."""
    out = pool.copy()
    if pool.dtype == np.uint8:
        k_new, v_new = quantize(k_new, k_scale), quantize(v_new, v_scale)
    B = pool.shape[3]
    for t, slot in enumerate(np.asarray(slot_mapping)):
        slot = int(slot)
        if slot < 0:
            continue
        block, offset = slot // B, slot % B
        for h in range(pool.shape[4]):
            out[layer, block, 0, offset, h, :] = k_new[t, h, :]
            out[layer, block, 1, offset, h, :] = v_new[t, h, :]
    return out


def copy_blocks(pool: np.ndarray, src, dst) -> np.ndarray:
    """Return a copy of `pool` in which every layer's K and V of physical
    block dst[i] equal those of block src[i] before the call ([Optimizing]
    §Copy-on-Write (CoW) for Parallel Sampling and Prefix Caching: a writer
    of a shared block gets a new physical block holding a copy of it).
    Pairs naming a block outside the pool, or src == dst, are skipped."""
    out = pool.copy()
    nb = pool.shape[1]
    for a, b in zip(np.asarray(src).tolist(), np.asarray(dst).tolist()):
        if 0 <= a < nb and 0 <= b < nb and a != b:
            out[:, b] = pool[:, a]
    return out


# ---------------------------------------------------------------------------
# decode attention


def gather_kv(pool: np.ndarray, layer: int, table_row, start_off: int, n: int):
    """Walk one block-table row ([Paged] §Two lookup structures: the row is
    the ordered list of physical blocks), concatenate those blocks' K and V
    in logical order, and keep the n attended tokens after start_off.
    Returns float64 arrays K, V of shape [n, num_kv_heads, head_dim]."""
    B = pool.shape[3]
    nb = -(-(start_off + n) // B)
    ks = [pool[layer, int(table_row[j]), 0] for j in range(nb)]
    vs = [pool[layer, int(table_row[j]), 1] for j in range(nb)]
    if nb == 0:
        shape = (0,) + pool.shape[4:]
        return np.zeros(shape), np.zeros(shape)
    K = to_f64(np.concatenate(ks, axis=0))[start_off:start_off + n]
    V = to_f64(np.concatenate(vs, axis=0))[start_off:start_off + n]
    return K, V


def softmax_weights(q_head: np.ndarray, K_head: np.ndarray, scale: float) -> np.ndarray:
    """Attention weights of one query head over its n keys:
    p_i = exp(z_i - max z) / sum_j exp(z_j - max z), z = K q * scale."""
    z = (K_head @ q_head) * scale
    e = np.exp(z - z.max())
    return e / e.sum()


def decode_attention_seq(pool: np.ndarray, layer: int, q_seq: np.ndarray, table_row,
                         ctx: int, window: int, scale: float, heads=None,
                         k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """Output [Hq, D] (float64) of one sequence: gather its K/V by walking its
    table, then for each query head h, with G = Hq / Hkv and KV head h // G,
    out_h = softmax(K q_h * scale) V.  The stored K and V are multiplied by
    k_scale and v_scale first (FP8 pools; 1 otherwise)."""
    q = to_f64(q_seq)
    Hq, D = q.shape
    Hkv = pool.shape[4]
    G = Hq // Hkv
    B = pool.shape[3]
    start_off, n, _ = row_span(int(ctx), window, B)
    out = np.zeros((Hq, D))
    if n == 0:
        return out
    K, V = gather_kv(pool, layer, table_row, start_off, n)
    K, V = K * k_scale, V * v_scale
    for h in (range(Hq) if heads is None else heads):
        kv = h // G
        p = softmax_weights(q[h], K[:, kv, :], scale)
        out[h] = p @ V[:, kv, :]
    return out


def decode_attention(pool: np.ndarray, layer: int, q: np.ndarray, block_tables, seq_lens,
                     window: int, scale: float, k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """Decode attention for every sequence: float64 [S, Hq, D]."""
    S = q.shape[0]
    out = np.zeros(q.shape, dtype=np.float64)
    for s in range(S):
        out[s] = decode_attention_seq(pool, layer, q[s], block_tables[s], int(seq_lens[s]),
                                      window, scale, k_scale=k_scale, v_scale=v_scale)
    return out


def decode_attention_bruteforce(pool: np.ndarray, layer: int, q: np.ndarray, block_tables,
                                seq_lens, window: int, scale: float) -> np.ndarray:
    """The same result computed token by token: for each attended position i
    of a sequence, translate it to (physical block, offset) =
    (table[i // B], i % B) ([Optimizing] §PagedAttention formulas), read
    that key and value, and accumulate scores and the weighted sum with
    scalar Python arithmetic.  For tiny inputs only."""
    S, Hq, D = q.shape
    Hkv = pool.shape[4]
    G = Hq // Hkv
    B = pool.shape[3]
    qf = to_f64(q)
    out = np.zeros((S, Hq, D))
    for s in range(S):
        ctx = int(seq_lens[s])
        first = max(0, ctx - window) if window > 0 else 0
        base_block = first // B
        positions = list(range(first, ctx))
        for h in range(Hq):
            kv = h // G
            scores = []
            for i in positions:
                blk = int(block_tables[s][i // B - base_block])
                key = to_f64(pool[layer, blk, 0, i % B, kv])
                scores.append(sum(float(qf[s, h, d]) * float(key[d]) for d in range(D)) * scale)
            if not scores:
                continue
            top = max(scores)
            weights = [math.exp(z - top) for z in scores]
            total = sum(weights)
            acc = [0.0] * D
            for w_i, i in zip(weights, positions):
                blk = int(block_tables[s][i // B - base_block])
                val = to_f64(pool[layer, blk, 1, i % B, kv])
                for d in range(D):
                    acc[d] += w_i * float(val[d])
            out[s, h] = [a / total for a in acc]
    return out
