"""Plain float64 statement of multi-token (prefill / chunked-prefill) paged
attention.

TEST INFRASTRUCTURE (see the package docstring).

[Optimizing] §The Block Manager and Dynamic Allocation Lifecycle, The
Prefill Phase: the prompt's key-value states are computed in one parallel
step and written into the blocks the scheduler allocated; §Production
Tuning: Ratios, Failure Modes, and Mitigations, Failure Mode 2 (chunked
prefill): a long prompt is split into chunks processed step by step, so a
chunk's queries attend the context cached by earlier chunks as well as the
chunk itself.  The pages give no formula;
the one used is causal scaled dot-product attention: the chunk of sequence
s holds its last q_len positions ctx-q_len .. ctx-1 (its K/V already in the
pool), and the query at position p attends the keys at positions
lo(p) .. p, lo(p) = 0, or max(0, p + 1 - W) under a sliding window W
([Pool] §Hybrid models get groups: a window layer needs only the last W
positions; for q_len = 1 this is exactly decode attention at context p + 1).

Table rows list the blocks covering every key some query of the chunk
attends: positions first .. ctx-1 with first = lo(ctx - q_len).
"""
from __future__ import annotations

import numpy as np

from .paged import to_f64


def chunk_first(ctx: int, q_len: int, window: int) -> int:
    """First position any query of the chunk attends."""
    p0 = ctx - q_len
    return max(0, p0 + 1 - window) if window > 0 else 0


def prefill_attention_seq(pool: np.ndarray, layer: int, q_chunk: np.ndarray, table_row, ctx: int,
                          window: int, scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
                          heads=None, tokens=None) -> np.ndarray:
    """Output [q_len, Hq, D] (float64) of one sequence's chunk: gather the
    keys and values of positions first .. ctx-1 by walking the table row,
    then for query token i (position p = ctx - q_len + i) and head h, with
    KV head h // G, softmax over the keys at lo(p) .. p of K q * scale,
    times V.  K and V are the stored values times k_scale, v_scale."""
    q = to_f64(q_chunk)
    q_len, Hq, D = q.shape
    B = pool.shape[3]
    Hkv = pool.shape[4]
    G = Hq // Hkv
    out = np.zeros((q_len, Hq, D))
    if q_len == 0 or ctx <= 0:
        return out
    first = chunk_first(ctx, q_len, window)
    fb = first // B
    nb = (ctx - 1) // B - fb + 1
    K = to_f64(np.concatenate([pool[layer, int(table_row[j]), 0] for j in range(nb)], axis=0))
    V = to_f64(np.concatenate([pool[layer, int(table_row[j]), 1] for j in range(nb)], axis=0))
    base = fb * B  # position of K[0]
    K, V = K * k_scale, V * v_scale
    for i in (range(q_len) if tokens is None else tokens):
        p = ctx - q_len + i
        if p < 0:
            continue  # a chunk longer than its context: no position, no keys
        lo = max(0, p + 1 - window) if window > 0 else 0
        ks, ke = lo - base, p - base + 1
        for h in (range(Hq) if heads is None else heads):
            kv = h // G
            z = (K[ks:ke, kv, :] @ q[i, h]) * scale
            e = np.exp(z - z.max())
            out[i, h] = (e / e.sum()) @ V[ks:ke, kv, :]
    return out


def prefill_attention(pool: np.ndarray, layer: int, q: np.ndarray, cu_q_lens, block_tables, seq_lens,
                      window: int, scale: float, k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """Chunked-prefill attention for every sequence: q is [T, Hq, D] with
    sequence s's chunk at rows cu_q_lens[s] .. cu_q_lens[s+1]-1; returns the
    float64 [T, Hq, D] outputs."""
    out = np.zeros(q.shape, dtype=np.float64)
    cu = np.asarray(cu_q_lens)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        out[a:b] = prefill_attention_seq(pool, layer, q[a:b], block_tables[s], int(seq_lens[s]), window, scale,
                                         k_scale, v_scale)
    return out


def prefill_attention_bruteforce(pool: np.ndarray, layer: int, q: np.ndarray, cu_q_lens, block_tables,
                                 seq_lens, window: int, scale: float) -> np.ndarray:
    """The same result position by position with scalar Python arithmetic:
    each attended key's block is table[pos // B - first // B], its slot
    pos % B.  Tiny inputs only."""
    import math

    T, Hq, D = q.shape
    B = pool.shape[3]
    G = Hq // pool.shape[4]
    qf = to_f64(q)
    out = np.zeros((T, Hq, D))
    cu = [int(x) for x in np.asarray(cu_q_lens)]
    for s in range(len(cu) - 1):
        ctx = int(seq_lens[s])
        q_len = cu[s + 1] - cu[s]
        first = chunk_first(ctx, q_len, window)
        for i in range(q_len):
            p = ctx - q_len + i
            lo = max(0, p + 1 - window) if window > 0 else 0
            keys = list(range(lo, p + 1))
            for h in range(Hq):
                kv = h // G
                z = []
                for pos in keys:
                    blk = int(block_tables[s][pos // B - first // B])
                    kvec = to_f64(pool[layer, blk, 0, pos % B, kv])
                    z.append(sum(float(qf[cu[s] + i, h, d]) * float(kvec[d]) for d in range(D)) * scale)
                if not z:
                    continue
                top = max(z)
                wts = [math.exp(x - top) for x in z]
                tot = sum(wts)
                acc = [0.0] * D
                for wt, pos in zip(wts, keys):
                    blk = int(block_tables[s][pos // B - first // B])
                    vvec = to_f64(pool[layer, blk, 1, pos % B, kv])
                    for d in range(D):
                        acc[d] += wt * float(vvec[d])
                out[cu[s] + i, h] = [x / tot for x in acc]
    return out
