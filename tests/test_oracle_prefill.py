"""Pins of the prefill (multi-token, causal) oracle to things other than
itself: scalar brute force, torch's float64 scaled_dot_product_attention
with an explicit causal mask over an independent per-position gather, the
decode oracle (a chunk's token at position p is a decode query at context
p + 1), closed forms, and planted mistakes."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from indep import widen


def gather_positions(w, s, positions):
    """K, V (float64) of sequence s at absolute positions, by per-position
    address translation (test-side, independent of the oracle's gather)."""
    B = w.block_size
    ctx, q_len = int(w.seq_lens[s]), int(w.q_lens[s])
    p0 = ctx - q_len
    first = max(0, p0 + 1 - w.window) if w.window > 0 else 0
    pos = np.asarray(positions)
    blocks = np.asarray(w.block_tables[s])[pos // B - first // B]
    return widen(w.pool[0, blocks, 0, pos % B]), widen(w.pool[0, blocks, 1, pos % B])


def sdpa_causal(w):
    """torch float64 SDPA per sequence with a boolean mask: query i (position
    p = ctx - q_len + i) may see key position k iff lo(p) <= k <= p."""
    T, Hq, D = w.q.shape
    G = Hq // w.num_kv_heads
    out = np.zeros((T, Hq, D))
    for s in range(w.num_seqs):
        a, b = int(w.cu_q_lens[s]), int(w.cu_q_lens[s + 1])
        ctx, q_len = int(w.seq_lens[s]), b - a
        if q_len == 0:
            continue
        p = ctx - q_len + np.arange(q_len)
        lo = np.maximum(0, p + 1 - w.window) if w.window > 0 else np.zeros_like(p)
        keys = np.arange(lo.min(), ctx)
        K, V = gather_positions(w, s, keys)
        mask = (keys[None, :] >= lo[:, None]) & (keys[None, :] <= p[:, None])
        qt = torch.from_numpy(widen(w.q[a:b])).permute(1, 0, 2).unsqueeze(0)          # [1, Hq, q, D]
        kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, 0).unsqueeze(0).contiguous()
        vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, 0).unsqueeze(0).contiguous()
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask),
                                                             scale=w.scale)
        out[a:b] = o[0].permute(1, 0, 2).numpy()
    return out


def run(w, **kw):
    return oracle.prefill_attention(w.pool, 0, w.q, w.cu_q_lens, w.block_tables, w.seq_lens, w.window, w.scale, **kw)


@pytest.mark.parametrize("window", [0, 7, 20])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_bruteforce(window, dtype):
    w = W.prefill_batch(11 + window, [0, 5, 16, 3], [3, 12, 1, 20], 4, 2, 8, window=window, dtype=dtype)
    a = run(w)
    b = oracle.prefill_attention_bruteforce(w.pool, 0, w.q, w.cu_q_lens, w.block_tables, w.seq_lens, w.window,
                                            w.scale)
    assert np.all(np.isfinite(a))
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


@pytest.mark.parametrize("window,B", [(0, 16), (24, 16), (0, 32), (40, 32)])
def test_prefill_sdpa_crosscheck(window, B):
    w = W.prefill_batch(21 + window + B, [0, 1, 15, 16, 31, 100], [1, 16, 17, 5, 64, 33], 8, 2, 16,
                        window=window, block_size=B)
    np.testing.assert_allclose(run(w), sdpa_causal(w), rtol=0, atol=1e-12)


@pytest.mark.parametrize("window", [0, 30])
def test_prefill_token_is_a_decode_query(window):
    """Token i of a chunk (position p) equals decode attention at context
    p + 1 over the same blocks: the decode row starts at the block holding
    decode's first attended position."""
    w = W.prefill_batch(31, [0, 9, 40], [5, 20, 33], 8, 4, 16, window=window)
    out = run(w)
    B = w.block_size
    for s in range(w.num_seqs):
        ctx, q_len = int(w.seq_lens[s]), int(w.q_lens[s])
        first = max(0, ctx - q_len + 1 - window) if window else 0
        for i in range(q_len):
            p = ctx - q_len + i
            d_first = max(0, p + 1 - window) if window else 0
            row = w.block_tables[s][d_first // B - first // B:]
            ref = oracle.decode_attention_seq(w.pool, 0, w.q[w.cu_q_lens[s] + i], row, p + 1, window, w.scale)
            np.testing.assert_allclose(out[w.cu_q_lens[s] + i], ref, rtol=0, atol=1e-12)


def test_prefill_closed_forms():
    """A fresh prompt's first token sees only itself: out = V[0] exactly;
    V constant over the keys gives that constant for every token."""
    w = W.prefill_batch(41, [0, 0], [9, 30], 4, 2, 8, dtype="f32")
    out = run(w)
    G = 2
    for s in range(2):
        V0 = widen(w.pool[0, w.block_tables[s][0], 1, 0])
        for h in range(4):
            assert np.array_equal(out[w.cu_q_lens[s], h], V0[h // G])
    pool = w.pool.copy()
    pool[0, :, 1] = np.float32(0.625)
    out = oracle.prefill_attention(pool, 0, w.q, w.cu_q_lens, w.block_tables, w.seq_lens, 0, w.scale)
    assert np.allclose(out, 0.625, rtol=0, atol=1e-15)


def test_prefill_empty_chunk_and_scales():
    """A sequence with no chunk contributes no rows; K/V scales multiply
    the keys and values (q scaled by k_scale gives the same scores)."""
    w = W.prefill_batch(51, [4, 10, 3], [2, 0, 6], 4, 2, 8, dtype="f32")
    assert w.cu_q_lens[1] == w.cu_q_lens[2]
    a = run(w, k_scale=2.0, v_scale=0.5)
    q2 = (w.q * 2.0).astype(np.float32)
    b = oracle.prefill_attention(w.pool, 0, q2, w.cu_q_lens, w.block_tables, w.seq_lens, 0, w.scale) * 0.5
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


@pytest.mark.parametrize("kind", ["strict_causal", "window_plus_one", "shifted_positions", "no_prior_context",
                                  "whole_context"])
def test_planted_prefill_mistake_is_caught(kind):
    """Plausible mistakes in a prefill oracle each break the SDPA cross-check."""
    w = W.prefill_batch(61, [0, 7, 20], [6, 9, 17], 4, 2, 8, window=12 if kind == "window_plus_one" else 0,
                        dtype="f32")
    ref = sdpa_causal(w)
    B = w.block_size
    T, Hq, D = w.q.shape
    out = np.zeros((T, Hq, D))
    for s in range(w.num_seqs):
        ctx, q_len = int(w.seq_lens[s]), int(w.q_lens[s])
        for i in range(q_len):
            p = ctx - q_len + i
            lo, hi = (max(0, p + 1 - w.window) if w.window else 0), p
            if kind == "strict_causal":
                hi = p - 1
            elif kind == "window_plus_one":
                lo = max(0, p - w.window)
            elif kind == "shifted_positions":
                hi = min(p + 1, ctx - 1)
            elif kind == "no_prior_context":
                lo = ctx - q_len
            elif kind == "whole_context":
                hi = ctx - 1
            if hi < lo:
                continue
            K, V = gather_positions(w, s, np.arange(lo, hi + 1))
            for h in range(Hq):
                z = K[:, h // 2] @ widen(w.q[w.cu_q_lens[s] + i, h]) * w.scale
                e = np.exp(z - z.max())
                out[w.cu_q_lens[s] + i, h] = e @ V[:, h // 2] / e.sum()
    assert not np.allclose(out, ref, rtol=0, atol=1e-9)
