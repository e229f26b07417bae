"""Pins of the CPU oracle to things other than itself.

* hand-derived cases in tests/golden/ (closed forms worked out on paper from
  the pages' paged addressing and the attention definition);
* an independent library routine (torch's scaled_dot_product_attention in
  float64 on the CPU) fed by an independent per-position gather;
* brute force with scalar arithmetic on tiny inputs;
* invariants: physical-id relabelling, shared-prefix aliasing, softmax rows
  summing to one, grouped-query consistency, the only-last-block-partial
  table rule;
* planted mistakes: each plausible bug in the oracle must fail a pin.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.paged as op
import workloads as W
from indep import widen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# helpers (test-side; independent of the oracle's gather)


def positions_of(ctx, window, B):
    first = max(0, ctx - window) if window > 0 else 0
    return first, np.arange(first, ctx)


def independent_gather(pool, layer, table_row, ctx, window):
    """Per-position address translation with numpy fancy indexing."""
    B = pool.shape[3]
    first, pos = positions_of(ctx, window, B)
    row = np.asarray(table_row)
    blocks = row[pos // B - first // B]
    offs = pos % B
    K = widen(pool[layer, blocks, 0, offs])
    V = widen(pool[layer, blocks, 1, offs])
    return K, V


def sdpa_reference(w_pool, layer, q, tables, seq_lens, window, scale):
    S, Hq, D = q.shape
    Hkv = w_pool.shape[4]
    G = Hq // Hkv
    out = np.zeros((S, Hq, D))
    for s in range(S):
        K, V = independent_gather(w_pool, layer, tables[s], int(seq_lens[s]), window)
        if K.shape[0] == 0:
            continue
        qt = torch.from_numpy(widen(q[s])).reshape(1, Hq, 1, D)
        kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
        vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
        out[s] = o.reshape(Hq, D).numpy()
    return out


def load_golden_attention():
    with open(os.path.join(GOLDEN, "attention_hand.json")) as f:
        return json.load(f)["cases"]


def build_case(case):
    """Pool, queries, tables and lengths of a golden case.  A case with
    "storage": "bf16" gives every element as a bf16 bit pattern ("0x3F80")
    and is built as uint16 arrays, the form the oracle takes for bf16."""
    B, NB = case["block_size"], case["num_blocks"]
    Hq, Hkv, D = case["num_q_heads"], case["num_kv_heads"], case["head_dim"]
    Wn = case["window"]
    bf16 = case.get("storage") == "bf16"
    if bf16:
        elt = np.uint16

        def conv(v):
            return np.vectorize(lambda h: int(h, 16), otypes=[np.uint16])(np.asarray(v))

        pool = np.full((1, NB, 2, B, Hkv, D), 0x7FC0, dtype=np.uint16)  # NaN in unused slots
    else:
        elt = np.float32

        def conv(v):
            return np.asarray(v, dtype=np.float32)

        pool = np.full((1, NB, 2, B, Hkv, D), np.nan, dtype=np.float32)
    seqs = case["seqs"]
    width = max(len(s["table"]) for s in seqs)
    tables = np.zeros((len(seqs), width), dtype=np.int32)
    ctxs = np.array([s["ctx"] for s in seqs], dtype=np.int32)
    q = np.stack([conv(s["q"]) for s in seqs]).astype(elt)
    for si, s in enumerate(seqs):
        tables[si, : len(s["table"])] = s["table"]
        ctx = s["ctx"]
        first, pos = positions_of(ctx, Wn, B)
        first_block = first // B
        fill = s.get("fill", {})
        for i in range(first_block * B, ctx):
            blk = s["table"][i // B - first_block]
            off = i % B
            if i < first:
                val = s["outside_window_value"]
                pool[0, blk, :, off] = val
                continue
            key = s.get("keys", {}).get(str(i), fill.get("key"))
            value = s.get("values", {}).get(str(i), fill.get("value"))
            if isinstance(value, str) and value == "position":
                value = np.full((Hkv, D), float(i))
            pool[0, blk, 0, off] = conv(key)
            pool[0, blk, 1, off] = conv(value)
    return pool, q, tables, ctxs


def golden_ok(attn_fn=None):
    """True when every hand-derived case holds for the oracle (or a stand-in)."""
    fn = attn_fn or oracle.decode_attention
    for case in load_golden_attention():
        pool, q, tables, ctxs = build_case(case)
        out = fn(pool, 0, q, tables, ctxs, case["window"], case["scale"])
        if not np.all(np.abs(out - np.asarray(case["expected"])) <= case["tol"]):
            return False
    return True


def tiny_random(seed, dtype="f32", window=0, G=2, D=8, ctx=(1, 5, 16, 17, 33)):
    return W.custom(seed, list(ctx), num_q_heads=2 * G, num_kv_heads=2, head_dim=D,
                    dtype=dtype, window=window)


# ---------------------------------------------------------------------------
# hand-derived values


@pytest.mark.parametrize("case", load_golden_attention(), ids=lambda c: c["name"])
def test_golden_attention(case):
    pool, q, tables, ctxs = build_case(case)
    out = oracle.decode_attention(pool, 0, q, tables, ctxs, case["window"], case["scale"])
    np.testing.assert_allclose(out, np.asarray(case["expected"]), rtol=0, atol=case["tol"])
    bf = oracle.decode_attention_bruteforce(pool, 0, q, tables, ctxs, case["window"], case["scale"])
    np.testing.assert_allclose(bf, np.asarray(case["expected"]), rtol=0, atol=case["tol"])


def test_golden_cache_write():
    with open(os.path.join(GOLDEN, "cache_write_hand.json")) as f:
        g = json.load(f)
    B, NB, Hkv, D = g["block_size"], g["num_blocks"], g["num_kv_heads"], g["head_dim"]
    rng = np.random.default_rng(0)
    pool = rng.standard_normal((1, NB, 2, B, Hkv, D)).astype(np.float32)
    T = len(g["slots"])
    k_new = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    v_new = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    out = oracle.cache_write(pool, 0, k_new, v_new, np.array(g["slots"], dtype=np.int32))
    expect = pool.copy()
    for t, bo in enumerate(g["expected_block_offset"]):
        if bo is None:
            continue
        expect[0, bo[0], 0, bo[1]] = k_new[t]
        expect[0, bo[0], 1, bo[1]] = v_new[t]
    assert out.tobytes() == expect.tobytes()
    assert pool.tobytes() != out.tobytes()  # the input is left alone, the copy changed


# ---------------------------------------------------------------------------
# brute force and an independent library routine


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("window", [0, 20])
@pytest.mark.parametrize("G", [1, 4])
def test_bruteforce_tiny(dtype, window, G):
    w = tiny_random(3 + G, dtype=dtype, window=window, G=G)
    a = oracle.decode_attention(w.pool, 0, w.q, w.block_tables, w.seq_lens, w.window, w.scale)
    b = oracle.decode_attention_bruteforce(w.pool, 0, w.q, w.block_tables, w.seq_lens, w.window, w.scale)
    assert np.all(np.isfinite(a))
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_bruteforce_config1():
    w = W.make(1)
    a = oracle.decode_attention(w.pool, 0, w.q, w.block_tables, w.seq_lens, 0, w.scale)
    b = oracle.decode_attention_bruteforce(w.pool, 0, w.q, w.block_tables, w.seq_lens, 0, w.scale)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


@pytest.mark.parametrize("window", [0, 24])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sdpa_crosscheck(window, dtype):
    w = W.custom(21, [1, 7, 16, 31, 32, 50, 95], num_q_heads=8, num_kv_heads=2, head_dim=16,
                 dtype=dtype, window=window)
    a = oracle.decode_attention(w.pool, 0, w.q, w.block_tables, w.seq_lens, w.window, w.scale)
    ref = sdpa_reference(w.pool, 0, w.q, w.block_tables, w.seq_lens, w.window, w.scale)
    np.testing.assert_allclose(a, ref, rtol=0, atol=1e-12)


def test_sdpa_crosscheck_config1():
    w = W.make(1)
    a = oracle.decode_attention(w.pool, 0, w.q, w.block_tables, w.seq_lens, 0, w.scale)
    ref = sdpa_reference(w.pool, 0, w.q, w.block_tables, w.seq_lens, 0, w.scale)
    np.testing.assert_allclose(a, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# closed forms


def test_single_key_returns_its_value():
    w = tiny_random(5, ctx=(1, 1, 1))
    out = oracle.decode_attention(w.pool, 0, w.q, w.block_tables, w.seq_lens, 0, w.scale)
    G = w.num_q_heads // w.num_kv_heads
    for s in range(w.num_seqs):
        blk = w.block_tables[s, 0]
        for h in range(w.num_q_heads):
            assert np.array_equal(out[s, h], widen(w.pool[0, blk, 1, 0, h // G]))


def test_zero_query_gives_mean_value():
    w = tiny_random(6, ctx=(3, 16, 40))
    q0 = np.zeros_like(w.q)
    out = oracle.decode_attention(w.pool, 0, q0, w.block_tables, w.seq_lens, 0, w.scale)
    G = w.num_q_heads // w.num_kv_heads
    for s in range(w.num_seqs):
        _, V = independent_gather(w.pool, 0, w.block_tables[s], int(w.seq_lens[s]), 0)
        for h in range(w.num_q_heads):
            np.testing.assert_allclose(out[s, h], V[:, h // G].mean(axis=0), rtol=0, atol=1e-14)


def test_constant_values_give_that_constant():
    w = tiny_random(7, ctx=(2, 17, 48))
    pool = w.pool.copy()
    pool[:, :, 1] = np.float32(0.375)
    out = oracle.decode_attention(pool, 0, w.q, w.block_tables, w.seq_lens, 0, w.scale)
    np.testing.assert_allclose(out, 0.375, rtol=0, atol=1e-15)


def test_needle_selects_one_value():
    """q_g = 32 e_g and K[t*] = 32 e_g give that key a score margin of
    1024/sqrt(D) over keys near zero; the output is the needle's value."""
    w = tiny_random(8, ctx=(40,), G=2, D=8)
    pool = w.pool.copy()
    q = np.zeros_like(w.q)
    blk, off = w.block_tables[0, 1], 7  # position 23
    pool[0, :, 0] = np.where(np.isnan(pool[0, :, 0]), pool[0, :, 0], 0.0)
    for h in range(w.num_q_heads):
        q[0, h, h % w.head_dim] = 32.0
    for kv in range(w.num_kv_heads):
        pool[0, blk, 0, off, kv] = 0.0
        for g in range(2):
            pool[0, blk, 0, off, kv, (2 * kv + g) % w.head_dim] = 32.0
    out = oracle.decode_attention(pool, 0, q, w.block_tables, w.seq_lens, 0, 1.0)
    for h in range(w.num_q_heads):
        np.testing.assert_allclose(out[0, h], widen(pool[0, blk, 1, off, h // 2]), rtol=0, atol=1e-300)


# ---------------------------------------------------------------------------
# invariants


def relabel(w, seed):
    """Move every block to a new physical id and rewrite the tables."""
    rng = np.random.default_rng(seed)
    pi = rng.permutation(w.num_blocks)
    pool = np.empty_like(w.pool)
    pool[:, pi] = w.pool
    return pool, pi[w.block_tables].astype(np.int32)


@pytest.mark.parametrize("window", [0, 20])
def test_permutation_invariance(window):
    w = tiny_random(9, dtype="bf16", window=window, ctx=(3, 16, 17, 45, 64))
    a = oracle.decode_attention(w.pool, 0, w.q, w.block_tables, w.seq_lens, w.window, w.scale)
    pool2, tables2 = relabel(w, 1)
    b = oracle.decode_attention(pool2, 0, w.q, tables2, w.seq_lens, w.window, w.scale)
    assert a.tobytes() == b.tobytes()


def test_shared_prefix_aliasing():
    """Sequences whose prefix blocks are one physical block give bit-identical
    results to the same data stored in private copies."""
    B = 16
    rng = np.random.default_rng(4)
    Hkv, D, Hq = 2, 8, 4
    pre, tails = 3, [5, 17, 30]
    NB = pre + sum(-(-t // B) for t in tails) + pre * len(tails)
    pool = W.f32_to_bf16_bits(rng.standard_normal((1, NB, 2, B, Hkv, D)))
    shared = list(range(pre))
    rows_shared, rows_priv, nxt = [], [], pre
    for t in tails:
        own = list(range(nxt, nxt + -(-t // B)))
        nxt += len(own)
        copies = list(range(nxt, nxt + pre))
        nxt += pre
        pool[:, copies] = pool[:, shared]
        rows_shared.append(shared + own)
        rows_priv.append(copies + own)
    width = max(len(r) for r in rows_shared)
    t1 = np.zeros((len(tails), width), np.int32)
    t2 = np.zeros((len(tails), width), np.int32)
    for i, (a, b) in enumerate(zip(rows_shared, rows_priv)):
        t1[i, : len(a)] = a
        t2[i, : len(b)] = b
    ctx = np.array([pre * B + t for t in tails], np.int32)
    q = W.f32_to_bf16_bits(rng.standard_normal((len(tails), Hq, D)))
    a = oracle.decode_attention(pool, 0, q, t1, ctx, 0, 0.25)
    b = oracle.decode_attention(pool, 0, q, t2, ctx, 0, 0.25)
    assert a.tobytes() == b.tobytes()


def test_softmax_rows_sum_to_one():
    w = tiny_random(10, ctx=(1, 9, 33, 70))
    G = w.num_q_heads // w.num_kv_heads
    for s in range(w.num_seqs):
        K, _ = oracle.gather_kv(w.pool, 0, w.block_tables[s], 0, int(w.seq_lens[s]))
        for h in range(w.num_q_heads):
            p = oracle.softmax_weights(widen(w.q[s, h]), K[:, h // G], w.scale)
            assert abs(p.sum() - 1.0) <= 1e-15
            assert np.all(p >= 0)


def test_gqa_consistency():
    w = tiny_random(11, G=4, ctx=(5, 33))
    G = 4
    q = w.q.copy()
    for kv in range(w.num_kv_heads):
        q[:, kv * G:(kv + 1) * G] = q[:, kv * G][:, None]
    out = oracle.decode_attention(w.pool, 0, q, w.block_tables, w.seq_lens, 0, w.scale)
    for kv in range(w.num_kv_heads):
        for g in range(1, G):
            assert out[:, kv * G + g].tobytes() == out[:, kv * G].tobytes()
    # G = 1 with the KV heads repeated equals the grouped result
    pool_mha = np.repeat(w.pool, G, axis=4)
    mha = oracle.decode_attention(pool_mha, 0, q, w.block_tables, w.seq_lens, 0, w.scale)
    assert mha.tobytes() == out.tobytes()


@pytest.mark.parametrize("config", [1, 2, 4, 5])
def test_generated_tables_are_well_formed(config):
    w = W.make(config)
    oracle.check_tables(w.block_tables, w.seq_lens, w.window, w.block_size, w.num_blocks, w.row_blocks)
    if w.block_tables_after is not None:
        oracle.check_tables(w.block_tables_after, w.seq_lens_after, 0, w.block_size,
                            w.num_blocks, w.row_blocks_after)


def test_table_rule_rejects_malformed_rows():
    ok = np.array([[3, 1, 2]], np.int32)
    oracle.check_tables(ok, [40], 0, 16, 8)
    with pytest.raises(ValueError):
        oracle.check_tables(np.array([[3, 3, 2]], np.int32), [40], 0, 16, 8)  # repeated id
    with pytest.raises(ValueError):
        oracle.check_tables(np.array([[3, 1, 9]], np.int32), [40], 0, 16, 8)  # out of range
    with pytest.raises(ValueError):
        oracle.check_tables(ok, [40], 0, 16, 8, row_blocks=[2])  # wrong length
    with pytest.raises(ValueError):
        oracle.check_tables(np.array([[3, 1]], np.int32), [40], 0, 16, 8)  # too short


def test_row_span_examples():
    # decode rule: 16 tokens fill one block, the 17th needs a second
    assert oracle.row_span(16, 0, 16) == (0, 16, 1)
    assert oracle.row_span(17, 0, 16) == (0, 17, 2)
    # window 4096 at context 5000: positions 904..4999, first block 56, offset 8
    assert oracle.row_span(5000, 4096, 16) == (904 % 16, 4096, -(-(8 + 4096) // 16))
    assert oracle.row_span(4096 + 16, 4096, 16) == (0, 4096, 256)
    assert oracle.row_span(0, 0, 16) == (0, 0, 0)


# ---------------------------------------------------------------------------
# cache write invariants


def test_cache_write_skips_negative_and_is_idempotent():
    w = W.make(1)
    slots = w.slot_mapping.copy()
    slots[1] = -1
    a = oracle.cache_write(w.pool, 0, w.k_new, w.v_new, slots)
    b = oracle.cache_write(a, 0, w.k_new, w.v_new, slots)
    assert a.tobytes() == b.tobytes()
    B = w.block_size
    diff = a.view(np.uint32) != w.pool.view(np.uint32)  # bitwise, so NaN == NaN
    changed = np.argwhere(np.any(diff, axis=(2, 4, 5)))
    expect = {(0, int(s) // B, int(s) % B) for s in slots if s >= 0}
    assert {tuple(map(int, c)) for c in changed} == expect


def test_cache_write_then_attend_matches_contiguous():
    """Write the next token of every config-1 sequence, then attend over
    ctx+1 keys: equals SDPA over the contiguous K/V with the new token last."""
    w = W.make(1)
    pool = oracle.cache_write(w.pool, 0, w.k_new, w.v_new, w.slot_mapping)
    out = oracle.decode_attention(pool, 0, w.q, w.block_tables_after, w.seq_lens_after, 0, w.scale)
    Hq, D = w.num_q_heads, w.head_dim
    G = Hq // w.num_kv_heads
    for s in range(w.num_seqs):
        K, V = independent_gather(w.pool, 0, w.block_tables[s], int(w.seq_lens[s]), 0)
        K = np.concatenate([K, widen(w.k_new[s])[None]], axis=0)
        V = np.concatenate([V, widen(w.v_new[s])[None]], axis=0)
        qt = torch.from_numpy(widen(w.q[s])).reshape(1, Hq, 1, D)
        kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, 0).unsqueeze(0).contiguous()
        vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, 0).unsqueeze(0).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=w.scale)
        np.testing.assert_allclose(out[s], ref.reshape(Hq, D).numpy(), rtol=0, atol=1e-12)


def test_copy_blocks_hand_values():
    """Each value names its own (layer, block, kv) place, so after the copy
    block 5 must read as block 2 and block 3 as block 0 in every layer; the
    out-of-range pair and the src == dst pair change nothing."""
    L, NB, B, Hkv, D = 2, 8, 16, 2, 4
    pool = np.zeros((L, NB, 2, B, Hkv, D), dtype=np.float32)
    for l in range(L):
        for b in range(NB):
            for kv in range(2):
                pool[l, b, kv] = 1000 * l + 10 * b + kv
    out = oracle.copy_blocks(pool, [2, 0, 9, 4], [5, 3, 1, 4])
    src_of = {5: 2, 3: 0}
    for l in range(L):
        for b in range(NB):
            for kv in range(2):
                assert np.all(out[l, b, kv] == 1000 * l + 10 * src_of.get(b, b) + kv)
    assert pool[0, 5, 0, 0, 0, 0] == 50  # the input is not modified


def test_copy_on_write_then_append_matches_private_history():
    """Two sequences share a partially filled last block ([Optimizing]
    Copy-on-Write: parallel samples share blocks until one writes).  The
    writer gets a copy of the shared block, its table is repointed, and its
    new token goes into the copy: its attention then equals attention over
    its own contiguous history, and the other sequence's is unchanged."""
    rng = np.random.default_rng(7)
    B, Hkv, D, Hq = 16, 2, 8, 4
    NB = 6
    pool = np.full((1, NB, 2, B, Hkv, D), np.nan, dtype=np.float32)
    ctx = 20  # blocks [1, 4]; block 4 holds 4 tokens, shared by both sequences
    hist = rng.standard_normal((2, ctx, Hkv, D)).astype(np.float32)
    for i in range(ctx):
        blk = [1, 4][i // B]
        pool[0, blk, :, i % B] = hist[:, i]
    k_new = rng.standard_normal((1, Hkv, D)).astype(np.float32)
    v_new = rng.standard_normal((1, Hkv, D)).astype(np.float32)
    q = rng.standard_normal((2, Hq, D)).astype(np.float32)
    # copy-on-write: sequence 0 gets block 2, a copy of block 4, then appends
    pool2 = oracle.copy_blocks(pool, [4], [2])
    pool2 = oracle.cache_write(pool2, 0, k_new, v_new, np.array([2 * B + ctx % B], dtype=np.int32))
    tables = np.array([[1, 2], [1, 4]], dtype=np.int32)
    lens = np.array([ctx + 1, ctx], dtype=np.int32)
    out = oracle.decode_attention(pool2, 0, q, tables, lens, 0, 0.5)
    G = Hq // Hkv
    for s, (K, V) in enumerate([
            (np.concatenate([hist[0], k_new]), np.concatenate([hist[1], v_new])),
            (hist[0], hist[1])]):
        qt = torch.from_numpy(widen(q[s])).reshape(1, Hq, 1, D)
        kt = torch.from_numpy(widen(K)).permute(1, 0, 2).repeat_interleave(G, 0).unsqueeze(0).contiguous()
        vt = torch.from_numpy(widen(V)).permute(1, 0, 2).repeat_interleave(G, 0).unsqueeze(0).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.5)
        np.testing.assert_allclose(out[s], ref.reshape(Hq, D).numpy(), rtol=0, atol=1e-12)
    # the shared block itself is untouched
    assert pool2[0, 4].tobytes() == pool[0, 4].tobytes()


# ---------------------------------------------------------------------------
# planted mistakes: each must fail a pin that does not use the oracle's own code


def _mutant(kind):
    def seq_fn(pool, layer, q_seq, table_row, ctx, window, scale, heads=None):
        q = op.to_f64(q_seq)
        Hq, D = q.shape
        Hkv = pool.shape[4]
        G = Hq // Hkv
        B = pool.shape[3]
        start_off, n, _ = op.row_span(int(ctx), window, B)
        if kind == "window_off_by_one" and window > 0 and ctx > window:
            start_off, n = start_off - 1 if start_off > 0 else start_off, n + 1
        if kind == "drop_last_block":
            n = max(0, min(n, ((start_off + n - 1) // B) * B - start_off))
        out = np.zeros((Hq, D))
        if n == 0:
            return out
        K, V = op.gather_kv(pool, layer, table_row, start_off, n)
        if kind == "swap_kv":
            K, V = V, K
        if kind == "reverse_table":
            nb = -(-(start_off + n) // B)
            K, V = op.gather_kv(pool, layer, list(table_row[:nb])[::-1], start_off, n)
        for h in range(Hq):
            kv = h % Hkv if kind == "head_modulo" else h // G
            z = K[:, kv] @ q[h] * (1.0 if kind == "no_scale" else scale)
            if kind == "flip_sign":
                z = -z
            e = np.exp(z - z.max())
            p = e if kind == "no_normalise" else e / e.sum()
            out[h] = p @ V[:, kv]
        return out

    def attn(pool, layer, q, tables, seq_lens, window, scale):
        out = np.zeros(q.shape)
        for s in range(q.shape[0]):
            out[s] = seq_fn(pool, layer, q[s], tables[s], int(seq_lens[s]), window, scale)
        return out

    return attn


def _independent_pins_pass(attn):
    if not golden_ok(attn):
        return False
    for window in (0, 24):
        w = W.custom(31, [3, 16, 31, 50], num_q_heads=8, num_kv_heads=2, head_dim=16,
                     dtype="bf16", window=window)
        a = attn(w.pool, 0, w.q, w.block_tables, w.seq_lens, w.window, w.scale)
        ref = sdpa_reference(w.pool, 0, w.q, w.block_tables, w.seq_lens, w.window, w.scale)
        if not np.allclose(a, ref, rtol=0, atol=1e-9):
            return False
    return True


def test_pins_pass_for_the_oracle():
    assert _independent_pins_pass(oracle.decode_attention)


@pytest.mark.parametrize("kind", ["window_off_by_one", "drop_last_block", "swap_kv", "reverse_table",
                                  "head_modulo", "no_scale", "flip_sign", "no_normalise"])
def test_planted_mistake_is_caught(kind):
    assert not _independent_pins_pass(_mutant(kind))


# ---------------------------------------------------------------------------
# the oracle's widening of stored elements, against torch's own dtypes


def test_bf16_widening_of_every_pattern():
    """All 65,536 bf16 bit patterns widen to the float64 value torch gives
    the same bits as a torch.bfloat16 (NaN patterns to NaN)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns stay NaN when widened
        got = op.to_f64(bits)
    want = widen(bits)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))  # -0.0 stays negative


def test_e4m3_widening_of_every_code():
    """All 256 E4M3 codes widen to the value torch gives them as
    torch.float8_e4m3fn (the OCP format with no infinities)."""
    codes = np.arange(256, dtype=np.uint8)
    got, want = op.to_f64(codes), widen(codes)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2  # S.1111.111
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def _widen_mutant(kind):
    real = op.to_f64

    def to_f64(x):
        x = np.asarray(x)
        if x.dtype != np.uint16:
            return real(x)
        if kind == "shift_15":
            return (x.astype(np.uint32) << 15).view(np.float32).astype(np.float64)
        if kind == "as_fp16":
            return x.view(np.float16).astype(np.float64)
        if kind == "bytes_swapped":
            return real(x.byteswap())
        raise ValueError(kind)

    return to_f64


@pytest.mark.parametrize("kind", ["shift_15", "as_fp16", "bytes_swapped"])
def test_planted_widening_mistake_is_caught(kind, monkeypatch):
    """A slip in how the oracle reads bf16 bits must fail a pin that reads
    them another way: the golden bf16-pattern case and the SDPA
    cross-check, whose gather widens through torch."""
    monkeypatch.setattr(op, "to_f64", _widen_mutant(kind))
    assert not _independent_pins_pass(oracle.decode_attention)


# ---------------------------------------------------------------------------
# FP8 (E4M3) codes: pinned to the format's definition by worked values, not
# by re-running the oracle's own formula


def test_e4m3_known_codes():
    """Values of E4M3 codes worked out by hand from the field layout (sign,
    exponent bias 7, 3 mantissa bits, subnormals at exponent field 0)."""
    known = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x0F: 1.875 * 2.0 ** -6,
             0x30: 0.5, 0x38: 1.0, 0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x48: 4.0, 0x7E: 448.0,
             0xB8: -1.0, 0xC0: -2.0, 0xFE: -448.0}
    vals = oracle.e4m3_decode(np.array(list(known), dtype=np.uint8))
    assert list(vals) == list(known.values())
    neg_zero = oracle.e4m3_decode(np.array([0x80], np.uint8))[0]
    assert neg_zero == 0.0 and np.signbit(neg_zero)
    assert np.all(np.isnan(oracle.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))))
    pos = oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)  # codes 0..0x7E are the positive values in order


def test_e4m3_encode_rounding_and_saturation():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    finite = ~np.isnan(vals)
    assert np.all(oracle.e4m3_encode(vals[finite]) == codes[finite])  # every code is its own nearest
    # midpoints of consecutive positive codes go to the code with the even mantissa;
    # a hair either side goes to the nearer one
    for c in range(0, 0x7E):
        lo, hi = vals[c], vals[c + 1]
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(mid) == even, hex(c)
        assert oracle.e4m3_encode(np.nextafter(mid, 0)) == c
        assert oracle.e4m3_encode(np.nextafter(mid, np.inf)) == c + 1
        assert oracle.e4m3_encode(-mid) == (even | 0x80)
    # beyond the largest code: saturate
    for x, c in ((448.0, 0x7E), (460.0, 0x7E), (464.0, 0x7E), (1e6, 0x7E), (np.inf, 0x7E), (-1e9, 0xFE)):
        assert oracle.e4m3_encode(x) == c, x
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00       # tie between 0 and 2^-9: even
    assert oracle.e4m3_encode(0.75 * 2.0 ** -9) == 0x01
    assert oracle.e4m3_encode(-2.0 ** -12) == 0x80      # rounds to -0


def test_fp8_quantize_uses_float32_product():
    """quantize(x, s) encodes the float32 product x * float32(1/s): for s = 3,
    1/s is not exact in float32 and 3 * fl(1/3) rounds to exactly 1."""
    bits = W.f32_to_bf16_bits(np.array([3.0, 6.0, -0.75], dtype=np.float32))
    assert list(oracle.quantize(bits, 3.0)) == [0x38, 0x40, 0xA8]   # 1.0, 2.0, -0.25
    assert list(oracle.quantize(np.array([896.0], np.float32), 1.0)) == [0x7E]


def test_fp8_cache_write_then_attend():
    """An FP8 pool: the write stores quantized codes, attention reads codes
    times the layer's scales; equals SDPA over the dequantized history."""
    rng = np.random.default_rng(11)
    B, Hkv, D, Hq = 16, 2, 16, 4
    pool = np.full((1, 4, 2, B, Hkv, D), 0x7F, dtype=np.uint8)
    codes = rng.integers(0, 0x7E, size=(2, 20, Hkv, D), dtype=np.uint8) | (rng.integers(0, 2, (2, 20, Hkv, D), dtype=np.uint8) << 7)
    for i in range(20):
        pool[0, [2, 0][i // B], :, i % B] = codes[:, i]
    k_new = W.f32_to_bf16_bits(rng.standard_normal((1, Hkv, D)).astype(np.float32))
    v_new = W.f32_to_bf16_bits(rng.standard_normal((1, Hkv, D)).astype(np.float32))
    ks, vs = 0.37, 1.9
    pool2 = oracle.cache_write(pool, 0, k_new, v_new, np.array([0 * B + 20 % B], np.int32), ks, vs)
    assert np.all(pool2[0, 0, 0, 4] == oracle.quantize(k_new[0], ks))
    assert np.all(pool2[0, 0, 1, 4] == oracle.quantize(v_new[0], vs))
    q = rng.standard_normal((1, Hq, D)).astype(np.float32)
    out = oracle.decode_attention(pool2, 0, q, np.array([[2, 0]], np.int32), np.array([21], np.int32), 0, 0.25,
                                  k_scale=ks, v_scale=vs)
    K = np.concatenate([oracle.e4m3_decode(codes[0]), oracle.e4m3_decode(oracle.quantize(k_new, ks))]) * ks
    V = np.concatenate([oracle.e4m3_decode(codes[1]), oracle.e4m3_decode(oracle.quantize(v_new, vs))]) * vs
    G = Hq // Hkv
    qt = torch.from_numpy(q[0].astype(np.float64)).reshape(1, Hq, 1, D)
    kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, 0).unsqueeze(0).contiguous()
    vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, 0).unsqueeze(0).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.25)
    np.testing.assert_allclose(out[0], ref.reshape(Hq, D).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("kind", ["ties_away", "truncate", "bias8", "no_saturation"])
def test_planted_fp8_mistake_is_caught(kind):
    """Plausible mistakes in an E4M3 encoder each break a worked value."""
    def mutant(x):
        x = np.asarray(x, dtype=np.float64)
        if kind == "bias8":  # the variant with exponent bias 8 halves every value
            return oracle.e4m3_encode(x * 2.0)
        if kind == "no_saturation":
            c = oracle.e4m3_encode(x)
            return np.where(np.abs(x) > 448, 0x7F, c).astype(np.uint8)
        a = np.abs(x)
        _, E = np.frexp(a)
        e = np.maximum(E - 1, -6)
        q = np.ldexp(1.0, e - 3)
        m = np.floor(a / q + 0.5) if kind == "ties_away" else np.floor(a / q)
        return oracle.e4m3_encode(np.copysign(m * q, x))
    vals = oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    even = np.array([c if c % 2 == 0 else c + 1 for c in range(0x7E)], dtype=np.uint8)
    ok_ties = np.all(mutant(mids) == even)
    ok_sat = mutant(1e6) == 0x7E
    ok_known = mutant(1.0) == 0x38
    ok_above = np.all(mutant(np.nextafter(mids, np.inf)) == np.arange(1, 0x7F, dtype=np.uint8))
    assert not (ok_ties and ok_sat and ok_known and ok_above)


# ---------------------------------------------------------------------------
# 32-token blocks ([Optimizing] Trade-offs of Block Size Tuning): the block
# size changes where a key lives, never which keys are attended


def _relaid(w16, B):
    """The same sequences' K/V in a pool of B-token blocks: each sequence's
    attended positions copied, in order, into fresh blocks of the new pool
    (ids a seeded permutation), with tables listing them."""
    rng = np.random.default_rng(77)
    rows, per = [], []
    for s in range(w16.num_seqs):
        ctx = int(w16.seq_lens[s])
        first = max(0, ctx - w16.window) if w16.window else 0
        fb, lb = first // B, (ctx - 1) // B if ctx else -1
        per.append((first, fb, lb - fb + 1 if ctx else 0))
    NB = sum(n for _, _, n in per) + 2
    ids = rng.permutation(NB).astype(np.int32)
    pool = np.empty((1, NB, 2, B) + w16.pool.shape[4:], dtype=w16.pool.dtype)
    pool[:] = W.BF16_NAN if pool.dtype == np.uint16 else np.nan
    tables = np.full((w16.num_seqs, max(n for _, _, n in per) + 1), ids[-1], dtype=np.int32)
    k = 0
    for s, (first, fb, n) in enumerate(per):
        ctx = int(w16.seq_lens[s])
        tables[s, :n] = ids[k:k + n]
        for pos in range(first, ctx):
            blk = ids[k + pos // B - fb]
            src16 = w16.block_tables[s][pos // 16 - first // 16]
            pool[0, blk, 0, pos % B] = w16.pool[0, src16, 0, pos % 16]
            pool[0, blk, 1, pos % B] = w16.pool[0, src16, 1, pos % 16]
        k += n
    return pool, tables


@pytest.mark.parametrize("window", [0, 20, 40, 100])
def test_block_size_32_is_a_relabelling(window):
    """The same keys in 32-token blocks give bit-identical oracle outputs;
    windows whose first position lies in a block's second half (40 at
    contexts 57 and 95: first positions 17 and 55) included."""
    w = W.custom(31, [1, 15, 16, 17, 31, 32, 33, 57, 64, 95, 200], num_q_heads=8, num_kv_heads=2, head_dim=16,
                 dtype="bf16", window=window)
    a = oracle.decode_attention(w.pool, 0, w.q, w.block_tables, w.seq_lens, w.window, w.scale)
    pool32, tables32 = _relaid(w, 32)
    oracle.check_tables(tables32, w.seq_lens, w.window, 32, pool32.shape[1])
    b = oracle.decode_attention(pool32, 0, w.q, tables32, w.seq_lens, w.window, w.scale)
    assert a.tobytes() == b.tobytes()
    c = oracle.decode_attention_bruteforce(pool32, 0, w.q, tables32, w.seq_lens, w.window, w.scale)
    np.testing.assert_allclose(b, c, rtol=0, atol=1e-12)


def test_block_size_32_generated_workloads():
    """Generated 32-token workloads keep the table rule and match the
    independent per-position gather through SDPA."""
    w = W.custom(32, [1, 31, 32, 33, 70, 130], num_q_heads=8, num_kv_heads=4, head_dim=16, window=48,
                 block_size=32)
    assert w.pool.shape[3] == 32
    oracle.check_tables(w.block_tables, w.seq_lens, w.window, 32, w.num_blocks, w.row_blocks)
    a = oracle.decode_attention(w.pool, 0, w.q, w.block_tables, w.seq_lens, w.window, w.scale)
    ref = sdpa_reference(w.pool, 0, w.q, w.block_tables, w.seq_lens, w.window, w.scale)
    np.testing.assert_allclose(a, ref, rtol=0, atol=1e-12)
    # row spans in 32-token blocks: context 70 under window 48 attends 22..69,
    # blocks 0..2, the first 22 slots of block 0 unattended
    assert oracle.row_span(70, 48, 32) == (22, 48, 3)
    assert oracle.row_span(33, 0, 32) == (0, 33, 2)


def test_block_size_32_cache_write():
    """slot = block * 32 + offset: the write lands at block slot // 32,
    offset slot % 32, and attention then sees it as the last key."""
    w = W.custom(33, [31, 32, 40], num_q_heads=4, num_kv_heads=2, head_dim=16, block_size=32)
    W.with_next_token(w, w.unused_blocks)
    assert [int(s) % 32 for s in w.slot_mapping] == [31, 0, 8]
    pool = oracle.cache_write(w.pool, 0, w.k_new, w.v_new, w.slot_mapping)
    for t, slot in enumerate(w.slot_mapping):
        assert np.array_equal(pool[0, slot // 32, 0, slot % 32], w.k_new[t])
        assert np.array_equal(pool[0, slot // 32, 1, slot % 32], w.v_new[t])
    out = oracle.decode_attention(pool, 0, w.q, w.block_tables_after, w.seq_lens_after, 0, w.scale)
    ref = sdpa_reference(pool, 0, w.q, w.block_tables_after, w.seq_lens_after, 0, w.scale)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
