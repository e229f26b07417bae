"""Seeded random sweep of the GPU paths against the oracle: each case draws
a batch shape (sequences, lengths with block-edge values mixed in, head
group, head_dim, window, pool dtype, block size) and checks decode
attention (default variant), the fused write-then-attend step (pool
bit-exact) and a chunked prefill over the same kind of batch; shared-prefix
batches (prefix length, tails, heads, pool dtype, block size) check the
cascade against the oracle and against plain decode.  The cases
are small enough for the fp64 oracle and vary what the fixed tests hold
apart.  KVP_RANDOM_DECODE_CASES and KVP_RANDOM_PREFILL_CASES raise the case
counts (16 and 12 by default) for a longer sweep, KVP_RANDOM_CASCADE_CASES
that of the shared-prefix batches (12)."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import (SHARP_C, Dev, compare, host_to_torch, pool_dtype, reference, say, to_f64, torch_dtype,
                         torch_to_bits, ulp_bf16)
from paged_kv_cache_37_amd.blockpool import shared_prefix_blocks

pytestmark = pytest.mark.gpu

N_DECODE = int(os.environ.get("KVP_RANDOM_DECODE_CASES", "16"))
N_PREFILL = int(os.environ.get("KVP_RANDOM_PREFILL_CASES", "12"))
N_CASCADE = int(os.environ.get("KVP_RANDOM_CASCADE_CASES", "12"))
EDGES = [1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 255, 256, 257]


def draw(seed):
    rng = np.random.default_rng(10_000 + seed)
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 5, 8, 16]))
    D = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "bf16", "fp8"]))
    B = int(rng.choice([16, 32]))
    S = int(rng.integers(1, 24))
    lens = [int(rng.choice(EDGES)) if rng.random() < 0.4 else int(rng.integers(0, 2500)) for _ in range(S)]
    window = int(rng.choice([0, 0, 0, int(rng.integers(1, 600))]))
    return dict(Hkv=Hkv, Hq=Hkv * G, D=D, dtype=dtype, B=B, lens=lens, window=window)


@pytest.mark.parametrize("seed", range(N_DECODE))
def test_random_decode_and_step(gpu, seed):
    c = draw(seed)
    say("random decode", seed, {k: v for k, v in c.items() if k != "lens"}, "S", len(c["lens"]))
    w = W.custom(20_000 + seed, c["lens"], num_q_heads=c["Hq"], num_kv_heads=c["Hkv"], head_dim=c["D"],
                 dtype=c["dtype"], window=c["window"], block_size=c["B"])
    dev = Dev(w)
    compare(dev.attend(), reference(w), "bf16", f"random decode {seed}")
    # the fused step: each sequence's next token written and attended
    if len(w.unused_blocks) >= len(c["lens"]):
        W.with_next_token(w, w.unused_blocks)
        dt = torch_dtype(w)
        out = dev.ops.paged_decode_step(dev.pool, 0, dev.q, torch.from_numpy(np.ascontiguousarray(w.block_tables_after)).cuda(),
                                        torch.from_numpy(w.seq_lens_after).cuda(), w.scale,
                                        host_to_torch(w.k_new, dt).cuda(), host_to_torch(w.v_new, dt).cuda(),
                                        torch.from_numpy(w.slot_mapping).cuda(), sliding_window=w.window)
        torch.cuda.synchronize()
        pool_ref = oracle.cache_write(w.pool, 0, w.k_new, w.v_new, w.slot_mapping, w.k_scale, w.v_scale)
        assert torch_to_bits(dev.pool.to_logical()).tobytes() == np.ascontiguousarray(pool_ref).tobytes()
        ref = reference(w, pool=pool_ref, tables=w.block_tables_after, lens=w.seq_lens_after)
        compare(out, ref, "bf16", f"random step {seed}")


@pytest.mark.parametrize("seed", range(N_PREFILL))
def test_random_prefill(gpu, seed):
    c = draw(seed + 100)
    rng = np.random.default_rng(30_000 + seed)
    S = min(len(c["lens"]), 8)
    prior = [int(x) for x in c["lens"][:S]]
    q_lens = [int(rng.choice([1, 16, 17, 64, 129, int(rng.integers(1, 300))])) for _ in range(S)]
    say("random prefill", seed, {k: v for k, v in c.items() if k != "lens"}, prior, q_lens)
    w = W.prefill_batch(40_000 + seed, prior, q_lens, c["Hq"], c["Hkv"], c["D"], window=c["window"],
                        dtype=c["dtype"], block_size=c["B"])
    from paged_kv_cache_37_amd import ops

    pool = ops.KVPool(1, w.num_blocks, w.num_kv_heads, w.head_dim, pool_dtype(w), "cuda:0", block_size=w.block_size)
    pool.load_logical(host_to_torch(w.pool, pool_dtype(w)))
    if w.dtype == "fp8":
        pool.set_fp8_scales(0, w.k_scale, w.v_scale)
    out = ops.paged_prefill_attention(pool, 0, host_to_torch(w.q, torch_dtype(w)).cuda(),
                                      torch.from_numpy(w.cu_q_lens).cuda(),
                                      torch.from_numpy(np.ascontiguousarray(w.block_tables)).cuda(),
                                      torch.from_numpy(np.ascontiguousarray(w.seq_lens)).cuda(), w.scale,
                                      int(max(w.q_lens)), sliding_window=w.window)
    torch.cuda.synchronize()
    ref = oracle.prefill_attention(w.pool, 0, w.q, w.cu_q_lens, w.block_tables, w.seq_lens, w.window, w.scale,
                                   k_scale=w.k_scale, v_scale=w.v_scale)
    compare(out, ref, "bf16", f"random prefill {seed}", bar="prefill")


@pytest.mark.parametrize("seed", range(N_CASCADE))
def test_random_cascade(gpu, seed):
    """A batch whose rows share a prefix of whole blocks: the cascade (the
    prefix read once per KV head beside the tails) against the oracle on
    every row and against plain decode (one bf16 step at the larger
    magnitude plus the decode sharp bar's rms term); then the fused step
    with the same hint (pool bit-exact)."""
    rng = np.random.default_rng(50_000 + seed)
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 5, 8, 16]))
    D = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "bf16", "fp8"]))
    B = int(rng.choice([16, 32]))
    S = int(rng.integers(1, 40))
    prefix = B * int(rng.integers(1, 48))
    tails = [int(rng.choice([0, 1, B - 1, B, B + 1])) if rng.random() < 0.4 else int(rng.integers(0, 3000))
             for _ in range(S)]
    say("random cascade", seed, dict(Hkv=Hkv, Hq=Hkv * G, D=D, dtype=dtype, B=B, prefix=prefix), "S", S)
    w = W.shared_prefix(60_000 + seed, prefix, tails, Hkv * G, Hkv, D, dtype=dtype, block_size=B)
    P = shared_prefix_blocks(np.asarray(w.block_tables), w.seq_lens, block_size=B)
    assert P >= prefix // B
    dev = Dev(w)
    out_c = dev.attend(shared_prefix_blocks=P)
    out_p = dev.attend()
    ref = reference(w)
    compare(out_c, ref, "bf16", f"random cascade {seed}")
    a, b = to_f64(out_c), to_f64(out_p)
    rms = np.sqrt(np.mean(b ** 2, axis=-1, keepdims=True))
    bound = ulp_bf16(np.maximum(np.abs(a), np.abs(b))) * 1.0001 + SHARP_C["decode"] * rms
    worst = float((np.abs(a - b) / bound).max())
    say(f"random cascade {seed} vs plain: worst", round(worst, 3), "of the bar")
    assert worst <= 1.0
    if len(w.unused_blocks) >= S:
        W.with_next_token(w, w.unused_blocks)
        dt = torch_dtype(w)
        out = dev.ops.paged_decode_step(dev.pool, 0, dev.q, torch.from_numpy(np.ascontiguousarray(w.block_tables_after)).cuda(),
                                        torch.from_numpy(w.seq_lens_after).cuda(), w.scale,
                                        host_to_torch(w.k_new, dt).cuda(), host_to_torch(w.v_new, dt).cuda(),
                                        torch.from_numpy(w.slot_mapping).cuda(), shared_prefix_blocks=P)
        torch.cuda.synchronize()
        pool_ref = oracle.cache_write(w.pool, 0, w.k_new, w.v_new, w.slot_mapping, w.k_scale, w.v_scale)
        assert torch_to_bits(dev.pool.to_logical()).tobytes() == np.ascontiguousarray(pool_ref).tobytes()
        ref = reference(w, pool=pool_ref, tables=w.block_tables_after, lens=w.seq_lens_after)
        compare(out, ref, "bf16", f"random cascade step {seed}")
