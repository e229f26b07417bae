"""GPU parity of the decode step with its new-token write (paged_decode_step)
and of the copy-on-write block copy (kv_pool_copy_blocks), through the
C-ABI, against the CPU oracle and against the unfused calls.

paged_decode_step must leave the pool and the outputs bit-identical to
cache_write followed by paged_decode_attention (same variant); the
attention must also match the oracle over the written pool.  Block copies
are bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import Dev, compare, host_to_torch, reference, say, torch_to_bits

pytestmark = pytest.mark.gpu

_CACHE = {}


def stepped(config):
    """A workload with one next token per sequence (tables and lengths after it)."""
    if config not in _CACHE:
        say("generating config", config)
        w = W.make(config)
        if config != 1:
            W.with_next_token(w, w.unused_blocks)
        _CACHE[config] = w
    return _CACHE[config]


def custom_stepped(seed, ctx, Hq, Hkv, D=128, window=0, dtype="bf16"):
    w = W.custom(seed, list(ctx), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, dtype=dtype, window=window)
    W.with_next_token(w, w.unused_blocks)
    return w


def run_both(w, variant, slots=None, lens=None, tables=None, partition_tokens=0):
    """(fused outputs, fused pool bits, unfused outputs, unfused pool bits)."""
    slots = w.slot_mapping if slots is None else slots
    lens = w.seq_lens_after if lens is None else lens
    tables = w.block_tables_after if tables is None else tables
    res = []
    for fused in (True, False):
        dev = Dev(w)
        dt = dev.dt
        k = host_to_torch(w.k_new, dt).cuda()
        v = host_to_torch(w.v_new, dt).cuda()
        sl = torch.from_numpy(np.ascontiguousarray(slots)).cuda()
        tb = torch.from_numpy(np.ascontiguousarray(tables)).cuda()
        ln = torch.from_numpy(np.ascontiguousarray(lens)).cuda()
        if fused:
            out = dev.ops.paged_decode_step(dev.pool, 0, dev.q, tb, ln, w.scale, k, v, sl,
                                            sliding_window=w.window, variant=variant,
                                            partition_tokens=partition_tokens)
        else:
            dev.ops.cache_write(dev.pool, 0, k, v, sl)
            out = dev.ops.paged_decode_attention(dev.pool, 0, dev.q, tb, ln, w.scale, sliding_window=w.window,
                                                 variant=variant, partition_tokens=partition_tokens)
        torch.cuda.synchronize()
        res += [out, torch_to_bits(dev.pool.to_logical())]
        del dev
    return res


def check_step(w, variant, what, seqs=None, partition_tokens=0, **kw):
    say("step", what, variant)
    f_out, f_pool, u_out, u_pool = run_both(w, variant, partition_tokens=partition_tokens, **kw)
    assert f_pool.tobytes() == u_pool.tobytes(), f"{what}: pool after the step differs from cache_write's"
    assert torch.equal(f_out.view(torch.int16) if f_out.dtype == torch.bfloat16 else f_out.view(torch.int32),
                       u_out.view(torch.int16) if u_out.dtype == torch.bfloat16 else u_out.view(torch.int32)), \
        f"{what}: step output differs from cache_write + attention"
    slots = np.asarray(kw.get("slots", w.slot_mapping))
    # the library skips a slot past the pool like a negative one; the oracle skips negatives
    slots = np.where(slots < w.num_blocks * 16, slots, -1).astype(np.int32)
    pool_ref = oracle.cache_write(w.pool, 0, w.k_new, w.v_new, slots, w.k_scale, w.v_scale)
    assert f_pool.tobytes() == np.ascontiguousarray(pool_ref).tobytes(), f"{what}: pool differs from the oracle"
    lens = kw.get("lens", w.seq_lens_after)
    tables = kw.get("tables", w.block_tables_after)
    ref = reference(w, pool=pool_ref, tables=tables, lens=lens, seqs=seqs)
    got = f_out if seqs is None else f_out[list(seqs)]
    compare(got, ref, w.dtype, f"{what}/{variant}")


@pytest.mark.parametrize("config", [1, 2, 4, 5])
def test_step_matches_write_then_attend(gpu, config):
    w = stepped(config)
    variants = ["valu"] if w.dtype == "f32" else ["stream", "mfma"]
    for v in variants:
        seqs = None if config in (1, 5) else list(range(0, w.num_seqs, 7))
        check_step(w, v, f"config{config}", seqs=seqs, partition_tokens=512 if v == "mfma" else 0)


@pytest.mark.parametrize("config", [2, 5])
def test_step_fp8_matches_write_then_attend(gpu, config):
    """FP8 pools: the fused step stores the new token's codes (the same
    rounding as cache_write) and attends with them."""
    w = W.make(config, dtype="fp8")
    W.with_next_token(w, w.unused_blocks)
    for v in ("stream", "mfma"):
        check_step(w, v, f"config{config}-fp8", seqs=list(range(0, w.num_seqs, 7)),
                   partition_tokens=512 if v == "mfma" else 0)


@pytest.mark.parametrize("Hq,Hkv,D,window", [(8, 2, 128, 0), (32, 1, 128, 0), (12, 4, 64, 0), (8, 2, 128, 33)])
def test_step_fp8_head_groups(gpu, Hq, Hkv, D, window):
    w = custom_stepped(320 + Hq + D + window, [1, 15, 16, 17, 31, 32, 200, 511], Hq, Hkv, D, window=window,
                       dtype="fp8")
    check_step(w, "stream", f"fp8 G{Hq // Hkv}-D{D}-W{window}")


@pytest.mark.parametrize("Hq,Hkv,D", [(8, 2, 128), (64, 8, 128), (32, 1, 128), (12, 4, 64), (48, 2, 64)])
def test_step_head_groups(gpu, Hq, Hkv, D):
    """G = 4, 8, 32 (two head groups per KV head: both patch, one writes), 3, 24."""
    w = custom_stepped(300 + Hq + D, [1, 15, 16, 17, 31, 32, 200, 511], Hq, Hkv, D)
    check_step(w, "stream", f"G{Hq // Hkv}-D{D}")


@pytest.mark.parametrize("window", [16, 33, 4096])
def test_step_sliding_window(gpu, window):
    w = custom_stepped(400 + window, [1, 15, 16, 40, 100, 4095, 4096, 5000], 8, 2, window=window)
    check_step(w, "stream", f"window{window}")


def test_step_padding_and_out_of_range_slots(gpu):
    """A negative slot: no new token (attention over the old context); a slot
    past the pool: nothing written, attention over the old context."""
    w = custom_stepped(77, [3, 16, 17, 40, 64, 100], 8, 2)
    slots = w.slot_mapping.copy()
    lens = w.seq_lens_after.copy()
    tables = w.block_tables_after.copy()
    for s, bad in ((1, -1), (4, w.num_blocks * 16 + 3)):
        slots[s] = bad
        lens[s] = w.seq_lens[s]
        tables[s, :] = 0
        tables[s, :w.block_tables.shape[1]] = w.block_tables[s]
    check_step(w, "stream", "padding", slots=slots, lens=lens, tables=tables)


def test_step_repeated_on_one_pool(gpu):
    """Three steps in a row on one pool: each appends a token and attends
    with it; the pool and outputs follow the oracle step by step."""
    from paged_kv_cache_37_amd import ops

    w = custom_stepped(501, [5, 30, 47, 64], 8, 2)
    dev = Dev(w)
    dt = dev.dt
    pool_ref = w.pool.copy()
    lens = w.seq_lens.copy()
    rng = np.random.default_rng(5)
    fresh = list(w.unused_blocks)
    tables = w.block_tables.copy()
    tables = np.concatenate([tables, np.zeros((w.num_seqs, 2), dtype=np.int32)], axis=1)
    for step in range(3):
        slots = np.empty(w.num_seqs, dtype=np.int32)
        for s in range(w.num_seqs):
            pos = int(lens[s])
            if pos % 16 == 0:
                tables[s, pos // 16] = fresh.pop(0)
            slots[s] = tables[s, pos // 16] * 16 + pos % 16
        lens = lens + 1
        kn = (rng.standard_normal((w.num_seqs, w.num_kv_heads, w.head_dim)).astype(np.float32))
        vn = (rng.standard_normal((w.num_seqs, w.num_kv_heads, w.head_dim)).astype(np.float32))
        kn_b, vn_b = W.f32_to_bf16_bits(kn), W.f32_to_bf16_bits(vn)
        out = ops.paged_decode_step(dev.pool, 0, dev.q, torch.from_numpy(tables).cuda(),
                                    torch.from_numpy(lens.astype(np.int32)).cuda(), w.scale,
                                    host_to_torch(kn_b, dt).cuda(), host_to_torch(vn_b, dt).cuda(),
                                    torch.from_numpy(slots).cuda())
        torch.cuda.synchronize()
        pool_ref = oracle.cache_write(pool_ref, 0, kn_b, vn_b, slots)
        assert torch_to_bits(dev.pool.to_logical()).tobytes() == np.ascontiguousarray(pool_ref).tobytes()
        ref = oracle.decode_attention(pool_ref, 0, w.q, tables, lens, 0, w.scale)
        compare(out, ref, "bf16", f"repeated step {step}")


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_copy_blocks_bit_exact(gpu, dtype, D):
    w = W.custom(61, [40, 17, 300], num_q_heads=8, num_kv_heads=2, head_dim=D, dtype=dtype, num_layers=3)
    dev = Dev(w)
    NB = w.num_blocks
    src = np.array([1, 0, NB + 4, 3, 7, 2], dtype=np.int32)
    dst = np.array([5, 6, 2, 3, 9, -1], dtype=np.int32)
    say("copy_blocks", dtype, D, "NB", NB)
    dev.ops.copy_blocks(dev.pool, torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda())
    torch.cuda.synchronize()
    ref = oracle.copy_blocks(w.pool, src, dst)
    assert torch_to_bits(dev.pool.to_logical()).tobytes() == np.ascontiguousarray(ref).tobytes()


def test_copy_on_write_then_step(gpu):
    """Two sequences share their partial last block; the first gets a device
    copy of it, its table is repointed, and its next token goes into the
    copy with the fused step: both sequences match the oracle."""
    from paged_kv_cache_37_amd import ops

    w = W.custom(88, [20, 20], num_q_heads=8, num_kv_heads=2, head_dim=128)
    # make sequence 1 share sequence 0's blocks (same tables, same data)
    tables = w.block_tables.copy()
    tables[1] = tables[0]
    dev = Dev(w)
    dt = dev.dt
    shared_last = int(tables[0, 1])
    new_block = int(w.unused_blocks[0])
    ops.copy_blocks(dev.pool, torch.tensor([shared_last], dtype=torch.int32).cuda(),
                    torch.tensor([new_block], dtype=torch.int32).cuda())
    tables_after = tables.copy()
    tables_after[0, 1] = new_block
    lens_after = np.array([21, 20], dtype=np.int32)
    slots = np.array([new_block * 16 + 4, -1], dtype=np.int32)
    rng = np.random.default_rng(3)
    kn = W.f32_to_bf16_bits(rng.standard_normal((2, 2, 128)).astype(np.float32))
    vn = W.f32_to_bf16_bits(rng.standard_normal((2, 2, 128)).astype(np.float32))
    out = ops.paged_decode_step(dev.pool, 0, dev.q, torch.from_numpy(tables_after).cuda(),
                                torch.from_numpy(lens_after).cuda(), w.scale, host_to_torch(kn, dt).cuda(),
                                host_to_torch(vn, dt).cuda(), torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    pool_ref = oracle.copy_blocks(w.pool, [shared_last], [new_block])
    pool_ref = oracle.cache_write(pool_ref, 0, kn, vn, slots)
    assert torch_to_bits(dev.pool.to_logical()).tobytes() == np.ascontiguousarray(pool_ref).tobytes()
    ref = oracle.decode_attention(pool_ref, 0, w.q, tables_after, lens_after, 0, w.scale)
    compare(out, ref, "bf16", "cow+step")
