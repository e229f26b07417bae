"""GPU parity of 32-token blocks ([Optimizing] Trade-offs of Block Size
Tuning) through the C-ABI.

Every kernel streams 16-token tiles; a 32-token block is two of them.  So
the same keys laid out in 32-token blocks must give bit-identical outputs
to the 16-token layout, for every variant, window offset (a window may
start in a block's second tile) and head shape; cache writes, block copies,
the fused step and the shared-prefix path are checked against the oracle
and against the unfused calls."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import Dev, compare, host_to_torch, reference, relaid, say, torch_to_bits

pytestmark = pytest.mark.gpu


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("dtype,Hq,Hkv,D,window", [
    ("bf16", 8, 2, 128, 0), ("bf16", 8, 2, 128, 40), ("bf16", 32, 8, 128, 100), ("bf16", 12, 4, 64, 48),
    ("bf16", 32, 1, 128, 0), ("fp8", 8, 2, 128, 40), ("fp8", 16, 4, 64, 0), ("f32", 8, 2, 64, 40)])
def test_block32_is_bitwise_the_16_token_layout(gpu, dtype, Hq, Hkv, D, window):
    """Same keys, 16- vs 32-token blocks: identical output bits per variant."""
    ctx = [1, 15, 16, 17, 31, 32, 33, 57, 64, 95, 200, 511, 1000]
    w16 = W.custom(500 + Hq + D + window, ctx, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, dtype=dtype,
                   window=window)
    w32 = relaid(w16, 32)
    oracle.check_tables(w32.block_tables, w32.seq_lens, w32.window, 32, w32.num_blocks, w32.row_blocks)
    d16, d32 = Dev(w16), Dev(w32)
    variants = [("valu", 0), ("valu", 64)] if dtype == "f32" else [("stream", 0), ("mfma", 0), ("mfma", 64)]
    if dtype == "bf16":
        variants.append(("valu", 0))
    ref = reference(w16)
    for variant, pt in variants:
        a = d16.attend(variant=variant, partition_tokens=pt)
        b = d32.attend(variant=variant, partition_tokens=pt)
        say("block32", dtype, Hq, Hkv, D, window, variant, pt)
        assert torch.equal(bits(a), bits(b)), f"{variant}/{pt}: 32-token layout changed output bits"
        compare(b, ref, dtype, f"B32 {dtype} G{Hq // Hkv} D{D} W{window} {variant}/{pt}")


@pytest.mark.parametrize("config,dtype", [(2, "bf16"), (5, "bf16"), (2, "fp8")])
def test_block32_configs(gpu, config, dtype):
    """Configs 2 and 5 generated in 32-token blocks, sampled sequences
    against the oracle."""
    w = W.make(config, dtype=dtype, block_size=32)
    dev = Dev(w)
    seqs = list(range(0, w.num_seqs, 9)) + [w.num_seqs - 1]
    ref = reference(w, seqs=seqs)
    for variant, pt in (("stream", 0), ("mfma", 512)):
        compare(dev.attend(variant=variant, partition_tokens=pt)[seqs], ref, w.dtype, f"{w.name}/{variant}")


@pytest.mark.parametrize("dtype", ["bf16", "f32", "fp8"])
def test_block32_cache_write_bit_exact(gpu, dtype):
    w = W.custom(41, [31, 32, 33, 63, 64, 100], num_q_heads=8, num_kv_heads=2, head_dim=128 if dtype != "f32" else 64,
                 dtype=dtype, block_size=32)
    W.with_next_token(w, w.unused_blocks)
    slots = w.slot_mapping.copy()
    slots[2] = -1
    dev = Dev(w)
    dev.ops.cache_write(dev.pool, 0, host_to_torch(w.k_new, dev.dt).cuda(), host_to_torch(w.v_new, dev.dt).cuda(),
                        torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    ref = oracle.cache_write(w.pool, 0, w.k_new, w.v_new, slots, w.k_scale, w.v_scale)
    assert torch_to_bits(dev.pool.to_logical()).tobytes() == np.ascontiguousarray(ref).tobytes()


@pytest.mark.parametrize("dtype,window", [("bf16", 0), ("bf16", 40), ("fp8", 0)])
def test_block32_fused_step(gpu, dtype, window):
    """The fused step into 32-token blocks: pool and outputs bit-identical to
    cache_write + attention, and the oracle over the written pool."""
    w = W.custom(42 + window, [1, 15, 16, 31, 32, 47, 63, 64, 200, 511], num_q_heads=8, num_kv_heads=2,
                 head_dim=128, dtype=dtype, window=window, block_size=32)
    W.with_next_token(w, w.unused_blocks)
    res = []
    for fused in (True, False):
        dev = Dev(w)
        k = host_to_torch(w.k_new, dev.dt).cuda()
        v = host_to_torch(w.v_new, dev.dt).cuda()
        sl = torch.from_numpy(w.slot_mapping).cuda()
        tb = torch.from_numpy(np.ascontiguousarray(w.block_tables_after)).cuda()
        ln = torch.from_numpy(np.ascontiguousarray(w.seq_lens_after)).cuda()
        if fused:
            out = dev.ops.paged_decode_step(dev.pool, 0, dev.q, tb, ln, w.scale, k, v, sl, sliding_window=w.window)
        else:
            dev.ops.cache_write(dev.pool, 0, k, v, sl)
            out = dev.ops.paged_decode_attention(dev.pool, 0, dev.q, tb, ln, w.scale, sliding_window=w.window)
        torch.cuda.synchronize()
        res.append((out, torch_to_bits(dev.pool.to_logical())))
    (fo, fp), (uo, up) = res
    assert fp.tobytes() == up.tobytes()
    assert torch.equal(bits(fo), bits(uo))
    pool_ref = oracle.cache_write(w.pool, 0, w.k_new, w.v_new, w.slot_mapping, w.k_scale, w.v_scale)
    assert fp.tobytes() == np.ascontiguousarray(pool_ref).tobytes()
    ref = reference(w, pool=pool_ref, tables=w.block_tables_after, lens=w.seq_lens_after)
    compare(fo, ref, w.dtype, f"B32 step {dtype} W{window}")


def test_block32_cascade(gpu):
    """A shared prefix of 32-token blocks (64 blocks = 128 tiles)."""
    tails = [0, 1, 15, 16, 17, 33, 100, 300]
    w = W.shared_prefix(61, 2048, tails, 32, 8, 128, block_size=32)
    dev = Dev(w)
    out_c = dev.attend(shared_prefix_blocks=64)
    out_p = dev.attend()
    ref = reference(w)
    compare(out_c, ref, "bf16", "B32 cascade")
    compare(out_p, ref, "bf16", "B32 plain")


def test_block32_copy_blocks(gpu):
    w = W.custom(62, [40, 70, 300], num_q_heads=8, num_kv_heads=2, head_dim=128, num_layers=2, block_size=32)
    dev = Dev(w)
    NB = w.num_blocks
    src = np.array([1, 0, NB + 4, 3, 7], dtype=np.int32)
    dst = np.array([5, 6, 2, 3, -1], dtype=np.int32)
    dev.ops.copy_blocks(dev.pool, torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda())
    torch.cuda.synchronize()
    assert torch_to_bits(dev.pool.to_logical()).tobytes() == np.ascontiguousarray(
        oracle.copy_blocks(w.pool, src, dst)).tobytes()
