"""GPU parity of FP8 (E4M3) pools through the C-ABI against the oracle.

Writes: every bf16 bit pattern is quantized by cache_write and compared
code for code with the oracle's encode (nearest code, ties to even,
saturating at +-448), at several scales.  Reads: every code widens exactly
(a one-token context returns its V row unchanged).  Attention over FP8
pools follows the oracle within the bf16 bound on the Llama-shaped
workloads and on head-group, head_dim, window and variant sweeps; per-layer
scales are applied per layer.  The fused step and the shared-prefix path
with FP8 pools are covered next to their bf16 cases."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import Dev, compare, host_to_torch, reference, say, torch_to_bits

pytestmark = pytest.mark.gpu

ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


@pytest.mark.parametrize("k_scale,v_scale", [(1.0, 1.0), (0.37, 3.0), (2.0 ** -10, 1000.0)])
def test_cache_write_quantizes_every_bf16_value(gpu, k_scale, v_scale):
    """All 65536 bf16 patterns (zeros, subnormals, ties, values past 448,
    infinities, NaNs) as K and as V, written to scattered slots."""
    from paged_kv_cache_37_amd import ops

    Hkv, D = 2, 128
    T = 65536 // (Hkv * D)
    rng = np.random.default_rng(17)
    k = rng.permutation(ALL_BF16).reshape(T, Hkv, D)
    v = ALL_BF16[::-1].copy().reshape(T, Hkv, D)
    NB = T // 16 + 3
    slots = rng.permutation(NB * 16)[:T].astype(np.int32)
    say("fp8 quantization", k_scale, v_scale, "tokens", T)
    pool = ops.KVPool(1, NB, Hkv, D, torch.float8_e4m3fn)
    pool.set_fp8_scales(0, k_scale, v_scale)
    pool.flat().zero_()
    ops.cache_write(pool, 0, host_to_torch(k, torch.bfloat16).cuda(), host_to_torch(v, torch.bfloat16).cuda(),
                    torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    got = torch_to_bits(pool.to_logical())
    ref = oracle.cache_write(np.zeros((1, NB, 2, 16, Hkv, D), np.uint8), 0, k, v, slots, k_scale, v_scale)
    # a NaN input may come back as either NaN code (the sign of a NaN carries nothing)
    both_nan = ((got & 0x7F) == 0x7F) & ((ref & 0x7F) == 0x7F)
    bad = (got != ref) & ~both_nan
    assert not bad.any(), f"{int(bad.sum())} codes differ, first at {np.argwhere(bad)[0]}"
    assert int(((ref & 0x7F) == 0x7F).sum()) == int(((got & 0x7F) == 0x7F).sum())


@pytest.mark.parametrize("variant", ["stream", "mfma"])
def test_every_code_widens_exactly(gpu, variant):
    """One-token contexts: the softmax weight is exactly 1, so the output is
    the V row itself, which bf16 holds exactly for every finite code."""
    from paged_kv_cache_37_amd import ops

    D, Hkv, Hq, S = 128, 1, 4, 2
    codes = np.arange(256, dtype=np.uint32).astype(np.uint8)
    codes[[0x7F, 0xFF]] = 0  # the NaN codes
    logical = np.zeros((1, 4, 2, 16, Hkv, D), np.uint8)
    rng = np.random.default_rng(5)
    logical[0, :, 0] = rng.integers(0, 0x7F, size=(4, 16, Hkv, D), dtype=np.uint8)  # K: any finite codes
    logical[0, 1, 1, 0, 0] = codes[:128]
    logical[0, 3, 1, 0, 0] = codes[128:]
    pool = ops.KVPool(1, 4, Hkv, D, torch.float8_e4m3fn)
    pool.load_logical(torch.from_numpy(logical))
    pool.set_fp8_scales(0, 0.37, 1.0)
    q = host_to_torch(W.f32_to_bf16_bits(rng.standard_normal((S, Hq, D)).astype(np.float32)),
                      torch.bfloat16).cuda()
    tables = torch.tensor([[1], [3]], dtype=torch.int32).cuda()
    lens = torch.tensor([1, 1], dtype=torch.int32).cuda()
    out = ops.paged_decode_attention(pool, 0, q, tables, lens, 0.1, variant=variant)
    torch.cuda.synchronize()
    want = oracle.e4m3_decode(codes).reshape(S, 1, D)
    got = out.float().cpu().numpy().astype(np.float64)  # bf16 -> float64 is exact
    # equal as numbers (the sum that forms the output turns -0 into +0)
    assert (got == np.broadcast_to(want, got.shape)).all(), "a code did not widen to its exact value"


_W = {}


def fp8_config(config):
    if config not in _W:
        say("generating fp8 config", config)
        _W[config] = W.make(config, dtype="fp8")
    return _W[config]


@pytest.mark.parametrize("config", [2, 3, 5])
def test_fp8_configs(gpu, config):
    w = fp8_config(config)
    dev = Dev(w)
    seqs = list(range(0, w.num_seqs, 11)) + [w.num_seqs - 1]
    ref = reference(w, seqs=seqs)
    for variant, pt in (("stream", 0), ("mfma", 512)):
        out = dev.attend(variant=variant, partition_tokens=pt)
        compare(out[seqs], ref, w.dtype, f"{w.name}/{variant}")


@pytest.mark.parametrize("Hq,Hkv,D,window", [(8, 8, 128, 0), (8, 2, 128, 0), (64, 8, 128, 0), (32, 1, 128, 0),
                                             (12, 4, 64, 0), (48, 2, 64, 0), (8, 2, 128, 48), (16, 4, 64, 100)])
def test_fp8_shapes(gpu, Hq, Hkv, D, window):
    """G = 1, 4, 8, 32 (two head groups), 3, 24; windows cutting blocks."""
    ctx = [1, 15, 16, 17, 33, 200, 511, 1000]
    w = W.custom(700 + Hq + D + window, ctx, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, dtype="fp8",
                 window=window)
    dev = Dev(w)
    ref = reference(w)
    for variant, pt in (("stream", 0), ("mfma", 0), ("mfma", 64)):
        compare(dev.attend(variant=variant, partition_tokens=pt), ref, w.dtype,
                f"fp8 G{Hq // Hkv} D{D} W{window} {variant}/{pt}")


def test_fp8_scales_are_per_layer(gpu):
    """Two layers with different scales: each call uses its layer's pair."""
    w = W.custom(808, [40, 300, 17], num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="fp8", num_layers=2)
    dev = Dev(w)
    dev.pool.set_fp8_scales(1, 0.9, 0.2)
    for layer, (ks, vs) in ((0, (w.k_scale, w.v_scale)), (1, (0.9, 0.2))):
        ref = oracle.decode_attention(w.pool, layer, w.q, w.block_tables, w.seq_lens, 0, w.scale,
                                      k_scale=ks, v_scale=vs)
        compare(dev.attend(layer=layer), ref, w.dtype, f"fp8 layer {layer}")


def test_fp8_relabelling_is_bitwise_invisible(gpu):
    """Moving every block to another physical id changes no output bit."""
    w = W.custom(809, [3, 17, 64, 200, 0, 31], num_q_heads=16, num_kv_heads=4, head_dim=128, dtype="fp8")
    out_a = Dev(w).attend()
    perm = np.random.default_rng(9).permutation(w.num_blocks).astype(np.int32)
    w2 = W.custom(809, [3, 17, 64, 200, 0, 31], num_q_heads=16, num_kv_heads=4, head_dim=128, dtype="fp8")
    w2.pool = np.empty_like(w.pool)
    w2.pool[:, perm] = w.pool
    w2.block_tables = perm[np.asarray(w.block_tables)]
    out_b = Dev(w2).attend()
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
