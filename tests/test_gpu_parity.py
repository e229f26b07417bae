"""GPU parity: the HIP kernels, called through the C-ABI, against the CPU
oracle on the same seeded inputs.  Cache writes must be bit-exact; decode
attention within 1e-4 (fp32) or 2e-2 + 1e-2 |ref| (bf16), plus the probes
that pin what the tolerance alone would let through (needles, masked
slots, relabelling, aliasing, split consistency)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import Dev, compare, host_to_torch, reference, say, to_f64, torch_dtype, torch_to_bits

pytestmark = pytest.mark.gpu

_CACHE = {}


def workload(config, seed=None):
    key = (config, seed)
    if key not in _CACHE:
        say("generating config", config, "seed", seed)
        _CACHE[key] = W.make(config, seed)
    return _CACHE[key]


def small(seed, ctx, Hq=8, Hkv=2, D=128, dtype="bf16", window=0):
    return W.custom(seed, list(ctx), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, dtype=dtype, window=window)


# ---------------------------------------------------------------------------
# layout and cache writes


@pytest.mark.parametrize("D,dtype", [(64, "f32"), (128, "bf16"), (64, "bf16"), (128, "f32")])
def test_layout_roundtrip_and_offsets(gpu, D, dtype):
    say("layout", D, dtype)
    w = small(40 + D, [5, 40, 77], D=D, dtype=dtype)
    dev = Dev(w)
    back = torch_to_bits(dev.pool.to_logical())
    assert back.tobytes() == np.ascontiguousarray(w.pool).tobytes()
    flat = torch_to_bits(dev.pool.flat())
    rng = np.random.default_rng(0)
    for _ in range(200):
        b, kv, h, t, d = (int(rng.integers(0, w.num_blocks)), int(rng.integers(0, 2)),
                          int(rng.integers(0, w.num_kv_heads)), int(rng.integers(0, 16)), int(rng.integers(0, D)))
        off = dev.pool.offset(0, b, kv, h, t, d)
        a, e = flat[off], w.pool[0, b, kv, t, h, d]
        assert a.tobytes() == e.tobytes()


def next_token_writes(w, seed):
    """One new token per sequence at position seq_lens[s] when its last
    block has room (slot = block * 16 + offset), else padding (-1)."""
    if w.slot_mapping is not None:
        return w.k_new, w.v_new, w.slot_mapping
    rng = np.random.default_rng(seed)
    S = w.num_seqs
    slots = np.full(S, -1, dtype=np.int32)
    for s in range(S):
        ctx = int(w.seq_lens[s])
        if ctx % 16:
            slots[s] = int(w.block_tables[s, w.row_blocks[s] - 1]) * 16 + ctx % 16
    shape = (S, w.num_kv_heads, w.head_dim)
    k = W.f32_to_bf16_bits(rng.standard_normal(shape)) if w.dtype == "bf16" else rng.standard_normal(shape).astype(np.float32)
    v = W.f32_to_bf16_bits(rng.standard_normal(shape)) if w.dtype == "bf16" else rng.standard_normal(shape).astype(np.float32)
    return k, v, slots


@pytest.mark.parametrize("config", [1, 2, 4, 5, 3])
def test_cache_write_bit_exact(gpu, config):
    w = workload(config)
    say("cache_write config", config)
    dev = Dev(w)
    k, v, slots = next_token_writes(w, 100 + config)
    dt = dev.dt
    dev.ops.cache_write(dev.pool, 0, host_to_torch(k, dt).cuda(), host_to_torch(v, dt).cuda(),
                        torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    expect = oracle.cache_write(w.pool, 0, k, v, slots)
    got = dev.pool.to_logical()
    exp_t = host_to_torch(expect, dt).cuda()
    if dt == torch.bfloat16:
        same = torch.equal(got.view(torch.int16), exp_t.view(torch.int16))
    else:
        same = torch.equal(got.view(torch.int32), exp_t.view(torch.int32))
    assert same, "pool differs from the oracle's scatter"
    # a second identical call changes nothing
    dev.ops.cache_write(dev.pool, 0, host_to_torch(k, dt).cuda(), host_to_torch(v, dt).cuda(),
                        torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    got2 = dev.pool.to_logical()
    assert torch.equal(got.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                       got2.view(torch.int16 if dt == torch.bfloat16 else torch.int32))


def test_cache_write_skips_padding_and_out_of_range(gpu):
    w = small(7, [3, 20, 33], D=64, dtype="bf16")
    dev = Dev(w)
    rng = np.random.default_rng(1)
    T = 6
    k = W.f32_to_bf16_bits(rng.standard_normal((T, w.num_kv_heads, 64)))
    v = W.f32_to_bf16_bits(rng.standard_normal((T, w.num_kv_heads, 64)))
    NBs = w.num_blocks * 16
    slots = np.array([5, -1, NBs, NBs + 100, 2**31 - 1, NBs - 1], dtype=np.int32)
    dev.ops.cache_write(dev.pool, 0, host_to_torch(k, torch.bfloat16).cuda(), host_to_torch(v, torch.bfloat16).cuda(),
                        torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    expect = oracle.cache_write(w.pool, 0, k[[0, 5]], v[[0, 5]], slots[[0, 5]])
    assert torch_to_bits(dev.pool.to_logical()).tobytes() == expect.tobytes()


@pytest.mark.parametrize("D,dtype,window", [(64, "f32", 0), (128, "bf16", 0), (64, "bf16", 0), (128, "bf16", 24)])
def test_prefill_write_fills_pool_like_loader(gpu, D, dtype, window):
    """Writing every attended token of every sequence through cache_write
    (a prefill) into a NaN pool gives the loader's pool bit for bit."""
    say("prefill", D, dtype, window)
    w = small(50 + D, [1, 15, 16, 17, 47, 64, 90], D=D, dtype=dtype, window=window)
    ref_dev = Dev(w)
    from paged_kv_cache_37_amd import ops

    dt = ref_dev.dt
    pool = ops.KVPool(1, w.num_blocks, w.num_kv_heads, D, dt)
    nan_pool = np.full_like(w.pool, np.nan if dtype == "f32" else 0x7FC0)
    pool.load_logical(host_to_torch(nan_pool, dt))
    slots, ks, vs = [], [], []
    for s in range(w.num_seqs):
        ctx = int(w.seq_lens[s])
        first = max(0, ctx - window) if window else 0
        fb = first // 16
        for i in range(first, ctx):
            blk = int(w.block_tables[s, i // 16 - fb])
            slots.append(blk * 16 + i % 16)
            ks.append(w.pool[0, blk, 0, i % 16])
            vs.append(w.pool[0, blk, 1, i % 16])
    ops.cache_write(pool, 0, host_to_torch(np.stack(ks), dt).cuda(), host_to_torch(np.stack(vs), dt).cuda(),
                    torch.tensor(slots, dtype=torch.int32).cuda())
    torch.cuda.synchronize()
    a = torch_to_bits(pool.to_logical())
    b = torch_to_bits(ref_dev.pool.to_logical())
    assert a.tobytes() == b.tobytes()


# ---------------------------------------------------------------------------
# decode attention on the five workloads


@pytest.mark.parametrize("config,variant,part", [
    (1, "valu", 0), (1, "valu", 16), (1, "auto", 32),
    (2, "auto", 0), (2, "stream", 0), (2, "mfma", 0), (2, "mfma", 512), (2, "mfma", 256), (2, "mfma", 1024),
    (2, "valu", 0), (2, "valu", 512),
    (4, "stream", 0), (4, "mfma", 0), (4, "valu", 0),
    (5, "stream", 0), (5, "mfma", 512), (5, "mfma", 0), (5, "valu", 512),
])
def test_decode_parity(gpu, config, variant, part):
    w = workload(config)
    say("decode config", config, variant, part)
    dev = Dev(w)
    out = dev.attend(variant=variant, partition_tokens=part)
    ref = _ref_cached(config)
    compare(out, ref, w.dtype, f"config{config}/{variant}/{part}")


_REF = {}


def _ref_cached(config):
    if config not in _REF:
        _REF[config] = reference(workload(config))
    return _REF[config]


@pytest.mark.parametrize("variant,part", [("stream", 0), ("mfma", 0), ("mfma", 512), ("valu", 0)])
def test_decode_parity_config3_sampled(gpu, variant, part):
    """The 70B-shaped layer at full size; the oracle checks 6 sequences."""
    w = workload(3)
    say("decode config 3", variant, part)
    dev = Dev(w)
    out = dev.attend(variant=variant, partition_tokens=part)
    seqs = [0, 1, 37, 64, 101, 127]
    if "c3" not in _REF:
        _REF["c3"] = reference(w, seqs=seqs)
    compare(out[seqs], _REF["c3"], w.dtype, f"config3/{variant}/{part}")


def test_mfma_needs_bf16(gpu):
    w = workload(1)
    dev = Dev(w)
    from paged_kv_cache_37_amd import KVPoolError

    with pytest.raises(KVPoolError):
        dev.attend(variant="mfma")


def test_workspace_too_small_is_rejected(gpu):
    w = workload(2)
    dev = Dev(w)
    from paged_kv_cache_37_amd import KVPoolError

    ws = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(KVPoolError):
        dev.attend(partition_tokens=256, workspace=ws)


# ---------------------------------------------------------------------------
# probes


@pytest.mark.parametrize("variant", ["stream", "mfma", "valu"])
@pytest.mark.parametrize("window", [0, 40])
def test_needle_is_returned_exactly(gpu, variant, window):
    """q_h = 32 e_d and K[t*] = 32 e_d for the group's KV head make one key
    win by a score margin of ~80: the output is V[t*] bit for bit.  t* is
    the first, a middle and the last attended slot, and block edges."""
    ctx = [70, 70, 70, 70, 70, 33, 33, 100]
    w = small(77, ctx, Hq=8, Hkv=2, D=128, window=window)
    pool = w.pool.copy()
    q = w.q.copy()
    G = 4
    picks = []
    for s, c in enumerate(ctx):
        first = max(0, c - window) if window else 0
        cands = [first, first + 1, 15, 16, 31, 32, c - 1, (first + c) // 2]
        cands = [p for p in cands if first <= p < c]
        picks.append(cands[s % len(cands)])
    one = W.f32_to_bf16_bits(np.array([32.0], dtype=np.float32))[0]
    zero = np.uint16(0)
    for s, pstar in enumerate(picks):
        first = max(0, ctx[s] - window) if window else 0
        blk = int(w.block_tables[s, pstar // 16 - first // 16])
        for kv in range(2):
            d = (5 * s + kv) % 128
            pool[0, blk, 0, pstar % 16, kv, :] = zero
            pool[0, blk, 0, pstar % 16, kv, d] = one
            for g in range(G):
                q[s, kv * G + g, :] = zero
                q[s, kv * G + g, d] = one
    w.pool, w.q = pool, q
    dev = Dev(w)
    out = dev.attend(variant=variant)
    got = torch_to_bits(out)
    for s, pstar in enumerate(picks):
        first = max(0, ctx[s] - window) if window else 0
        blk = int(w.block_tables[s, pstar // 16 - first // 16])
        for h in range(8):
            assert got[s, h].tobytes() == pool[0, blk, 1, pstar % 16, h // G].tobytes(), (s, h, pstar)


@pytest.mark.parametrize("variant", ["stream", "mfma", "valu"])
def test_masked_slots_never_count(gpu, variant):
    """Needles planted where no position maps (after the last token, before
    a window's first position) leave the output bit-identical."""
    ctx = [20, 37, 50, 100]
    w = small(88, ctx, window=40)
    dev = Dev(w)
    base = torch_to_bits(dev.attend(variant=variant))
    pool = w.pool.copy()
    big = W.f32_to_bf16_bits(np.float32(64.0))
    for s, c in enumerate(ctx):
        first = max(0, c - 40)
        fb = first // 16
        nb = w.row_blocks[s]
        last = int(w.block_tables[s, nb - 1])
        for t in range((c % 16) or 16, 16):
            pool[0, last, :, t] = big
        head = int(w.block_tables[s, 0])
        for t in range(0, first - fb * 16):
            pool[0, head, :, t] = big
    w2 = W.Workload(**{**w.__dict__, "pool": pool})
    dev2 = Dev(w2)
    assert torch_to_bits(dev2.attend(variant=variant)).tobytes() == base.tobytes()


@pytest.mark.parametrize("variant", ["stream", "mfma", "valu"])
def test_constant_values(gpu, variant):
    w = small(91, [1, 16, 17, 300, 1000], window=0)
    pool = w.pool.copy()
    pool[:, :, 1] = W.f32_to_bf16_bits(np.float32(1.0))
    w.pool = pool
    out = Dev(w).attend(variant=variant, partition_tokens=256)
    assert torch.all(out.float() == 1.0)


@pytest.mark.parametrize("variant", ["stream", "mfma", "valu"])
def test_relabelling_is_bitwise_invisible(gpu, variant):
    w = small(92, [3, 16, 45, 200, 777], Hq=16, Hkv=4)
    a = torch_to_bits(Dev(w).attend(variant=variant, partition_tokens=128))
    pi = np.random.default_rng(5).permutation(w.num_blocks)
    pool = np.empty_like(w.pool)
    pool[:, pi] = w.pool
    w2 = W.Workload(**{**w.__dict__, "pool": pool, "block_tables": pi[w.block_tables].astype(np.int32)})
    b = torch_to_bits(Dev(w2).attend(variant=variant, partition_tokens=128))
    assert a.tobytes() == b.tobytes()


@pytest.mark.parametrize("variant", ["stream", "mfma", "valu"])
def test_shared_prefix_equals_private_copies(gpu, variant):
    w = W.config4(seed=4, num_seqs=12)
    a = torch_to_bits(Dev(w).attend(variant=variant))
    # give every sequence its own copy of the 128 prefix blocks
    S = w.num_seqs
    NB2 = w.num_blocks + 128 * S
    pool = np.concatenate([w.pool, np.zeros((1, 128 * S) + w.pool.shape[2:], w.pool.dtype)], axis=1)
    tables = w.block_tables.copy()
    for s in range(S):
        for j in range(128):
            nb = w.num_blocks + 128 * s + j
            pool[0, nb] = w.pool[0, w.block_tables[s, j]]
            tables[s, j] = nb
    w2 = W.Workload(**{**w.__dict__, "pool": pool, "num_blocks": NB2, "block_tables": tables})
    b = torch_to_bits(Dev(w2).attend(variant=variant))
    assert a.tobytes() == b.tobytes()
    compare(torch.from_numpy(a.view(np.int16)).view(torch.bfloat16), reference(w), "bf16", f"shared-prefix/{variant}")


@pytest.mark.parametrize("variant", ["mfma", "valu"])
def test_split_matches_single_pass(gpu, variant):
    """Rows of up to 1024 tokens: one partition versus 512/256/128-token
    partitions.  Both round the same fp32-accumulated result to bf16, so
    they agree to one bf16 ulp plus the fp32 accumulation-order noise,
    bounded by 1e-5 of the row's rms (near-zero outputs of a row come from
    cancellation, where an ulp of the output means nothing)."""
    from gpu_helpers import ulp_bf16

    w = small(93, [1, 100, 511, 512, 513, 1000, 1024], Hq=16, Hkv=2)
    dev = Dev(w)
    single = to_f64(dev.attend(variant=variant, partition_tokens=1024))
    rms = np.sqrt(np.mean(single ** 2, axis=-1, keepdims=True))
    for part in (512, 256, 128):
        split = to_f64(dev.attend(variant=variant, partition_tokens=part))
        bound = np.maximum(ulp_bf16(single), ulp_bf16(split)) + 1e-5 * rms
        ratio = np.abs(split - single) / bound
        worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        say("split", variant, part, "max/bound", float(ratio.max()), "at", worst, single[worst], split[worst])
        assert np.all(ratio <= 1.0), part


@pytest.mark.parametrize("variant", ["stream", "mfma", "valu"])
def test_gqa_heads_with_equal_queries_agree(gpu, variant):
    w = small(94, [9, 64, 130], Hq=16, Hkv=2)
    q = w.q.copy()
    for kv in range(2):
        q[:, kv * 8:(kv + 1) * 8] = q[:, kv * 8][:, None]
    w.q = q
    out = torch_to_bits(Dev(w).attend(variant=variant))
    for kv in range(2):
        for g in range(1, 8):
            assert out[:, kv * 8 + g].tobytes() == out[:, kv * 8].tobytes()


def test_write_then_attend(gpu):
    """Config 1: write each sequence's next token, then attend over ctx+1."""
    w = workload(1)
    dev = Dev(w)
    dt = dev.dt
    dev.ops.cache_write(dev.pool, 0, host_to_torch(w.k_new, dt).cuda(), host_to_torch(w.v_new, dt).cuda(),
                        torch.from_numpy(w.slot_mapping).cuda())
    tables = torch.from_numpy(w.block_tables_after).cuda()
    lens = torch.from_numpy(w.seq_lens_after).cuda()
    out = dev.attend(tables=tables, lens=lens)
    pool_after = oracle.cache_write(w.pool, 0, w.k_new, w.v_new, w.slot_mapping)
    ref = oracle.decode_attention(pool_after, 0, w.q, w.block_tables_after, w.seq_lens_after, 0, w.scale)
    compare(out, ref, "f32", "config1 write+attend")


# ---------------------------------------------------------------------------
# edge cases and shape sweeps


@pytest.mark.parametrize("variant", ["stream", "mfma", "valu"])
def test_empty_and_tiny_sequences(gpu, variant):
    w = small(95, [0, 1, 0, 2, 16, 0], Hq=8, Hkv=2)
    out = Dev(w).attend(variant=variant)
    ref = reference(w)
    compare(out, ref, "bf16", f"empty/{variant}")
    assert torch.all(out[[0, 2, 5]].float() == 0)


@pytest.mark.parametrize("variant", ["stream", "mfma", "valu"])
@pytest.mark.parametrize("window", [0, 33])
def test_length_sweep_around_block_edges(gpu, variant, window):
    ctx = list(range(1, 66)) + [255, 256, 257, 511, 512, 513]
    w = small(96 + window, ctx, Hq=8, Hkv=2, window=window)
    out = Dev(w).attend(variant=variant, partition_tokens=64)
    compare(out, reference(w), "bf16", f"lengths/{variant}/w{window}")


@pytest.mark.parametrize("variant", ["stream", "mfma", "valu"])
def test_window_offsets_sweep(gpu, variant):
    """Windowed rows whose first attended slot sits at every offset 0..15."""
    W_ = 64
    ctx = [W_ + o + 16 * k for k in (1, 3) for o in range(16)]
    w = small(97, ctx, Hq=8, Hkv=2, window=W_)
    out = Dev(w).attend(variant=variant, partition_tokens=32)
    compare(out, reference(w), "bf16", f"window-offsets/{variant}")


@pytest.mark.parametrize("variant", ["stream", "mfma", "valu"])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (8, 2), (16, 2), (32, 2), (24, 8), (64, 2)])
@pytest.mark.parametrize("D", [64, 128])
def test_head_group_and_dim_sweep(gpu, variant, Hq, Hkv, D):
    w = small(98 + Hq + D, [7, 64, 129, 300], Hq=Hq, Hkv=Hkv, D=D)
    out = Dev(w).attend(variant=variant)
    compare(out, reference(w), "bf16", f"G{Hq // Hkv}/D{D}/{variant}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("window", [0, 50])
def test_fp32_pools(gpu, D, window):
    w = small(99 + D, [1, 16, 17, 99, 300], Hq=8, Hkv=2, D=D, dtype="f32", window=window)
    out = Dev(w).attend(partition_tokens=64)
    compare(out, reference(w), "f32", f"fp32/D{D}/w{window}")


def test_multi_layer_pool(gpu):
    """Layers are separate slices of one pool; attend layer 1."""
    w = W.custom(31, [40, 100], num_q_heads=8, num_kv_heads=2, head_dim=128, num_layers=3)
    dev = Dev(w)
    for layer in (0, 2):
        out = dev.attend(layer=layer)
        compare(out, reference(w, layer=layer), "bf16", f"layer{layer}")


def test_workspace_is_reusable(gpu):
    """One workspace serves call after call and every variant."""
    w = small(35, [100, 700, 1000, 33], Hq=8, Hkv=2)
    dev = Dev(w)
    ws = dev.ops.make_workspace(dev.pool, w.num_seqs, w.num_q_heads, w.block_tables.shape[1], 128)
    ws.fill_(0xFF)  # contents need no initialisation
    ref = reference(w)
    for variant in ("mfma", "valu", "stream", "mfma", "stream"):
        out = dev.attend(variant=variant, partition_tokens=128 if variant != "stream" else 0, workspace=ws)
        compare(out, ref, "bf16", f"reuse/{variant}")


def test_call_on_a_side_stream_without_workspace(gpu):
    """Calls launched on a stream other than the current one, with out and
    workspace made by the binding, while the current stream allocates and
    fills memory meanwhile: every output equals the current-stream call's."""
    w = small(36, [700, 1000, 2000, 33, 4000], Hq=8, Hkv=2)
    dev = Dev(w)
    runs = (("stream", 0), ("mfma", 128), ("stream", 0), ("mfma", 256))
    base = {r: torch_to_bits(dev.attend(variant=r[0], partition_tokens=r[1])) for r in runs}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for variant, part in runs:
        outs.append(dev.ops.paged_decode_attention(dev.pool, 0, dev.q, dev.tables, dev.lens, w.scale,
                                                   variant=variant, partition_tokens=part, stream=side))
        junk = torch.empty(32 << 20, dtype=torch.uint8, device="cuda")
        junk.fill_(0xFF)
        del junk
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r, o in zip(runs, outs):
        assert torch_to_bits(o).tobytes() == base[r].tobytes(), r


@pytest.mark.parametrize("dtype,B,D,window", [("bf16", 16, 128, 0), ("fp8", 16, 128, 0), ("bf16", 32, 64, 0),
                                              ("fp8", 32, 128, 40), ("bf16", 16, 128, 33), ("fp8", 16, 64, 0)])
def test_shared_blocks_hint_changes_no_bit(gpu, dtype, B, D, window):
    """The streaming kernel reads tiles with non-temporal loads by default
    and with cached loads under the shared_blocks hint; the outputs are the
    same bits, for attention and for the fused step (pool included), and
    match the oracle."""
    lens = [0, 1, 15, 16, 17, 31, 33, 100, 257, 700, 1500, 2048]
    w = W.custom(7100 + B + D + window, lens, num_q_heads=8, num_kv_heads=2, head_dim=D, dtype=dtype, window=window,
                 block_size=B, extra_blocks=len(lens))
    say("shared_blocks hint", dtype, B, D, window)
    devs = [Dev(w), Dev(w)]
    outs = [d.attend(variant="stream", shared_blocks=hint) for d, hint in zip(devs, (False, True))]
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    compare(outs[0], reference(w), "bf16", f"stream {dtype} B{B} D{D} w{window}")
    # the partitioned kernel (split into 256-token partitions) likewise
    parts = [d.attend(variant="mfma", partition_tokens=256, shared_blocks=hint) for d, hint in zip(devs, (False, True))]
    assert torch.equal(parts[0].view(torch.int16), parts[1].view(torch.int16))
    compare(parts[0], reference(w), "bf16", f"mfma {dtype} B{B} D{D} w{window}")
    W.with_next_token(w, w.unused_blocks)
    dt = torch_dtype(w)
    steps = []
    for d, hint in zip(devs, (False, True)):
        steps.append(d.ops.paged_decode_step(d.pool, 0, d.q, torch.from_numpy(np.ascontiguousarray(w.block_tables_after)).cuda(),
                                             torch.from_numpy(w.seq_lens_after).cuda(), w.scale,
                                             host_to_torch(w.k_new, dt).cuda(), host_to_torch(w.v_new, dt).cuda(),
                                             torch.from_numpy(w.slot_mapping).cuda(), sliding_window=w.window,
                                             shared_blocks=hint))
    torch.cuda.synchronize()
    assert torch.equal(steps[0].view(torch.int16), steps[1].view(torch.int16))
    pools = [torch_to_bits(d.pool.to_logical()) for d in devs]
    assert pools[0].tobytes() == pools[1].tobytes()
    pool_ref = oracle.cache_write(w.pool, 0, w.k_new, w.v_new, w.slot_mapping, w.k_scale, w.v_scale)
    assert pools[0].tobytes() == np.ascontiguousarray(pool_ref).tobytes()
    compare(steps[0], reference(w, pool=pool_ref, tables=w.block_tables_after, lens=w.seq_lens_after), "bf16",
            f"step {dtype} B{B} D{D} w{window}")


@pytest.mark.parametrize("dtype,B,D", [("bf16", 16, 128), ("bf16", 32, 64), ("f32", 16, 64), ("fp8", 16, 128),
                                       ("fp8", 32, 128)])
def test_cache_write_slot_patterns(gpu, dtype, B, D):
    """Token groups of four that fill one V quad in order are written as one
    transposed store per dimension, every other pattern token by token: a
    batch mixing whole quads, quads cut by padding or by the pool's end,
    shifted, reversed and partly repeated groups, and a ragged tail, written
    bit-exact against the oracle's scatter."""
    rng = np.random.default_rng(7400 + B + D)
    w = W.custom(7400 + B + D, [B * 6], num_q_heads=4, num_kv_heads=2, head_dim=D, dtype=dtype, block_size=B,
                 pool_factor=3.0)
    NS = w.num_blocks * B
    b0, b1, b2 = (int(x) * B for x in w.unused_blocks[:3])
    last = NS - 4  # the pool's last quad
    groups = [
        [b0, b0 + 1, b0 + 2, b0 + 3],                # whole quad
        [b0 + 4, b0 + 5, b0 + 6, b0 + 7],            # the next one
        [b0 + 8, b0 + 9, -1, b0 + 11],               # padding inside
        [b0 + 13, b0 + 14, b0 + 15, b2 + 8],        # shifted by one
        [b1 + 7, b1 + 6, b1 + 5, b1 + 4],            # reversed
        [b1, b1 + 1, b1 + 2, NS + 2],                # last slot outside the pool
        [last, last + 1, last + 2, last + 3],        # the pool's last quad
        [b2 + B - 4, b2 + B - 3, b2 + B - 2, b2 + B - 1],  # a block's last quad
        [b2, b2 + 1, b2 + 2],                        # ragged tail: three tokens
    ]
    slots = np.array([s for g in groups for s in g], dtype=np.int32)
    T = len(slots)
    say("cache_write slot patterns", dtype, B, D, T)
    shape = (T, w.num_kv_heads, D)
    if dtype == "f32":
        k, v = rng.standard_normal(shape).astype(np.float32), rng.standard_normal(shape).astype(np.float32)
    else:
        k, v = W.f32_to_bf16_bits(rng.standard_normal(shape)), W.f32_to_bf16_bits(rng.standard_normal(shape))
    dev = Dev(w)
    dt = torch_dtype(w)
    dev.ops.cache_write(dev.pool, 0, host_to_torch(k, dt).cuda(), host_to_torch(v, dt).cuda(),
                        torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    keep = (slots >= 0) & (slots < NS)
    expect = oracle.cache_write(w.pool, 0, k[keep], v[keep], slots[keep], w.k_scale, w.v_scale)
    assert torch_to_bits(dev.pool.to_logical()).tobytes() == np.ascontiguousarray(expect).tobytes()
