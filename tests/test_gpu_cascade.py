"""GPU parity of shared-prefix (cascade) decode attention: every row starts
with the same full blocks, the STREAM variant attends them once per KV head
for all sequences and merges with the private tails.  Checked against the
oracle (which knows nothing of the sharing: it walks each row), against the
same call without the hint (≤ 1 bf16 ulp: only the summation order
differs), and for the cases where the hint must be ignored (bitwise)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import SHARP_C, Dev, compare, host_to_torch, reference, say, to_f64, torch_to_bits, ulp_bf16
from paged_kv_cache_37_amd.blockpool import shared_prefix_blocks

pytestmark = pytest.mark.gpu


def close_to_plain(a, b, ref, what):
    """Cascade and plain results differ only by fp32 summation order: at most
    one bf16 step after rounding."""
    d = np.abs(to_f64(a) - to_f64(b))
    bound = ulp_bf16(ref) * 1.0001 + 1e-6
    worst = float((d / bound).max())
    say(what, "cascade vs plain: worst", round(worst, 3), "ulp bounds")
    assert worst <= 1.0, f"{what}: cascade and plain differ by more than one bf16 ulp"


def test_cascade_config4(gpu):
    w = W.make(4)
    P = shared_prefix_blocks(np.asarray(w.block_tables), w.seq_lens)
    assert P == 128
    dev = Dev(w)
    out_c = dev.attend(shared_prefix_blocks=P)
    out_p = dev.attend()
    seqs = list(range(0, w.num_seqs, 7)) + [w.num_seqs - 1]
    ref = reference(w, seqs=seqs)
    compare(out_c[seqs], ref, "bf16", "config4 cascade")
    close_to_plain(out_c[seqs], out_p[seqs], ref, "config4")


def test_cascade_fused_step_config4(gpu):
    w = W.make(4)
    W.with_next_token(w, w.unused_blocks)
    dev = Dev(w)
    dt = dev.dt
    tables = torch.from_numpy(np.ascontiguousarray(w.block_tables_after)).cuda()
    lens = torch.from_numpy(np.ascontiguousarray(w.seq_lens_after)).cuda()
    out = dev.ops.paged_decode_step(dev.pool, 0, dev.q, tables, lens, w.scale, host_to_torch(w.k_new, dt).cuda(),
                                    host_to_torch(w.v_new, dt).cuda(), torch.from_numpy(w.slot_mapping).cuda(),
                                    shared_prefix_blocks=128)
    torch.cuda.synchronize()
    pool_ref = oracle.cache_write(w.pool, 0, w.k_new, w.v_new, w.slot_mapping)
    assert torch_to_bits(dev.pool.to_logical()).tobytes() == np.ascontiguousarray(pool_ref).tobytes()
    seqs = list(range(3, w.num_seqs, 9))
    ref = reference(w, pool=pool_ref, tables=w.block_tables_after, lens=w.seq_lens_after, seqs=seqs)
    compare(out[seqs], ref, "bf16", "config4 cascade step")


@pytest.mark.parametrize("prefix,Hq,Hkv,D", [(16, 8, 2, 128), (48, 32, 8, 128), (1024, 8, 2, 64),
                                            (256, 32, 1, 128), (4096, 64, 8, 128)])
def test_cascade_shapes(gpu, prefix, Hq, Hkv, D):
    """Prefixes of 1..256 blocks, tails of 0 (prefix only), 1, 15, 16, 17, a
    few blocks; G = 4, 4, 4, 32 (two head groups per KV head), 8."""
    tails = [0, 1, 15, 16, 17, 100, 300, 7]
    w = W.shared_prefix(900 + prefix + Hq + D, prefix, tails, Hq, Hkv, D)
    P = prefix // 16
    assert shared_prefix_blocks(np.asarray(w.block_tables), w.seq_lens) == P
    dev = Dev(w)
    out_c = dev.attend(shared_prefix_blocks=P)
    out_p = dev.attend(shared_blocks=True)  # every row lists the prefix: cached tile loads
    ref = reference(w)
    compare(out_c, ref, "bf16", f"cascade prefix {prefix} G {Hq // Hkv} D {D}")
    close_to_plain(out_c, out_p, ref, f"prefix {prefix}")
    # the hint changes no bit: the tails without it, and the whole rows with or without it
    assert torch.equal(out_c.view(torch.int16), dev.attend(shared_prefix_blocks=P, shared_blocks=True).view(torch.int16))
    assert torch.equal(out_p.view(torch.int16), dev.attend().view(torch.int16))


@pytest.mark.parametrize("S,Hq,Hkv", [(1040, 32, 8), (1100, 16, 16), (500, 32, 8)])
def test_cascade_grid_split(gpu, S, Hq, Hkv):
    """The launch shares its slots between the tails and the prefix pass
    when the prefix pass's row tiles (KV heads x 128-row tiles) fit in a
    quarter of them (500 sequences, G = 4: 128 tiles), else the tails take
    every slot (1040 sequences: 264 tiles; MHA-shaped 1100: 144 tiles)."""
    rng = np.random.default_rng(S + Hq)
    tails = rng.integers(0, 48, size=S)
    tails[:4] = [0, 1, 16, 47]
    w = W.shared_prefix(1700 + S, 160, tails, Hq, Hkv, 128)
    P = 10
    assert shared_prefix_blocks(np.asarray(w.block_tables), w.seq_lens) == P
    dev = Dev(w)
    out_c = dev.attend(shared_prefix_blocks=P)
    out_p = dev.attend()
    seqs = [0, 1, 2, 3] + list(range(5, S, 97)) + [S - 1]
    ref = reference(w, seqs=seqs)
    compare(out_c[seqs], ref, "bf16", f"cascade S {S} Hq {Hq} Hkv {Hkv}")
    # every row against plain decode (no oracle value for most rows): one
    # bf16 step at the larger of the two magnitudes, plus the decode sharp
    # bar's fp32 term (c rms(row)) for outputs that are a cancellation of
    # terms of the row's size (over these 4M outputs a few near-zero ones
    # differ by ~1e-5 rms)
    a, b = to_f64(out_c), to_f64(out_p)
    rms = np.sqrt(np.mean(b ** 2, axis=-1, keepdims=True))
    bound = ulp_bf16(np.maximum(np.abs(a), np.abs(b))) * 1.0001 + SHARP_C["decode"] * rms
    worst = float((np.abs(a - b) / bound).max())
    say(f"cascade S {S} vs plain: worst", round(worst, 3), "of the bar")
    assert worst <= 1.0


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_cascade_tails_cut_into_many_pieces(gpu, dtype):
    """Tails long enough to span many waves' ranges (every wave holds a
    tile): their first pieces come from the row's own slots, the rest from
    the wave slots in several merge rounds; short tails and empty ones
    beside them.  Against the oracle on the long rows and a sample, and
    against plain decode on every row."""
    rng = np.random.default_rng(41)
    tails = rng.integers(0, 200, size=64)
    tails[:6] = [9000, 0, 8191, 1, 4097, 16]
    w = W.shared_prefix(4100, 512, tails, 32, 8, 128, dtype=dtype)
    P = 32
    assert shared_prefix_blocks(np.asarray(w.block_tables), w.seq_lens) == P
    dev = Dev(w)
    out_c = dev.attend(shared_prefix_blocks=P)
    out_p = dev.attend()
    seqs = [0, 1, 2, 3, 4, 5, 33, 63]
    ref = reference(w, seqs=seqs)
    compare(out_c[seqs], ref, w.dtype, f"cascade, tails cut into many pieces, {dtype}")
    a, b = to_f64(out_c), to_f64(out_p)
    rms = np.sqrt(np.mean(b ** 2, axis=-1, keepdims=True))
    bound = ulp_bf16(np.maximum(np.abs(a), np.abs(b))) * 1.0001 + SHARP_C["decode"] * rms
    worst = float((np.abs(a - b) / bound).max())
    say(f"cascade, many pieces, {dtype} vs plain: worst", round(worst, 3), "of the bar")
    assert worst <= 1.0


@pytest.mark.parametrize("prefix,Hq,Hkv,D", [(2048, 32, 8, 128), (256, 8, 2, 64)])
def test_cascade_fp8(gpu, prefix, Hq, Hkv, D):
    """FP8 pools: the prefix pass widens the same codes as the tail pass."""
    tails = [0, 1, 15, 16, 17, 100, 300, 7]
    w = W.shared_prefix(950 + prefix + D, prefix, tails, Hq, Hkv, D, dtype="fp8")
    dev = Dev(w)
    out_c = dev.attend(shared_prefix_blocks=prefix // 16)
    out_p = dev.attend()
    ref = reference(w)
    compare(out_c, ref, w.dtype, f"fp8 cascade prefix {prefix} D {D}")
    close_to_plain(out_c, out_p, ref, f"fp8 prefix {prefix}")


def test_cascade_fp8_fused_step(gpu):
    w = W.make(4, dtype="fp8")
    W.with_next_token(w, w.unused_blocks)
    dev = Dev(w)
    dt = dev.dt
    tables = torch.from_numpy(np.ascontiguousarray(w.block_tables_after)).cuda()
    lens = torch.from_numpy(np.ascontiguousarray(w.seq_lens_after)).cuda()
    out = dev.ops.paged_decode_step(dev.pool, 0, dev.q, tables, lens, w.scale, host_to_torch(w.k_new, dt).cuda(),
                                    host_to_torch(w.v_new, dt).cuda(), torch.from_numpy(w.slot_mapping).cuda(),
                                    shared_prefix_blocks=128)
    torch.cuda.synchronize()
    pool_ref = oracle.cache_write(w.pool, 0, w.k_new, w.v_new, w.slot_mapping, w.k_scale, w.v_scale)
    assert torch_to_bits(dev.pool.to_logical()).tobytes() == np.ascontiguousarray(pool_ref).tobytes()
    seqs = list(range(3, w.num_seqs, 9))
    ref = reference(w, pool=pool_ref, tables=w.block_tables_after, lens=w.seq_lens_after, seqs=seqs)
    compare(out[seqs], ref, "fp8", "config4-fp8 cascade step")


def test_cascade_partial_hint(gpu):
    """A hint shorter than the real shared prefix is still a valid promise."""
    w = W.shared_prefix(77, 160, [5, 40, 0, 33], 8, 2, 128)
    dev = Dev(w)
    ref = reference(w)
    for P in (1, 4, 10):
        compare(dev.attend(shared_prefix_blocks=P), ref, "bf16", f"hint {P} of 10")


def test_cascade_relabelling_is_bitwise_invisible(gpu):
    """Moving every block to another physical id (tables follow) changes no
    output bit of the cascade path either."""
    w = W.shared_prefix(55, 320, [3, 17, 64, 200, 0, 31], 16, 4, 128)
    out_a = Dev(w).attend(shared_prefix_blocks=20)
    rng = np.random.default_rng(9)
    perm = rng.permutation(w.num_blocks).astype(np.int32)
    w2 = W.shared_prefix(55, 320, [3, 17, 64, 200, 0, 31], 16, 4, 128)
    w2.pool = np.empty_like(w.pool)
    w2.pool[:, perm] = w.pool
    w2.block_tables = perm[np.asarray(w.block_tables)]
    out_b = Dev(w2).attend(shared_prefix_blocks=20)
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))


def test_cascade_hint_ignored_where_unsupported(gpu):
    """Sliding-window rows and the partitioned variant ignore the hint:
    bit-identical to the call without it."""
    w = W.shared_prefix(66, 64, [10, 20, 30], 8, 2, 128)
    dev = Dev(w)
    a = dev.attend(variant="mfma", partition_tokens=256, shared_prefix_blocks=4)
    b = dev.attend(variant="mfma", partition_tokens=256)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    w = W.custom(66, [100, 200, 300], num_q_heads=8, num_kv_heads=2, head_dim=128, window=48)
    dev = Dev(w)
    a = dev.attend(shared_prefix_blocks=2)
    b = dev.attend()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_cascade_hint_beyond_table_is_rejected(gpu):
    from paged_kv_cache_37_amd.ops import KVPoolError

    w = W.shared_prefix(67, 32, [1, 2], 8, 2, 128)
    dev = Dev(w)
    with pytest.raises(KVPoolError):
        dev.attend(shared_prefix_blocks=np.asarray(w.block_tables).shape[1] + 1)


@pytest.mark.parametrize("scale", [-0.0884, 0.0])
def test_cascade_scale_sign_and_zero(gpu, scale):
    """The prefix pass runs on the prefill kernel, which carries a negative
    scale in the queries' signs and makes a zero scale a vanishing one: the
    cascade still matches the oracle and the plain call."""
    w = W.shared_prefix(950, 256, [0, 1, 17, 100, 300], 32, 8, 128)
    w.scale = float(np.float32(scale))  # float32-representable, as the kernel receives it
    dev = Dev(w)
    out_c = dev.attend(shared_prefix_blocks=16)
    out_p = dev.attend()
    ref = reference(w)
    compare(out_c, ref, "bf16", f"cascade scale {scale}")
    close_to_plain(out_c, out_p, ref, f"cascade scale {scale}")


def test_cascade_long_prefix(gpu):
    """A shared prefix longer than 4096 tiles (4500 blocks, 72000 tokens):
    the prefix pass walks any number of table entries, in chunks."""
    w = W.shared_prefix(960, 4500 * 16, [0, 5, 40], 8, 2, 64)
    say("long prefix", w.num_blocks, "blocks")
    dev = Dev(w)
    out_c = dev.attend(shared_prefix_blocks=4500)
    ref = reference(w)
    compare(out_c, ref, "bf16", "cascade long prefix")
    close_to_plain(out_c, dev.attend(), ref, "long prefix")
