"""Decode at the edges of its size limits: the streaming kernel at the
largest batch it takes (4096 sequences, whose per-sequence tile counts it
keeps in LDS), the automatic choice one sequence past that (the partitioned
matrix-core kernel), and the partitioned kernels at the largest batch the
interface takes (65535 sequences, one grid row each).  Outputs of sampled
sequences are checked against the oracle; every row must be finite and an
empty sequence's row zero; where two variants must be the same launch
(automatic choice against the variant it picks) the outputs are compared
bit for bit."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import Dev, compare, host_to_torch, reference, say, torch_dtype, torch_to_bits

pytestmark = pytest.mark.gpu

STREAM_MAX = 4096   # sequences the streaming kernel takes
GRID_MAX = 65535    # sequences the interface takes


def lengths(seed, S, hi):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, hi + 1, S)
    lens[:6] = [0, 1, 15, 16, 17, hi]  # empty, one token, block edges, the longest
    lens[-1] = 0
    return lens


def sample(S, seed, n=48):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(6), [S - 2, S - 1], rng.integers(0, S, n)]))


def check_rows(out, w, seqs, what):
    got = out.float().cpu().numpy()
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    empty = np.nonzero(w.seq_lens == 0)[0]
    assert np.all(got[empty] == 0), f"{what}: an empty sequence's row is not zero"
    compare(out[torch.from_numpy(seqs)], reference(w, seqs=seqs), "bf16", what)


@pytest.mark.parametrize("S", [STREAM_MAX, STREAM_MAX + 1])
def test_streaming_limit_and_auto_choice(gpu, S):
    """At 4096 sequences the automatic choice is the streaming kernel, one
    more and it is the partitioned matrix-core kernel; asking for the
    streaming kernel past its limit is refused."""
    say("limits: streaming limit", S)
    w = W.custom(61_000 + S, lengths(S, S, 70), num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="bf16")
    dev = Dev(w)
    out_auto = dev.attend()
    seqs = sample(S, S)
    check_rows(out_auto, w, seqs, f"auto at S={S}")
    if S <= STREAM_MAX:
        same = dev.attend(variant="stream")
    else:
        same = dev.attend(variant="mfma")
        with pytest.raises(RuntimeError, match="at most 4096"):
            dev.attend(variant="stream")
    assert torch.equal(out_auto.view(torch.int16), same.view(torch.int16)), f"auto at S={S} is not the chosen variant"


def test_fused_step_at_streaming_limit(gpu):
    """The fused write-then-attend step over 4096 sequences: the pool
    bit-exact, sampled outputs within tolerance of the oracle."""
    import oracle

    S = STREAM_MAX
    say("limits: fused step", S)
    w = W.custom(62_000, lengths(7, S, 70), num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="bf16",
                 extra_blocks=S)
    dev = Dev(w)
    W.with_next_token(w, w.unused_blocks)
    dt = torch_dtype(w)
    out = dev.ops.paged_decode_step(dev.pool, 0, dev.q, torch.from_numpy(np.ascontiguousarray(w.block_tables_after)).cuda(),
                                    torch.from_numpy(w.seq_lens_after).cuda(), w.scale,
                                    host_to_torch(w.k_new, dt).cuda(), host_to_torch(w.v_new, dt).cuda(),
                                    torch.from_numpy(w.slot_mapping).cuda())
    torch.cuda.synchronize()
    pool_ref = oracle.cache_write(w.pool, 0, w.k_new, w.v_new, w.slot_mapping)
    assert torch_to_bits(dev.pool.to_logical()).tobytes() == np.ascontiguousarray(pool_ref).tobytes()
    seqs = sample(S, 8)
    ref = reference(w, pool=pool_ref, tables=w.block_tables_after, lens=w.seq_lens_after, seqs=seqs)
    compare(out[torch.from_numpy(seqs)], ref, "bf16", f"fused step at S={S}")


@pytest.mark.parametrize("variant", ["mfma", "valu"])
def test_partitioned_kernels_at_interface_limit(gpu, variant):
    """65535 sequences of 0..40 tokens (one grid row per sequence), and the
    interface refusing one more."""
    S = GRID_MAX
    say("limits: interface limit", variant, S)
    w = W.custom(63_000, lengths(9, S, 40), num_q_heads=4, num_kv_heads=1, head_dim=64, dtype="bf16")
    dev = Dev(w)
    out = dev.attend(variant=variant)
    check_rows(out, w, sample(S, 10), f"{variant} at S={S}")
    q1 = torch.zeros((S + 1, 4, 64), dtype=torch.bfloat16, device="cuda:0")
    t1 = torch.zeros((S + 1, dev.tables.shape[1]), dtype=torch.int32, device="cuda:0")
    l1 = torch.zeros(S + 1, dtype=torch.int32, device="cuda:0")
    with pytest.raises(RuntimeError, match="65535"):
        dev.ops.paged_decode_attention(dev.pool, 0, q1, t1, l1, w.scale, variant=variant)
