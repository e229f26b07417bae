"""paged_decode_step_noalloc (the decode step whose workspace is the library's
static scratch) against paged_decode_step with a caller workspace: the same
kernels, so the outputs and the pool must be bit-identical, call after call,
including a smaller call after a larger one (the scratch keeps the last
call's contents)."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import Dev, compare, host_to_torch, reference, say, torch_to_bits

pytestmark = pytest.mark.gpu


def step_inputs(w):
    dt = torch.bfloat16
    return dict(block_tables=torch.from_numpy(np.ascontiguousarray(w.block_tables_after)).cuda(),
                seq_lens=torch.from_numpy(w.seq_lens_after).cuda(),
                k_new=host_to_torch(w.k_new, dt).cuda(), v_new=host_to_torch(w.v_new, dt).cuda(),
                slot_mapping=torch.from_numpy(w.slot_mapping).cuda())


def both_ways(w, what, **kw):
    """The step through both entry points, each on its own copy of the pool;
    returns the no-alloc output after checking it bit for bit."""
    say("no-alloc step", what, kw)
    a, b = Dev(w), Dev(w)
    x = step_inputs(w)
    ref = a.ops.paged_decode_step(a.pool, 0, a.q, x["block_tables"], x["seq_lens"], w.scale, x["k_new"], x["v_new"],
                                  x["slot_mapping"], sliding_window=w.window, **kw)
    out = torch.full_like(b.q, float("nan"))
    got = b.ops.paged_decode_step_noalloc(b.pool, 0, b.q, x["block_tables"], x["seq_lens"], w.scale, x["k_new"],
                                          x["v_new"], x["slot_mapping"], out, sliding_window=w.window, **kw)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"{what}: outputs differ"
    assert torch.equal(b.pool.storage, a.pool.storage), f"{what}: pools differ"
    return got


def test_noalloc_step_matches_the_step_twice(gpu):
    """Two calls in a row, the second smaller: the Llama-3-8B-shaped batch
    (64 sequences), then 6 short sequences; each bit-identical to
    paged_decode_step, and the small one checked against the oracle."""
    w = W.make(2)
    W.with_next_token(w, w.unused_blocks)
    both_ways(w, "config 2")
    s = W.custom(801, [1, 15, 16, 17, 100, 333], num_q_heads=8, num_kv_heads=2, head_dim=128,
                 extra_blocks=6)
    W.with_next_token(s, s.unused_blocks)
    got = both_ways(s, "small")
    import oracle

    pool_ref = oracle.cache_write(s.pool, 0, s.k_new, s.v_new, s.slot_mapping)
    compare(got, reference(s, pool=pool_ref, tables=s.block_tables_after, lens=s.seq_lens_after), "bf16",
            "no-alloc small step")


def test_noalloc_step_other_paths(gpu):
    """The shared-prefix (cascade) step, an FP8 pool, and the partitioned
    kernel with its split-K reduce, each bit-identical to paged_decode_step."""
    w = W.config4(seed=4, num_seqs=64)
    W.with_next_token(w, w.unused_blocks)
    from paged_kv_cache_37_amd.blockpool import shared_prefix_blocks

    P = shared_prefix_blocks(np.asarray(w.block_tables_after), w.seq_lens_after, block_size=w.block_size)
    assert P == 128
    both_ways(w, "cascade", shared_prefix_blocks=P)
    f = W.custom(802, [5, 64, 700, 1500], num_q_heads=16, num_kv_heads=4, head_dim=128, dtype="fp8",
                 extra_blocks=4)
    W.with_next_token(f, f.unused_blocks)
    both_ways(f, "fp8")
    m = W.custom(803, [33, 600, 1024, 2049], num_q_heads=8, num_kv_heads=2, head_dim=64, extra_blocks=4)
    W.with_next_token(m, m.unused_blocks)
    both_ways(m, "partitioned", variant="mfma", partition_tokens=256)


def test_noalloc_refuses_a_call_past_its_scratch(gpu):
    """A call needing more scratch than the library holds is refused before
    anything runs: the output and the pool are untouched."""
    from paged_kv_cache_37_amd import KVPoolError, ops
    from paged_kv_cache_37_amd._lib import KVP_ERR_WORKSPACE_TOO_SMALL, NOALLOC_SCRATCH_BYTES

    w = W.make(2)
    W.with_next_token(w, w.unused_blocks)
    dev = Dev(w)
    x = step_inputs(w)
    mb = int(x["block_tables"].shape[1])
    need = ops.paged_decode_workspace_bytes(dev.pool, w.num_seqs, w.num_q_heads, mb, 16)
    assert need > NOALLOC_SCRATCH_BYTES  # 16-token partitions: one partial result per tile
    before = dev.pool.storage.clone()
    out = torch.full_like(dev.q, 7.0)
    with pytest.raises(KVPoolError) as e:
        ops.paged_decode_step_noalloc(dev.pool, 0, dev.q, x["block_tables"], x["seq_lens"], w.scale, x["k_new"],
                                      x["v_new"], x["slot_mapping"], out, variant="mfma", partition_tokens=16)
    torch.cuda.synchronize()
    assert e.value.status == KVP_ERR_WORKSPACE_TOO_SMALL
    assert "no-allocation" in str(e.value)
    assert torch.equal(dev.pool.storage, before)
    assert torch.all(out == 7.0)
