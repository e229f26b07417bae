"""The decode and prefill calls under HIP graph capture: the library
allocates nothing and launches only on the caller's stream, so a serving
loop can capture a step once and replay it.  Each test captures one call
into a graph, then replays it several times with new queries written into
the captured input, eager work and synchronisations between the replays,
and checks every replay bit for bit against an eager call on the same
inputs (the same kernels on the same data), and the eager call against the
oracle once."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import Dev, compare, host_to_torch, pool_dtype, reference, say, torch_dtype

pytestmark = pytest.mark.gpu

REPLAYS = 4


def bits(t):
    return t.view(torch.int16).clone()


def replay_and_check(call, q, fresh_q, what):
    """call(out) launches on the current stream; q is the captured input."""
    torch.cuda.synchronize()
    out_g = torch.empty_like(q)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out_g)
    torch.cuda.synchronize()
    out_e = torch.empty_like(q)
    for r in range(REPLAYS):
        q.copy_(fresh_q(r))
        g.replay()
        torch.cuda.synchronize()
        got = bits(out_g)
        call(out_e)  # eager, same inputs
        torch.cuda.synchronize()
        assert torch.equal(got, bits(out_e)), f"{what}: replay {r} differs from the eager call"
    say(what, "replays", REPLAYS, "bit-identical")
    return out_e


def queries(w, dt, seed):
    rng = np.random.default_rng(seed)
    shape = w.q.shape
    return lambda r: torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(dt).cuda()


@pytest.mark.parametrize("dtype,prefix", [("bf16", 0), ("fp8", 0), ("bf16", 64)])
def test_fused_step_in_a_graph(gpu, dtype, prefix):
    """The fused write-then-attend step (streaming kernel + merge; with a
    shared prefix also the prefix pass), replayed: the new tokens are
    written again into the same slots, so every replay sees the same pool."""
    if prefix:
        w = W.shared_prefix(7300, prefix * 16, [0, 1, 15, 16, 17, 100, 300, 7], 8, 2, 128)
    else:
        w = W.custom(7301, [1, 15, 16, 17, 100, 300, 1000, 2500], num_q_heads=8, num_kv_heads=2, head_dim=128,
                     dtype=dtype, extra_blocks=8)
    W.with_next_token(w, w.unused_blocks)
    say("graph: fused step", dtype, "prefix", prefix)
    dev = Dev(w)
    dt = torch_dtype(w)
    tables = torch.from_numpy(np.ascontiguousarray(w.block_tables_after)).cuda()
    lens = torch.from_numpy(w.seq_lens_after).cuda()
    k_new, v_new = host_to_torch(w.k_new, dt).cuda(), host_to_torch(w.v_new, dt).cuda()
    slots = torch.from_numpy(w.slot_mapping).cuda()
    q = dev.q.clone()
    ws = dev.ops.make_workspace(dev.pool, w.num_seqs, w.num_q_heads, tables.shape[1])

    def call(out):
        dev.ops.paged_decode_step(dev.pool, 0, q, tables, lens, w.scale, k_new, v_new, slots, out=out,
                                  workspace=ws, shared_prefix_blocks=prefix)

    call(torch.empty_like(q))  # eager warm-up (sizes the grid outside the capture)
    out = replay_and_check(call, q, queries(w, dt, 1), f"fused step {dtype} prefix {prefix}")
    pool_ref = oracle.cache_write(w.pool, 0, w.k_new, w.v_new, w.slot_mapping, w.k_scale, w.v_scale)
    # the last replay's queries are in q
    ref = reference(w, pool=pool_ref, q=W.f32_to_bf16_bits(q.float().cpu().numpy()), tables=w.block_tables_after,
                    lens=w.seq_lens_after)
    compare(out, ref, "bf16", f"graph fused step {dtype} prefix {prefix}")


def test_split_partitions_in_a_graph(gpu):
    """The partitioned matrix-core kernel with its reduce kernel (rows split
    into 256-token partitions), replayed."""
    w = W.custom(7302, [0, 1, 40, 255, 256, 257, 1500, 3000], num_q_heads=16, num_kv_heads=2, head_dim=128)
    say("graph: partitioned")
    dev = Dev(w)
    q = dev.q.clone()
    ws = dev.ops.make_workspace(dev.pool, w.num_seqs, w.num_q_heads, dev.tables.shape[1], 256)

    def call(out):
        dev.ops.paged_decode_attention(dev.pool, 0, q, dev.tables, dev.lens, w.scale, out=out, partition_tokens=256,
                                       variant="mfma", workspace=ws)

    call(torch.empty_like(q))
    out = replay_and_check(call, q, queries(w, torch.bfloat16, 2), "partitioned mfma")
    compare(out, reference(w, q=W.f32_to_bf16_bits(q.float().cpu().numpy())), "bf16", "graph partitioned")


def test_prefill_in_a_graph(gpu):
    """Chunked-prefill attention, replayed."""
    w = W.prefill_batch(7303, [0, 17, 300, 1000], [1, 64, 129, 200], 8, 2, 128)
    say("graph: prefill")
    from paged_kv_cache_37_amd import ops

    pool = ops.KVPool(1, w.num_blocks, w.num_kv_heads, w.head_dim, pool_dtype(w), "cuda:0", block_size=w.block_size)
    pool.load_logical(host_to_torch(w.pool, pool_dtype(w)))
    q = host_to_torch(w.q, torch.bfloat16).cuda()
    cu = torch.from_numpy(w.cu_q_lens).cuda()
    tables = torch.from_numpy(np.ascontiguousarray(w.block_tables)).cuda()
    lens = torch.from_numpy(np.ascontiguousarray(w.seq_lens)).cuda()
    mq = int(max(w.q_lens))

    def call(out):
        ops.paged_prefill_attention(pool, 0, q, cu, tables, lens, w.scale, mq, out=out)

    call(torch.empty_like(q))
    out = replay_and_check(call, q, queries(w, torch.bfloat16, 3), "prefill")
    qb = W.f32_to_bf16_bits(q.float().cpu().numpy())
    ref = oracle.prefill_attention(w.pool, 0, qb, w.cu_q_lens, w.block_tables, w.seq_lens, w.window, w.scale)
    compare(out, ref, "bf16", "graph prefill", bar="prefill")
