"""The streaming decode's in-launch merge (cut rows merged by workgroups of
the same launch, on the XCD whose waves wrote the pieces) against the
separate merge kernel (KVP_LAUNCH_MERGE=0): outputs and pool bit-identical,
call after call on one workspace, after the workspace held other contents,
for attention alone, the fused step, FP8 pools and several head shapes; and
against the oracle.  The in-launch merge applies when the KV heads are a
multiple of 8 (with at most 16 query heads each) and no shared prefix is
passed; other shapes take the merge kernel either way."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import Dev, compare, host_to_torch, reference, say, torch_to_bits

pytestmark = pytest.mark.gpu


class merge_kernel:
    """Within the block, calls keep the separate merge kernel."""

    def __enter__(self):
        self.old = os.environ.get("KVP_LAUNCH_MERGE")
        os.environ["KVP_LAUNCH_MERGE"] = "0"

    def __exit__(self, *exc):
        if self.old is None:
            del os.environ["KVP_LAUNCH_MERGE"]
        else:
            os.environ["KVP_LAUNCH_MERGE"] = self.old


def bits(t):
    return torch_to_bits(t)


def step_once(dev, w, ws):
    k = host_to_torch(w.k_new, dev.dt).cuda()
    v = host_to_torch(w.v_new, dev.dt).cuda()
    sl = torch.from_numpy(np.ascontiguousarray(w.slot_mapping)).cuda()
    tb = torch.from_numpy(np.ascontiguousarray(w.block_tables_after)).cuda()
    ln = torch.from_numpy(np.ascontiguousarray(w.seq_lens_after)).cuda()
    out = dev.ops.paged_decode_step(dev.pool, 0, dev.q, tb, ln, w.scale, k, v, sl, sliding_window=w.window,
                                    variant="stream", workspace=ws)
    torch.cuda.synchronize()
    return out


def make(config=None, ctx=None, Hq=32, Hkv=8, D=128, window=0, dtype="bf16", seed=11, step=True):
    """A workload; with step, one next token per sequence (the *_after
    tables and lengths include it: attention over them needs the write)."""
    if config is not None:
        w = W.make(config, dtype=dtype)
    else:
        w = W.custom(seed, list(ctx), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, dtype=dtype, window=window)
    if step:
        W.with_next_token(w, w.unused_blocks)
    return w


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_step_bit_identical_to_merge_kernel(gpu, dtype):
    """The 8B-shaped batch: the fused step with the in-launch merge equals
    the step with the merge kernel, three calls in a row on one workspace
    (each call clears its marks for the next), and matches the oracle."""
    w = make(config=2, dtype=dtype)
    res = {}
    for mode in ("launch", "kernel"):
        dev = Dev(w)
        ws = dev.ops.make_workspace(dev.pool, w.num_seqs, w.num_q_heads, w.block_tables_after.shape[1])
        outs = []
        for i in range(3):
            if mode == "kernel":
                with merge_kernel():
                    outs.append(bits(step_once(dev, w, ws)))
            else:
                outs.append(bits(step_once(dev, w, ws)))
        res[mode] = (outs, bits(dev.pool.to_logical()))
        if mode == "launch":
            first = step_once(dev, w, ws)  # a fourth call, for the oracle comparison
        del dev
    for i in range(3):
        assert res["launch"][0][i].tobytes() == res["kernel"][0][i].tobytes(), f"call {i}: outputs differ"
        assert res["launch"][0][i].tobytes() == res["launch"][0][0].tobytes(), f"call {i} differs from call 0"
    assert res["launch"][1].tobytes() == res["kernel"][1].tobytes(), "pools differ"
    import oracle
    pool_ref = oracle.cache_write(w.pool, 0, w.k_new, w.v_new, w.slot_mapping, w.k_scale, w.v_scale)
    ref = reference(w, pool=pool_ref, tables=w.block_tables_after, lens=w.seq_lens_after)
    compare(first, ref, w.dtype, f"launch merge step {dtype}")


def test_attention_after_other_workspace_contents(gpu):
    """Attention alone, on a workspace first filled with random bytes and
    then used by a partitioned call (whose partials overwrite it): the
    in-launch merge still equals the merge kernel bit for bit."""
    w = make(config=5, step=False)
    dev = Dev(w)
    tb, ln = dev.tables, dev.lens
    ws = dev.ops.make_workspace(dev.pool, w.num_seqs, w.num_q_heads, tb.shape[1], 512)
    g = torch.Generator(device="cuda").manual_seed(5)
    ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device="cuda", generator=g))
    with merge_kernel():
        ref_bits = bits(dev.attend(tables=tb, lens=ln, variant="stream", workspace=ws))
    dev.attend(tables=tb, lens=ln, variant="mfma", partition_tokens=512, workspace=ws)
    for i in range(2):
        got = bits(dev.attend(tables=tb, lens=ln, variant="stream", workspace=ws))
        assert got.tobytes() == ref_bits.tobytes(), f"call {i}: in-launch merge differs from the merge kernel"
    ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device="cuda", generator=g))
    got = bits(dev.attend(tables=tb, lens=ln, variant="stream", workspace=ws))
    assert got.tobytes() == ref_bits.tobytes(), "after random workspace contents"
    seqs = [0, 7, 31]
    compare(dev.attend(tables=tb, lens=ln, variant="stream", workspace=ws)[seqs], reference(w, seqs=seqs), w.dtype,
            "launch merge, sliding window")


@pytest.mark.parametrize("Hq,Hkv,D,window", [(64, 8, 128, 0), (16, 16, 128, 0), (128, 8, 64, 0), (32, 8, 128, 300),
                                            (24, 8, 64, 0)])
def test_head_shapes(gpu, Hq, Hkv, D, window):
    """Head groups of 8, 1, 16 and 3 per KV head, 8 and 16 KV heads, a
    window: in-launch merge equals the merge kernel; oracle on a sample."""
    rng = np.random.default_rng(Hq * 7 + Hkv + D + window)
    ctx = rng.integers(1, 3000, size=40)
    ctx[:4] = [1, 16, 17, 2999]
    w = make(ctx=ctx, Hq=Hq, Hkv=Hkv, D=D, window=window, seed=Hq + D, step=False)
    dev = Dev(w)
    tb, ln = dev.tables, dev.lens
    with merge_kernel():
        ref_bits = bits(dev.attend(tables=tb, lens=ln, variant="stream"))
    out = dev.attend(tables=tb, lens=ln, variant="stream")
    assert bits(out).tobytes() == ref_bits.tobytes(), "in-launch merge differs from the merge kernel"
    seqs = [0, 1, 2, 3, 17, 39]
    compare(out[seqs], reference(w, seqs=seqs), w.dtype, f"launch merge Hq{Hq}/Hkv{Hkv}/D{D}/W{window}")


def test_graph_replays(gpu):
    """The fused step captured in a HIP graph: replays (the same marks each
    time, cleared by every call) equal eager calls, which equal calls with
    the merge kernel."""
    w = make(config=2)
    dev = Dev(w)
    ws = dev.ops.make_workspace(dev.pool, w.num_seqs, w.num_q_heads, w.block_tables_after.shape[1])
    k = host_to_torch(w.k_new, dev.dt).cuda()
    v = host_to_torch(w.v_new, dev.dt).cuda()
    sl = torch.from_numpy(np.ascontiguousarray(w.slot_mapping)).cuda()
    tb = torch.from_numpy(np.ascontiguousarray(w.block_tables_after)).cuda()
    ln = torch.from_numpy(np.ascontiguousarray(w.seq_lens_after)).cuda()

    def call(out):
        dev.ops.paged_decode_step(dev.pool, 0, dev.q, tb, ln, w.scale, k, v, sl, out=out, variant="stream",
                                  workspace=ws)

    out_e = torch.empty_like(dev.q)
    call(out_e)  # eager warm-up (sizes the grid outside the capture)
    torch.cuda.synchronize()
    with merge_kernel():
        out_k = torch.empty_like(dev.q)
        call(out_k)
        torch.cuda.synchronize()
    assert bits(out_e).tobytes() == bits(out_k).tobytes(), "eager in-launch merge differs from the merge kernel"
    out_g = torch.empty_like(dev.q)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out_g)
    torch.cuda.synchronize()
    for r in range(4):
        g.replay()
        torch.cuda.synchronize()
        assert bits(out_g).tobytes() == bits(out_e).tobytes(), f"replay {r} differs from the eager call"
        call(out_e)  # eager work between replays
        torch.cuda.synchronize()
    say("launch merge: graph replays bit-identical")
