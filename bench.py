"""Benchmark of the paged decode hot path on one MI355X.

A step is one decode step of one layer for the whole batch: the write of
every sequence's new token into its slot, then paged decode attention of
every sequence over its context (new token included): one
paged_decode_step call (the streaming kernel fuses the write), or with
--unfused a cache_write call and a paged_decode_attention call.  Steps rotate over
`--layers` layer slices of one pool so that the KV read each step is not
served from the 256 MB last-level cache.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--kv-dtype bf16|fp8]
                    [--block-size 16|32]
    python bench.py --mode prefill [...]   # the chunked-prefill step (config 7)

Prints one JSON line.  `value` is the step's algorithmic bytes (K/V of the
attended slots, each physical slot once, queries, outputs, tables, the
written K/V) per second;
`roofline` relates the timed call's algorithmic bytes to its average
duration and the 8 TB/s HBM peak: the fused step's from the HIP events
around the K back-to-back steps on the launch stream (the pass that also
gives `value`); with --unfused the attention call's, from events around
each call in a second pass of the same K steps (`call_us` in the line is
always that second pass's per-call figure);
`cpu_baseline` times the CPU oracle on a bounded sample of the same batch.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention: achieved HBM GB/s (% of peak) + seq·layer steps/s"
PREFILL_METRIC = "paged prefill attention: achieved TFLOP/s (% of dense bf16 MFMA peak) + tokens/s"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 (no sparsity)
DEFAULT_LAYERS = {1: 1, 2: 2, 3: 1, 4: 4, 5: 2, 6: 1}  # layer slices so that each step reads >= ~1 GB
KERNEL_SOURCES = ("decode_stream.hip", "stream_body.inc", "prefill.hip", "prefill_body.inc", "prefill_common.h",
                  "copy_blocks.hip", "decode_mfma.hip", "decode_valu.hip", "decode_reduce.hip", "cache_write.hip",
                  "mfma_tile.h", "decode_common.h", "internal.h", "fp8.h", "kvpool_api.cpp")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def _code_only(src: str) -> str:
    """Source text without comments and blank space, so that a comment edit
    does not mark the profiled kernels as changed (string literals in these
    files hold no comment markers)."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_37_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def profile_slug(workload_name: str) -> str:
    """File-name form of a workload name (profiles/ are named kernel.workload.*)."""
    return workload_name.replace("/", "-").replace("..", "-")


def traffic_from_profiles(workload_name: str, label: str):
    """Counter-measured HBM bytes per timed call, if the profiles were taken
    on the current kernel sources (`label` names the call: decode_<variant>
    for the attention call, decode_<variant>_step for the fused step)."""
    path = os.path.join(ROOT, "profiles", f"{label}.{profile_slug(workload_name)}.traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_hash") != kernel_hash() or rec.get("label", rec.get("variant")) != label:
        return None
    return rec.get("hbm_bytes_per_call")


def copy_probe(mib: int) -> None:
    """A plain device-to-device copy of known size (counter calibration)."""
    import torch

    n = mib * (1 << 20)
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copied {mib} MiB x3")


def attended_slots(w) -> int:
    """Distinct physical slots the step's attention reads (after the
    next-token write): each sequence's attended positions mapped through
    its table, union over sequences."""
    import numpy as np

    slots = []
    for s in range(w.num_seqs):
        ctx = int(w.seq_lens_after[s])
        first = max(0, ctx - w.window) if w.window else 0
        B = w.block_size
        so = first % B
        idx = np.arange(so, so + ctx - first)
        slots.append(w.block_tables_after[s][idx // B].astype(np.int64) * B + idx % B)
    return int(np.unique(np.concatenate(slots)).size) if slots else 0


# The CPU baseline runs the oracle in forked worker processes, one per host
# core, BLAS at one thread each.  It runs before the process touches the GPU,
# so no worker inherits a device context.  The box gives one GPU's job 16
# cores whatever the affinity mask shows, hence the cap.
MAX_BASELINE_WORKERS = 16
_BASELINE = {}  # what the forked workers read: the workload and the work function


def baseline_cores() -> int:
    return max(1, min(len(os.sched_getaffinity(0)), MAX_BASELINE_WORKERS))


def _baseline_worker(args):
    """One worker: units i, i + n, i + 2n, ... of the sample (cycling) until
    the shared deadline; returns (units done, work done, seconds)."""
    from threadpoolctl import threadpool_limits

    i, n, deadline = args
    fn, units = _BASELINE["fn"], _BASELINE["units"]
    done, work = 0, 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        k = i
        while time.time() < deadline:
            work += fn(units[k % len(units)])
            done += 1
            k += n
        return done, work, time.perf_counter() - t0


def run_cpu_baseline(fn, units, budget_s: float):
    """Run fn(unit) (returning its work: bytes or FLOPs) over `units` on
    every baseline core for about budget_s seconds.  Returns (units done,
    work done, wall seconds, cores, mean per-core rate)."""
    import multiprocessing

    cores = baseline_cores()
    _BASELINE.update(fn=fn, units=units)
    with multiprocessing.get_context("fork").Pool(cores) as pool:
        pool.map(abs, range(cores))  # workers up before the clock starts
        t0 = time.time()
        res = pool.map(_baseline_worker, [(i, cores, t0 + budget_s) for i in range(cores)])
        wall = time.time() - t0
    _BASELINE.clear()
    done = sum(r[0] for r in res)
    work = sum(r[1] for r in res)
    per_core = sum(r[1] / r[2] for r in res if r[2] > 0) / cores
    return done, work, wall, cores, per_core


def cpu_baseline(w, budget_s: float = 10.0) -> dict:
    """Time the CPU oracle (as it is) on whole sequences of the batch, one
    sequence per task, on every host core for about `budget_s` seconds."""
    import oracle

    per_token = 2 * w.num_kv_heads * w.head_dim * w.elt_bytes
    valid = w.valid_tokens()

    def one_sequence(s):
        oracle.decode_attention_seq(w.pool, 0, w.q[s], w.block_tables[s], int(w.seq_lens[s]), w.window,
                                    w.scale, k_scale=w.k_scale, v_scale=w.v_scale)
        return int(valid[s]) * per_token

    done, kv_bytes, dt, cores, per_core = run_cpu_baseline(one_sequence, list(range(w.num_seqs)), budget_s)
    return {
        "value": kv_bytes / dt / 1e9,
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{done} sequence-layer steps ({done / w.num_seqs:.2f} passes over the {w.num_seqs} sequences, "
                  f"all {w.num_q_heads} query heads, layer 0; fp64 numpy in {cores} worker processes, BLAS one "
                  f"thread each): {done / dt:.2f} seq-layer steps/s",
        "seconds": round(dt, 3),
        "per_core_value": round(per_core / 1e9, 4),
    }


def prefill_flops(w) -> int:
    """Algorithmic FLOPs of one prefill call: per query token and query
    head, 2 D multiply-adds per attended key for q.K and 2 D for p.V."""
    import numpy as np

    keys = 0
    for s in range(w.num_seqs):
        ctx, q_len = int(w.seq_lens[s]), int(w.q_lens[s])
        p = ctx - q_len + np.arange(q_len)
        lo = np.maximum(0, p + 1 - w.window) if w.window else np.zeros_like(p)
        keys += int(np.maximum(p - lo + 1, 0).sum())
    return 4 * w.head_dim * w.num_q_heads * keys


def cpu_baseline_prefill(w, budget_s: float = 10.0) -> dict:
    """The prefill oracle (as it is) on a bounded sample: one chunk token of
    one sequence per task (all heads; the tokens of a chunk spread evenly),
    on every host core for about budget_s seconds."""
    import oracle

    units = []
    for k in range(8):
        for s in range(w.num_seqs):
            q_len = int(w.q_lens[s])
            if q_len:
                units.append((s, (k * q_len) // 8))

    def one_token(u):
        s, i = u
        a, q_len, ctx = int(w.cu_q_lens[s]), int(w.q_lens[s]), int(w.seq_lens[s])
        oracle.prefill_attention_seq(w.pool, 0, w.q[a:a + q_len], w.block_tables[s], ctx, w.window,
                                     w.scale, k_scale=w.k_scale, v_scale=w.v_scale, tokens=[i])
        p = ctx - q_len + i
        lo = max(0, p + 1 - w.window) if w.window else 0
        return 4 * w.head_dim * w.num_q_heads * (p - lo + 1)

    done, flops, dt, cores, per_core = run_cpu_baseline(one_token, units, budget_s)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{done} query tokens (all {w.num_q_heads} heads, eight spread over each chunk; fp64 numpy in "
                  f"{cores} worker processes, BLAS one thread each): {done / dt:.1f} tokens/s",
        "seconds": round(dt, 3),
        "per_core_value": round(per_core / 1e12, 6),
    }


def bench_prefill(args) -> int:
    """One step = paged_prefill_step of the whole chunked-prefill batch on
    one layer slice: the chunks' K/V stored into their slots, then causal
    attention of every chunk token over its context."""
    import numpy as np
    import torch

    import workloads as W

    dev = torch.device("cuda:0")
    L = args.layers or (8 if args.kv_dtype == "bf16" else 16)
    log(f"generating the chunked-prefill batch with {L} layer slice(s)")
    w = W.prefill_config(num_layers=L, dtype=args.kv_dtype, block_size=args.block_size)
    log(f"generated: {w.name}, {w.num_blocks} blocks/layer")
    baseline = None
    if not args.no_cpu_baseline:  # before the GPU is touched (the workers are forked)
        log(f"timing the CPU oracle on {baseline_cores()} cores")
        baseline = cpu_baseline_prefill(w)
    from paged_kv_cache_37_amd import ops
    pool_dt = {"bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[w.dtype]
    pool = ops.KVPool(L, w.num_blocks, w.num_kv_heads, w.head_dim, pool_dt, dev, block_size=w.block_size)
    if w.dtype == "bf16":
        pool.load_logical(torch.from_numpy(w.pool.view(np.int16)).view(torch.bfloat16))
    else:
        pool.load_logical(torch.from_numpy(w.pool))
        for layer in range(L):
            pool.set_fp8_scales(layer, w.k_scale, w.v_scale)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    T = int(w.cu_q_lens[-1])
    q = up(w.q)
    rng = np.random.default_rng(7)
    k_new = up(W.f32_to_bf16_bits(rng.standard_normal((T, w.num_kv_heads, w.head_dim)).astype(np.float32)))
    v_new = up(W.f32_to_bf16_bits(rng.standard_normal((T, w.num_kv_heads, w.head_dim)).astype(np.float32)))
    B = w.block_size
    slots = np.empty(T, np.int32)
    for s in range(w.num_seqs):
        ctx, q_len = int(w.seq_lens[s]), int(w.q_lens[s])
        for i in range(q_len):
            p = ctx - q_len + i
            slots[w.cu_q_lens[s] + i] = w.block_tables[s][p // B] * B + p % B
    slots_t = torch.from_numpy(slots).to(dev)
    cu = torch.from_numpy(w.cu_q_lens).to(dev)
    tables = torch.from_numpy(np.ascontiguousarray(w.block_tables)).to(dev)
    lens = torch.from_numpy(np.ascontiguousarray(w.seq_lens)).to(dev)
    out = torch.empty_like(q)
    mq = int(max(w.q_lens))
    stream = torch.cuda.current_stream(dev)

    def step(i):
        ops.paged_prefill_step(pool, i % L, q, cu, tables, lens, w.scale, mq, k_new, v_new, slots_t, out=out,
                               stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(K):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / K
    # per-call events: the write, then the attention
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for i in range(K):
        ev[i][0].record(stream)
        ops.cache_write(pool, i % L, k_new, v_new, slots_t, stream=stream)
        ev[i][1].record(stream)
        ops.paged_prefill_attention(pool, i % L, q, cu, tables, lens, w.scale, mq, out=out, stream=stream)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    write_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    attn_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / K
    log(f"step {ms_per_step * 1e3:.1f} us; per call (write {write_ms * 1e3:.1f} us, attention {attn_ms * 1e3:.1f} us)")
    flops = prefill_flops(w)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (attn_ms * 1e-3) / 1e12
    result = {
        "metric": PREFILL_METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "fp8 KV, bf16 MFMA",
        "data": "synthetic",
        "config": {
            "workload": w.name, "kv_dtype": w.dtype, "num_seqs": w.num_seqs, "chunk_tokens": T,
            "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
            "block_size": w.block_size, "prior_tokens": [int(x) for x in w.prior], "layer_slices": L,
            "seed": w.seed,
        },
        "tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
        "attention_us": round(attn_ms * 1e3, 2),
        "cache_write_us": round(write_ms * 1e3, 2),
        "flops_per_call": flops,
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": traffic_from_profiles(w.name, "prefill"),
            "kernel": "paged_prefill_attention (prefill_kernel)",
            "flops_per_call": flops,
        },
        "cpu_baseline": baseline,
    }
    print(json.dumps(result), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--mode", default="decode", choices=["decode", "prefill"],
                    help="decode (the default step) or the chunked-prefill step")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, choices=[2, 3, 4, 5, 6],
                    help="2..5 as in the workload generator; 6 = 16 long contexts (32k..40k tokens)")
    ap.add_argument("--kv-dtype", default="bf16", choices=["bf16", "fp8"],
                    help="pool storage: bf16, or FP8 E4M3 codes with per-layer scales")
    ap.add_argument("--block-size", type=int, default=16, choices=[16, 32], help="tokens per KV block")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--layers", type=int, default=None, help="layer slices to rotate over")
    ap.add_argument("--variant", default="auto", choices=["auto", "stream", "mfma", "valu"])
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--no-shared-prefix", action="store_true",
                    help="do not pass the batch's shared prefix (cascade) to the library")
    ap.add_argument("--unfused", action="store_true",
                    help="time cache_write and paged_decode_attention as two calls instead of paged_decode_step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a device copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (each GPU would run "
              "the same kernels on its own sequences or KV heads); run it with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.copy_probe:
        copy_probe(args.copy_probe)
        return 0
    if args.mode == "prefill":
        return bench_prefill(args)

    import workloads as W

    dev = torch.device("cuda:0")
    # an FP8 pool holds half the bytes per layer: twice the slices for the same footprint
    L = args.layers or DEFAULT_LAYERS[args.config] * (2 if args.kv_dtype == "fp8" else 1)
    log(f"generating config {args.config} with {L} layer slice(s)")
    t0 = time.time()
    w = W.make(args.config, args.seed, num_layers=L, dtype=args.kv_dtype, block_size=args.block_size)
    W.with_next_token(w, w.unused_blocks)
    log(f"generated in {time.time() - t0:.1f}s: {w.name}, {w.num_blocks} blocks/layer")
    baseline = None
    if not args.no_cpu_baseline:  # before the GPU is touched (the workers are forked)
        log(f"timing the CPU oracle on {baseline_cores()} cores")
        baseline = cpu_baseline(w)
    from paged_kv_cache_37_amd import ops
    from paged_kv_cache_37_amd.blockpool import rows_share_blocks, shared_prefix_blocks

    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16  # queries, outputs, new tokens
    pool_dt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[w.dtype]

    def up(a):
        a = np.ascontiguousarray(a)
        if dt == torch.bfloat16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    pool = ops.KVPool(L, w.num_blocks, w.num_kv_heads, w.head_dim, pool_dt, dev, block_size=w.block_size)
    if w.dtype == "bf16":
        pool.load_logical(torch.from_numpy(w.pool.view(np.int16)).view(torch.bfloat16))
    else:
        pool.load_logical(torch.from_numpy(w.pool))  # float32 values or uint8 codes
    if w.dtype == "fp8":
        for layer in range(L):
            pool.set_fp8_scales(layer, w.k_scale, w.v_scale)
    q = up(w.q)
    k_new, v_new = up(w.k_new), up(w.v_new)
    slots = torch.from_numpy(w.slot_mapping).to(dev)
    tables = torch.from_numpy(w.block_tables_after).to(dev)
    lens = torch.from_numpy(w.seq_lens_after).to(dev)
    out = torch.empty_like(q)
    ws = ops.make_workspace(pool, w.num_seqs, w.num_q_heads, tables.shape[1], args.partition_tokens)
    # blocks every row shares (a cached prompt prefix): attended once for the batch
    shared = 0 if args.no_shared_prefix else shared_prefix_blocks(np.asarray(w.block_tables_after), w.seq_lens_after,
                                                                  block_size=w.block_size)
    # blocks listed by several rows past that prefix: tiles read with cached loads
    reuse = rows_share_blocks(np.asarray(w.block_tables_after), w.seq_lens_after, prefix_blocks=shared,
                              block_size=w.block_size, window=w.window)
    log(f"shared prefix: {shared} blocks; other blocks shared between rows: {reuse}")
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()

    def write(layer):
        ops.cache_write(pool, layer, k_new, v_new, slots, stream=stream)

    def attend(layer):
        ops.paged_decode_attention(pool, layer, q, tables, lens, w.scale, out=out, sliding_window=w.window,
                                   partition_tokens=args.partition_tokens, variant=args.variant, workspace=ws,
                                   stream=stream, shared_prefix_blocks=shared, shared_blocks=reuse)

    def fused(layer):
        ops.paged_decode_step(pool, layer, q, tables, lens, w.scale, k_new, v_new, slots, out=out,
                              sliding_window=w.window, partition_tokens=args.partition_tokens, variant=args.variant,
                              workspace=ws, stream=stream, shared_prefix_blocks=shared, shared_blocks=reuse)

    def step(i):
        if args.unfused:
            write(i % L)
            attend(i % L)
        else:
            fused(i % L)

    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Pass 1 (the bench value): K steps back to back, timed as a whole.
    K = args.steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"timing {K} steps")
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / K

    # Pass 2 (the roofline): the same K steps with events around each call.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        layer = i % L
        ev[i][0].record(stream)
        if args.unfused:
            write(layer)
            ev[i][1].record(stream)
            attend(layer)
        else:
            ev[i][1].record(stream)
            fused(layer)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    write_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    call_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / K  # the attention call, or the fused step call
    log(f"step {ms_per_step * 1e3:.1f} us; per call ("
        + (f"write {write_ms * 1e3:.1f} us, attention {call_ms * 1e3:.1f} us)" if args.unfused
           else f"fused write + attention {call_ms * 1e3:.1f} us)"))

    # algorithmic bytes: K/V of every attended slot counted once (a prefix
    # block shared by many sequences is one physical block: HBM serves it
    # once), plus queries, outputs, table rows and lengths
    S, Hq, D, Hkv, eb = w.num_seqs, w.num_q_heads, w.head_dim, w.num_kv_heads, w.elt_bytes
    ab = 4 if w.dtype == "f32" else 2  # bytes of a query, output or new-token element
    valid_after = np.minimum(w.seq_lens_after, w.window) if w.window else w.seq_lens_after
    per_token = 2 * Hkv * D * eb
    kv_logical = int(valid_after.astype(np.int64).sum()) * per_token
    kv_read = attended_slots(w) * per_token
    other = 2 * S * Hq * D * ab + int(np.asarray(w.row_blocks_after).sum()) * 4 + S * 4
    attn_bytes = kv_read + other
    write_bytes = 2 * S * Hkv * D * (ab + eb) + S * 4  # new K/V read, stored into the pool
    step_bytes = attn_bytes + write_bytes
    call_bytes = attn_bytes if args.unfused else step_bytes
    # the timed call's average duration: for the fused step the step itself,
    # from the events around the K back-to-back calls of the first pass (no
    # events between calls); for --unfused the attention call between its
    # own events
    roof_ms = call_ms if args.unfused else ms_per_step
    achieved = call_bytes / (roof_ms * 1e-3) / 1e9
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    variant = args.variant
    if variant == "auto":
        variant = "valu" if w.dtype == "f32" else ("mfma" if args.partition_tokens else "stream")
    path = "cascade" if shared and variant == "stream" and not w.window else variant
    label = f"decode_{path}" if args.unfused else f"decode_{path}_step"
    # the streaming launch merges cut rows itself when no row crosses an XCD
    # (KV heads a multiple of 8, one head group per KV head, no shared prefix)
    one_launch = (variant == "stream" and not shared and w.num_kv_heads % 8 == 0
                  and w.num_q_heads // w.num_kv_heads <= 16 and os.environ.get("KVP_LAUNCH_MERGE", "1") != "0")
    merge = "merged in the same launch" if one_launch else "merge launches"
    kernel = (f"paged_decode_attention (decode, {merge})" if args.unfused else
              "paged_decode_step (" + (f"fused write + decode, {merge})" if variant == "stream"
                                       else "cache_write, decode, merge launches)"))

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "kv_dtype": w.dtype,
            "num_seqs": S,
            "num_q_heads": Hq,
            "num_kv_heads": Hkv,
            "head_dim": D,
            "block_size": w.block_size,
            "context_tokens_total": int(valid_after.sum()),
            "sliding_window": w.window,
            "layer_slices": L,
            "variant": variant,
            "partition_tokens": args.partition_tokens,
            "fused_step": not args.unfused,
            "shared_prefix_blocks": shared,
            "shared_blocks": bool(reuse),
            "seed": w.seed,
        },
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "seq_layer_steps_per_s": round(S / (ms_per_step * 1e-3), 1),
        "call_us": round(call_ms * 1e3, 2),
        "attention_us": round(call_ms * 1e3, 2) if args.unfused else None,
        "cache_write_us": round(write_ms * 1e3, 2) if args.unfused else None,
        "kv_bytes_logical": kv_logical,
        "kv_bytes_unique": kv_read,
        "logical_kv_gbs": round(kv_logical / (call_ms * 1e-3) / 1e9, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_from_profiles(w.name, label),
            "kernel": kernel,
            "bytes_per_call": call_bytes,
            "call_us": round(roof_ms * 1e3, 2),
        },
        "cpu_baseline": baseline,
    }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
