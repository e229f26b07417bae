"""Needle and anti-needle probes at full size, through the default (streaming)
path and the fused decode step, on the Llama-3-8B-shaped, 70B-shaped,
sliding-window and long-context batches.

A needle makes one key win a query head's softmax by a margin the fp32
arithmetic cannot blur: q_h = 32 e_d and K[t*] = 32 e_d give a score of
1024 scale = 90.5 at head_dim 128, against at most ~13 for N(0,1) keys, so
every other weight is below e^-77 and the output is V[t*] bit for bit.  Each
query head of a group gets its own needle (its own dimension d), placed at
the row's first and last attended positions and on both sides of the
boundaries where the streaming kernel's equal split of the tile list cuts the
row between waves (so rows cut into many pieces, merged in several rounds,
are probed).  A block read from the wrong place, dropped, or merged from the
wrong piece returns another row's value: O(1) error, not an ulp.
Anti-needles (keys of twice the needle's score) fill the unattended slots of
each row's last block and, under a window, the slots before its first
position: reading any of them would win the softmax.

The row layout the wave boundaries are computed from is the streaming
kernel's: rows ordered (KV head, sequence), one tile per 16 tokens, the tile
list split into equal ranges over (compute units x 2 workgroups x 4 waves).
If the grid differs, the needles land elsewhere in the rows and the probe
stays exact, only less pointed.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import Dev, host_to_torch, say, to_f64, torch_to_bits, ulp_bf16

pytestmark = pytest.mark.gpu

NEEDLE = 32.0
ANTI = 64.0
_CACHE = {}


def workload(config):
    if config not in _CACHE:
        say("generating config", config)
        _CACHE.clear()  # one large batch held at a time
        w = W.make(config)
        W.with_next_token(w, w.unused_blocks)
        _CACHE[config] = w
    return _CACHE[config]


def stream_waves() -> int:
    return torch.cuda.get_device_properties(0).multi_processor_count * 2 * 4


def row_tiles(ctx: int, window: int, B: int = 16):
    """(first attended position, first listed block's first position, tiles) of a row."""
    first = max(0, ctx - window) if window else 0
    base = (first // B) * B
    return first, base, (ctx - base + 15) // 16 if ctx > 0 else 0


def plan_needles(lens, window: int, G: int, Hkv: int, waves: int, B: int = 16):
    """Needle positions [S][Hkv][G] (absolute token positions): the row's
    first and last attended positions, then both sides of each wave
    boundary inside the row, then evenly spread positions."""
    S = len(lens)
    spans = [row_tiles(int(c), window, B) for c in lens]
    per_row = sum(n for *_, n in spans)
    pre = np.concatenate([[0], np.cumsum([n for *_, n in spans])])
    T = per_row * Hkv
    bounds = np.array([(w * T) // waves for w in range(1, waves)], dtype=np.int64)
    pos = np.zeros((S, Hkv, G), dtype=np.int64)
    for s in range(S):
        first, base, nb = spans[s]
        ctx = int(lens[s])
        for k in range(Hkv):
            a = k * per_row + pre[s]
            inside = bounds[(bounds > a) & (bounds < a + nb)] - a  # first tile of a wave, in the row
            if len(inside):  # rows take turns at which of their boundaries come first
                r = (s * Hkv + k) % len(inside)
                inside = np.concatenate([inside[r:], inside[:r]])
            cands = [first, ctx - 1]
            for j in inside:
                cands += [base + 16 * int(j) - 1, base + 16 * int(j)]
            cands = [p for p in dict.fromkeys(cands) if first <= p < ctx]
            spread = [first + (ctx - first) * (i + 1) // (G + 1) for i in range(G)]
            while len(cands) < G:
                cands.append(spread[len(cands)])
            pos[s, k] = cands[:G]
    return pos


def needle_dims(G: int, D: int, s: int, k: int):
    return [(7 * g + 3 * k + s) % D for g in range(G)]


class Rows:
    """Element offsets of whole K or V rows of a pool on the device (row base
    from kv_pool_offset, dims at the stride it shows)."""

    def __init__(self, pool):
        self.pool = pool
        D = pool.head_dim
        o0, o1, oL = (pool.offset(0, 0, kv, 0, 0, d) for kv in (0,) for d in (0, 1, D - 1))
        self.k_stride = o1 - o0
        assert oL == o0 + (D - 1) * self.k_stride

    def k_index(self, blocks, heads, slots) -> torch.Tensor:
        D = self.pool.head_dim
        base = np.array([self.pool.offset(0, int(b), 0, int(h), int(t), 0) for b, h, t in zip(blocks, heads, slots)],
                        dtype=np.int64)
        return torch.from_numpy(base[:, None] + self.k_stride * np.arange(D)[None, :])


def plant(w, dev: Dev, lens, tables, new_token: bool):
    """Write needles and anti-needles into dev's pool (K rows only) and build
    the queries; returns (q, expected output bits, k_new or None).  With
    new_token the fused step's new token (at lens[s] - 1) may be a needle:
    its key comes from the returned k_new."""
    S, Hq, D, Hkv, B = w.num_seqs, w.num_q_heads, w.head_dim, w.num_kv_heads, w.block_size
    G = Hq // Hkv
    pos = plan_needles(lens, w.window, G, Hkv, stream_waves(), B)
    q = np.zeros((S, Hq, D), dtype=np.uint16)
    expect = np.zeros((S, Hq, D), dtype=np.uint16)
    one = W.f32_to_bf16_bits(np.array([NEEDLE], np.float32))[0]
    big = W.f32_to_bf16_bits(np.array([ANTI], np.float32))[0]
    k_new = w.k_new.copy() if new_token else None
    rows_b, rows_h, rows_t, rows_v = [], [], [], []
    for s in range(S):
        ctx = int(lens[s])
        first, base, nb = row_tiles(ctx, w.window, B)
        fb = first // B
        for k in range(Hkv):
            dims = needle_dims(G, D, s, k)
            key_rows = {}
            for g in range(G):
                p = int(pos[s, k, g])
                key_rows.setdefault(p, []).append(dims[g])
                q[s, k * G + g, dims[g]] = one
                if new_token and p == ctx - 1:
                    expect[s, k * G + g] = w.v_new[s, k]
                else:
                    blk = int(tables[s][p // B - fb])
                    expect[s, k * G + g] = w.pool[0, blk, 1, p % B, k]
            for p, ds in key_rows.items():
                row = np.zeros(D, np.uint16)
                row[ds] = one
                if new_token and p == ctx - 1:
                    k_new[s, k] = row
                    continue
                rows_b.append(int(tables[s][p // B - fb])), rows_h.append(k), rows_t.append(p % B)
                rows_v.append(row)
            anti = np.zeros(D, np.uint16)
            anti[dims] = big
            last_blk = int(tables[s][nb - 1]) if B == 16 else None
            for t in range((ctx % B) or B, B):  # past the row's last token
                rows_b.append(last_blk), rows_h.append(k), rows_t.append(t), rows_v.append(anti)
            for t in range(first - fb * B):      # before a window's first position
                rows_b.append(int(tables[s][0])), rows_h.append(k), rows_t.append(t), rows_v.append(anti)
    rows = Rows(dev.pool)
    idx = rows.k_index(rows_b, rows_h, rows_t).to("cuda")
    vals = torch.from_numpy(np.stack(rows_v).view(np.int16)).to("cuda")
    flat = dev.pool.flat().view(torch.int16)
    flat[idx.reshape(-1)] = vals.reshape(-1)
    torch.cuda.synchronize()
    say(f"planted {len(rows_b)} K rows ({S} seqs x {Hkv} KV heads x {G} needles + anti-needles)")
    return host_to_torch(q, torch.bfloat16).cuda(), expect, k_new


def check_bits(out: torch.Tensor, expect: np.ndarray, what: str):
    got = torch_to_bits(out)
    bad = np.argwhere(np.any(got != expect, axis=-1))
    say(what, f"{len(bad)} rows differ of {expect.shape[0] * expect.shape[1]}")
    assert bad.size == 0, f"{what}: needle rows differ at (seq, head) {bad[:8].tolist()}"


@pytest.mark.parametrize("config", [2, 3, 5, 6])
def test_full_size_needles_attention(gpu, config):
    """paged_decode_attention (default path: the streaming kernel) returns
    every needle's value bit for bit, anti-needles untouched."""
    w = workload(config)
    say("needles, attention, config", config)
    dev = Dev(w)
    q, expect, _ = plant(w, dev, w.seq_lens, w.block_tables, new_token=False)
    out = dev.attend(q=q)
    check_bits(out, expect, f"config {config} attention")


@pytest.mark.parametrize("config", [2, 3, 5, 6])
def test_full_size_needles_fused_step(gpu, config):
    """paged_decode_step (the new token stored and attended in one launch):
    needles in the pool and in the new token itself come back bit for bit."""
    w = workload(config)
    say("needles, fused step, config", config)
    dev = Dev(w)
    q, expect, k_new = plant(w, dev, w.seq_lens_after, w.block_tables_after, new_token=True)
    out = dev.ops.paged_decode_step(
        dev.pool, 0, q, torch.from_numpy(np.ascontiguousarray(w.block_tables_after)).cuda(),
        torch.from_numpy(w.seq_lens_after).cuda(), w.scale, host_to_torch(k_new, torch.bfloat16).cuda(),
        host_to_torch(w.v_new, torch.bfloat16).cuda(), torch.from_numpy(w.slot_mapping).cuda(),
        sliding_window=w.window)
    torch.cuda.synchronize()
    check_bits(out, expect, f"config {config} fused step")


@pytest.mark.parametrize("config", [3, 5, 6])
def test_stream_matches_partitioned(gpu, config):
    """The streaming kernel (rows cut wherever the equal split falls, pieces
    merged in rounds of eight) and the partitioned kernel (512-token
    partitions, then the split-K reduce) agree to one bf16 ulp plus fp32
    accumulation-order noise (1e-5 of the row's rms) on every output."""
    w = workload(config)
    say("stream vs partitioned, config", config)
    dev = Dev(w)
    a = to_f64(dev.attend(variant="stream"))
    b = to_f64(dev.attend(variant="mfma", partition_tokens=512))
    rms = np.sqrt(np.mean(a ** 2, axis=-1, keepdims=True))
    bound = np.maximum(ulp_bf16(a), ulp_bf16(b)) + 1e-5 * rms
    ratio = np.abs(a - b) / bound
    say(f"config {config}: max |stream - partitioned| / bound = {float(ratio.max()):.3f}")
    assert np.all(ratio <= 1.0)
