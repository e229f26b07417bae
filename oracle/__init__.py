"""CPU oracle for paged decode attention and the paged cache write.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU
library never calls it and shares no code with it.

Everything here is a plain, slow, obviously correct statement of what the
paged KV cache computes, in float64:

* ``cache_write``  -- scatter each new token's K and V into the slot a slot
  mapping names (slot = physical block * block_size + offset);
* ``copy_blocks`` -- the copy-on-write block copy: every layer's K and V of
  one physical block into another;
* ``fp8`` -- the E4M3 codes of an FP8 KV cache: decode, encode (nearest,
  ties to even, saturating) and the scaled quantization a write applies;
* ``decode_attention`` -- for every sequence, walk its block table, gather
  its keys and values into contiguous arrays, and run softmax(q K^T scale) V
  for every query head;
* ``decode_attention_bruteforce`` -- the same result by per-token address
  translation and scalar loops (tiny inputs only);
* ``prefill_attention`` -- multi-token (prefill / chunked-prefill)
  attention: each query of a sequence's chunk attends, causally, the keys up
  to its own position (``prefill_attention_bruteforce`` is the scalar
  version for tiny inputs);
* ``row_span`` / ``check_tables`` -- how many table entries a sequence owns
  and the rule that only a row's last block (and, under a sliding window,
  its first) may be partial.

Sources (the pages this follows; titles as printed on them):

* [Optimizing] "Optimizing KV Cache Memory Management in vLLM with
  PagedAttention and Dynamic Block Allocation" -- §PagedAttention: Virtual
  Memory for LLMs (logical block index = floor(i / B), offset = i mod B; the
  kernel looks the physical block up in the sequence's block table), §The
  Block Manager and Dynamic Allocation Lifecycle (prefill and decode writes
  into physical blocks; decode appends into the last block while it has
  room), §The Math of the KV Cache Bottleneck (GQA: fewer KV heads than
  query heads), §Copy-on-Write (CoW) for Parallel Sampling and Prefix
  Caching (a writer of a shared block gets a private copy first).
* [Paged] the paged-attention post on zhangchitc.github.io -- §What a
  physical block looks like (a block is [2, block_size, num_kv_heads,
  head_dim] per layer), §Two lookup structures (req_to_blocks is the
  ordered logical-to-physical list).
* [Pool] "How the block pool manages KV memory" -- §Hybrid models get
  groups (a sliding-window layer needs only the blocks inside the last
  window).
* [Memory] "The memory behind the next token" -- §Why the next token needs
  yesterday's state (blocks a window no longer needs are removed; layouts
  depend on the attention backend).

The pages never write the attention formula; the one used is the standard
scaled dot-product attention of one decode query over all cached keys,
softmax(q . K^T * scale) . V, with query head h reading KV head h // G
(G = query heads per KV head).

Each function is pinned by ``tests/test_oracle.py`` against the pages'
worked values, closed forms, invariants and an independent library routine.
"""
from .fp8 import e4m3_decode, e4m3_encode, quantize  # noqa: F401
from .paged import (  # noqa: F401
    cache_write,
    copy_blocks,
    check_tables,
    decode_attention,
    decode_attention_bruteforce,
    decode_attention_seq,
    gather_kv,
    row_span,
    softmax_weights,
    to_f64,
)
from .prefill import chunk_first, prefill_attention, prefill_attention_bruteforce, prefill_attention_seq  # noqa: F401,E501
