"""Host-side bookkeeping of the paged KV pool: which physical block holds
which tokens of which request.  It produces the block tables and slot
mappings the GPU library consumes; it never touches device memory.

Sources (page titles as printed):

* "How the block pool manages KV memory" -- §Blocks, not one buffer for each
  request (a pool of 16-token blocks, a table per request), §Finding a prefix
  again (chained block hashes over full blocks only, lookup stops at the
  first miss, SHA-256), §Eviction (freed blocks keep their hash on a free
  list; a new block comes from its head and only then loses its old hash),
  §Hybrid models get groups (a sliding-window layer keeps only the blocks of
  the last window).
* "Why the KV cache is a pool of 16-token blocks" -- §When memory runs out
  (no free block: the scheduler preempts a request and frees all its
  blocks), §Follow-ups (a per-tenant cache_salt goes into the hash).
* "The memory behind the next token" -- §Sharing requires explicit
  ownership (touch removes a ref-0 block from the free queue before the
  reference count rises; a finished request frees its blocks in reverse
  order; blocks that never got a cache identity are reclaimed first),
  §How vLLM recognizes a reusable prefix (parent hash + block tokens + extra
  keys; full blocks only; append-only tables; the last token of a fully
  cached prompt is recomputed; the salt enters the first block's identity).
* the paged-attention post on zhangchitc.github.io -- §What a physical
  block looks like (KVCacheBlock: block_id, ref_cnt, block hash, free-list
  links), §Two lookup structures (BlockHashToBlockMap, req_to_blocks),
  §Walking through two requests .. §Picking freed blocks back up (the worked
  example the tests replay).
* "Optimizing KV Cache Memory Management in vLLM with PagedAttention and
  Dynamic Block Allocation" -- §The Block Manager and Dynamic Allocation
  Lifecycle (prefill takes ceil(P/B) blocks; decode writes into the last
  block while S mod B != 0 and allocates at a boundary), §Copy-on-Write
  (a write into a block with ref_count > 1 allocates a new block, copies the
  shared one on the device, drops the old reference and remaps).
"""
from __future__ import annotations

import hashlib
import math
from typing import Dict, Hashable, Iterable, List, Optional, Sequence, Tuple

import numpy as np

ROOT_HASH = bytes(32)


class NoFreeBlocks(MemoryError):
    """The pool has too few free blocks; the caller must preempt."""


class KVCacheBlock:
    """Metadata of one physical block (the device memory lives elsewhere)."""

    __slots__ = ("block_id", "ref_cnt", "block_hash", "prev_free", "next_free")

    def __init__(self, block_id: int):
        self.block_id = block_id
        self.ref_cnt = 0
        self.block_hash: Optional[bytes] = None
        self.prev_free: Optional["KVCacheBlock"] = None
        self.next_free: Optional["KVCacheBlock"] = None

    def __repr__(self) -> str:
        h = self.block_hash.hex()[:8] if self.block_hash else "-"
        return f"KVCacheBlock(id={self.block_id}, ref={self.ref_cnt}, hash={h})"


class FreeBlockQueue:
    """Doubly linked list of free blocks: O(1) pop from the head, append at
    the tail, push at the head and removal from the middle (a cache hit on a
    free block)."""

    def __init__(self, blocks: Iterable[KVCacheBlock] = ()):
        self._head = KVCacheBlock(-1)
        self._tail = KVCacheBlock(-2)
        self._head.next_free = self._tail
        self._tail.prev_free = self._head
        self._n = 0
        for b in blocks:
            self.append(b)

    def __len__(self) -> int:
        return self._n

    def _link(self, b: KVCacheBlock, before: KVCacheBlock) -> None:
        prev = before.prev_free
        prev.next_free = b
        b.prev_free = prev
        b.next_free = before
        before.prev_free = b
        self._n += 1

    def append(self, b: KVCacheBlock) -> None:
        self._link(b, self._tail)

    def appendleft(self, b: KVCacheBlock) -> None:
        self._link(b, self._head.next_free)

    def remove(self, b: KVCacheBlock) -> None:
        if b.prev_free is None or b.next_free is None:
            raise ValueError(f"block {b.block_id} is not in the free queue")
        b.prev_free.next_free = b.next_free
        b.next_free.prev_free = b.prev_free
        b.prev_free = b.next_free = None
        self._n -= 1

    def popleft(self) -> KVCacheBlock:
        if self._n == 0:
            raise NoFreeBlocks("no free block")
        b = self._head.next_free
        self.remove(b)
        return b

    def __contains__(self, b: KVCacheBlock) -> bool:
        return b.prev_free is not None

    def ids(self) -> List[int]:
        out, b = [], self._head.next_free
        while b is not self._tail:
            out.append(b.block_id)
            b = b.next_free
        return out


def hash_block(parent: Optional[bytes], tokens: Sequence[int], extra: bytes = b"",
               salt: Optional[bytes] = None) -> bytes:
    """SHA-256 of (parent hash, salt, extra keys, token ids), each field
    length-prefixed.  The parent makes one hash name the whole prefix; the
    salt is passed for the first block only; `extra` stands for the other
    inputs that change K/V (an adapter id, image ids)."""
    h = hashlib.sha256()
    for field in (parent or ROOT_HASH, salt or b"", extra,
                  np.asarray(list(tokens), dtype="<i4").tobytes()):
        h.update(len(field).to_bytes(8, "little"))
        h.update(field)
    return h.digest()


class _Request:
    __slots__ = ("blocks", "tokens", "hashes", "salt", "extra", "released")

    def __init__(self, tokens, salt, extra):
        self.blocks: List[Optional[KVCacheBlock]] = []
        self.tokens: List[int] = list(tokens)
        self.hashes: List[bytes] = []
        self.salt = salt
        self.extra = extra
        self.released = 0  # leading blocks returned because a window no longer needs them


class BlockPool:
    """The block pool of one KV-cache group."""

    def __init__(self, num_blocks: int, block_size: int = 16, initial_order: Optional[Sequence[int]] = None):
        if num_blocks < 1 or block_size < 1:
            raise ValueError("num_blocks and block_size must be >= 1")
        self.block_size = block_size
        self.blocks = [KVCacheBlock(i) for i in range(num_blocks)]
        order = list(range(num_blocks)) if initial_order is None else [int(i) for i in initial_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("initial_order must be a permutation of the block ids")
        self.free_queue = FreeBlockQueue(self.blocks[i] for i in order)
        self.cached: Dict[bytes, Dict[int, KVCacheBlock]] = {}   # BlockHashToBlockMap
        self.requests: Dict[Hashable, _Request] = {}             # req_to_blocks and tokens
        self.pending_copies: List[Tuple[int, int]] = []           # copy-on-write (src, dst)
        self.queries = self.hits = self.evictions = self.preemptions = 0

    # -- hashes and lookup ------------------------------------------------

    def block_hashes(self, tokens: Sequence[int], salt: Optional[bytes] = None, extra: bytes = b"") -> List[bytes]:
        """Chained hashes of the full blocks of `tokens`."""
        B = self.block_size
        out: List[bytes] = []
        parent = None
        for i in range(len(tokens) // B):
            parent = hash_block(parent, tokens[i * B:(i + 1) * B], extra, salt if i == 0 else None)
            out.append(parent)
        return out

    def lookup_prefix(self, hashes: Sequence[bytes], num_tokens: int) -> List[KVCacheBlock]:
        """Cached blocks for the leading hashes, up to the first miss, and at
        most (num_tokens - 1) // B blocks: the last prompt token is always
        computed, since its logits are needed."""
        cap = max(0, (num_tokens - 1) // self.block_size)
        hits: List[KVCacheBlock] = []
        for h in hashes[:cap]:
            self.queries += 1
            owners = self.cached.get(h)
            if not owners:
                break
            self.hits += 1
            hits.append(next(iter(owners.values())))
        return hits

    # -- block state transitions --------------------------------------------

    def touch(self, blocks: Iterable[KVCacheBlock]) -> None:
        """Adopt cached blocks: a free one leaves the queue before its count rises."""
        for b in blocks:
            if b.ref_cnt == 0:
                self.free_queue.remove(b)
            b.ref_cnt += 1

    def allocate(self, n: int) -> List[KVCacheBlock]:
        """n blocks from the head of the free queue; a block still carrying a
        hash loses it (and its map entry) only now."""
        if n > len(self.free_queue):
            raise NoFreeBlocks(f"need {n} blocks, {len(self.free_queue)} free")
        out = []
        for _ in range(n):
            b = self.free_queue.popleft()
            if b.block_hash is not None:
                owners = self.cached.get(b.block_hash)
                if owners is not None:
                    owners.pop(b.block_id, None)
                    if not owners:
                        del self.cached[b.block_hash]
                b.block_hash = None
                self.evictions += 1
            b.ref_cnt = 1
            out.append(b)
        return out

    def _cache(self, b: KVCacheBlock, h: bytes) -> None:
        b.block_hash = h
        self.cached.setdefault(h, {})[b.block_id] = b

    def _release(self, blocks: Sequence[KVCacheBlock]) -> None:
        """Drop one reference per block, visiting them in reverse logical
        order; blocks that reach zero return to the free queue -- those that
        never became cache entries at its head (reclaimed first), cached ones
        at its tail (the tail of the request before its prefix)."""
        plain, cached = [], []
        for b in reversed(blocks):
            if b is None:
                continue
            b.ref_cnt -= 1
            if b.ref_cnt < 0:
                raise RuntimeError(f"block {b.block_id} released more often than taken")
            if b.ref_cnt == 0:
                (cached if b.block_hash is not None else plain).append(b)
        for b in reversed(plain):
            self.free_queue.appendleft(b)
        for b in cached:
            self.free_queue.append(b)

    # -- requests -------------------------------------------------------------

    def add_request(self, req: Hashable, tokens: Sequence[int], salt: Optional[bytes] = None,
                    extra: bytes = b"") -> int:
        """Admit a prompt: reuse its cached prefix, allocate ceil(P/B) blocks
        in total, and give every full block its hash.  Returns the number of
        prompt tokens whose K/V are already in the pool."""
        if req in self.requests:
            raise ValueError(f"request {req!r} already present")
        B = self.block_size
        hashes = self.block_hashes(tokens, salt, extra)
        hits = self.lookup_prefix(hashes, len(tokens))
        need = math.ceil(len(tokens) / B) - len(hits)
        free_after_touch = len(self.free_queue) - sum(1 for b in hits if b.ref_cnt == 0)
        if need > free_after_touch:
            raise NoFreeBlocks(f"request needs {need} new blocks, {free_after_touch} free")
        self.touch(hits)
        new = self.allocate(need)
        r = _Request(tokens, salt, extra)
        r.blocks = list(hits) + new
        r.hashes = hashes
        for i in range(len(hits), len(hashes)):
            self._cache(r.blocks[i], hashes[i])
        self.requests[req] = r
        return len(hits) * B

    def append_token(self, req: Hashable, token: int) -> int:
        """Decode one token: returns the slot its K/V go to.  At a block
        boundary (S mod B == 0) a new block is allocated; a write into a block
        other requests share (ref_cnt > 1) first copies it (the (src, dst)
        pair is queued in pending_copies for the device).  A block that
        becomes full gets its hash."""
        r = self.requests[req]
        B = self.block_size
        pos = len(r.tokens)
        lb = pos // B
        if lb == len(r.blocks):
            r.blocks.extend(self.allocate(1))
        else:
            b = r.blocks[lb]
            if b is None:
                raise RuntimeError("write into a released block")
            if b.ref_cnt > 1:
                (nb,) = self.allocate(1)
                b.ref_cnt -= 1
                r.blocks[lb] = nb
                self.pending_copies.append((b.block_id, nb.block_id))
        r.tokens.append(int(token))
        slot = r.blocks[lb].block_id * B + pos % B
        if (pos + 1) % B == 0 and len(r.hashes) == lb:
            parent = r.hashes[-1] if lb > 0 else None
            h = hash_block(parent, r.tokens[lb * B:(lb + 1) * B], r.extra, r.salt if lb == 0 else None)
            r.hashes.append(h)
            self._cache(r.blocks[lb], h)
        return slot

    def fork(self, parent: Hashable, child: Hashable) -> None:
        """The child shares every block of the parent (parallel sampling)."""
        if child in self.requests:
            raise ValueError(f"request {child!r} already present")
        p = self.requests[parent]
        c = _Request(p.tokens, p.salt, p.extra)
        c.blocks = list(p.blocks)
        c.hashes = list(p.hashes)
        c.released = p.released
        self.touch(b for b in c.blocks if b is not None)
        self.requests[child] = c

    def free_request(self, req: Hashable, preempted: bool = False) -> None:
        """Return all blocks of a finished (or preempted) request."""
        r = self.requests.pop(req)
        self._release(r.blocks)
        if preempted:
            self.preemptions += 1

    def release_outside_window(self, req: Hashable, window: int) -> int:
        """Give back the blocks lying wholly before the last `window`
        positions; returns how many were released."""
        r = self.requests[req]
        first_block = max(0, len(r.tokens) - window) // self.block_size
        drop = [b for b in r.blocks[r.released:first_block] if b is not None]
        for i in range(r.released, first_block):
            r.blocks[i] = None
        r.released = max(r.released, first_block)
        self._release(drop)
        return len(drop)

    # -- views for the GPU library --------------------------------------------

    def num_tokens(self, req: Hashable) -> int:
        return len(self.requests[req].tokens)

    def block_table(self, req: Hashable, window: int = 0) -> List[int]:
        """Physical ids in logical order (the row the kernel walks).  With a
        window: only the blocks covering the last `window` positions."""
        r = self.requests[req]
        first = 0
        if window > 0:
            first = max(0, len(r.tokens) - window) // self.block_size
        row = r.blocks[first:]
        if any(b is None for b in row):
            raise RuntimeError("table row includes a released block")
        return [b.block_id for b in row]

    def slot_of(self, req: Hashable, pos: int) -> int:
        r = self.requests[req]
        b = r.blocks[pos // self.block_size]
        if b is None:
            raise RuntimeError("position lies in a released block")
        return b.block_id * self.block_size + pos % self.block_size

    def tables(self, reqs: Sequence[Hashable], window: int = 0, width: Optional[int] = None,
               filler: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """(block_tables int32 [S, width], seq_lens int32 [S]) for a batch."""
        rows = [self.block_table(r, window) for r in reqs]
        w = max([len(x) for x in rows] + [1]) if width is None else width
        bt = np.full((len(reqs), w), filler, dtype=np.int32)
        for i, row in enumerate(rows):
            if len(row) > w:
                raise ValueError("table width too small")
            bt[i, :len(row)] = row
        lens = np.array([self.num_tokens(r) for r in reqs], dtype=np.int32)
        return bt, lens

    def check_writes(self, slots: Sequence[int]) -> None:
        """Host validator of one cache_write batch: slots in range, no slot
        twice, and no write into a block other requests share."""
        B = self.block_size
        seen = set()
        for s in slots:
            s = int(s)
            if s < 0:
                continue
            if s >= len(self.blocks) * B:
                raise ValueError(f"slot {s} beyond the pool")
            if s in seen:
                raise ValueError(f"slot {s} written twice in one batch")
            seen.add(s)
            if self.blocks[s // B].ref_cnt > 1:
                raise ValueError(f"slot {s} lies in shared block {s // B}")

    def stats(self) -> dict:
        n = len(self.blocks)
        free = len(self.free_queue)
        return {
            "num_blocks": n,
            "free": free,
            "used": n - free,
            "usage": (n - free) / n,
            "cached_hashes": len(self.cached),
            "queries": self.queries,
            "hits": self.hits,
            "evictions": self.evictions,
            "preemptions": self.preemptions,
        }


def reservation_waste(used_tokens: int, reserved_tokens: int) -> float:
    """Fraction of a full-length reservation a request leaves unused."""
    return 1.0 - used_tokens / reserved_tokens


def paging_waste_slots(num_tokens: int, block_size: int = 16) -> int:
    """Slots left empty in a request's last block."""
    return (-num_tokens) % block_size


def rows_share_blocks(rows: Sequence[Sequence[int]], seq_lens: Sequence[int], prefix_blocks: int = 0,
                      block_size: int = 16, window: int = 0) -> bool:
    """Whether some physical block is listed by more than one row past the
    first `prefix_blocks` entries (the part of each row decode attention
    reads itself): sequences of one prompt keep listing the same blocks
    until copy-on-write gives them their own ([Optimizing] "Copy-on-Write
    (CoW) for Parallel Sampling and Prefix Caching"; the reference counts of
    the pool show the same).  paged_decode_attention's shared_blocks hint.
    Only the entries holding attended positions count (with a sliding
    window a row lists the blocks covering the last `window` positions)."""
    seen = set()
    for r, ctx in zip(rows, seq_lens):
        ctx = int(ctx)
        if ctx <= 0:
            continue
        first = max(0, ctx - window) if window > 0 else 0
        used = (ctx - 1) // block_size - first // block_size + 1
        for b in r[prefix_blocks:used]:
            b = int(b)
            if b in seen:
                return True
            seen.add(b)
    return False


def shared_prefix_blocks(rows: Sequence[Sequence[int]], seq_lens: Sequence[int], block_size: int = 16) -> int:
    """Leading table entries that name the same physical block in every row
    and are full, attended blocks in every sequence: the part of a batch's
    context that decode attention can read once for all of its sequences
    (paged_decode_attention's shared_prefix_blocks).  Requests that found a
    cached prefix share its blocks ([Pool] "Finding a prefix again"), and
    only full blocks are shared ([Memory] "How vLLM recognizes a reusable
    prefix")."""
    if len(rows) == 0:
        return 0
    n = min(min(len(r) for r in rows), min(int(c) // block_size for c in seq_lens))
    first = rows[0]
    k = 0
    while k < n and all(int(r[k]) == int(first[k]) for r in rows):
        k += 1
    return k
