"""Host bookkeeping against the pages' worked examples (tests/golden/) and
their stated rules."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W
from paged_kv_cache_37_amd.blockpool import (BlockPool, FreeBlockQueue, KVCacheBlock, NoFreeBlocks,
                                             hash_block, paging_waste_slots, reservation_waste)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def letters(s):
    return [ord(c) - ord("A") for c in s]


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_walkthrough_two_requests_and_reuse():
    """The paged-attention post's walkthrough, times 0..4."""
    g = load("bookkeeping_walkthrough.json")
    pool = BlockPool(g["num_blocks"], block_size=g["block_size"])
    B = g["block_size"]
    evicted_hash = None
    for st in g["steps"]:
        if st["action"] == "add":
            if "expect_evicted_prefix" in st:
                evicted_hash = pool.block_hashes(letters(st["expect_evicted_prefix"]))[-1]
                assert evicted_hash in pool.cached  # still cached before the request arrives
            cached = pool.add_request(st["req"], letters(st["prompt"]))
            assert cached == st["expect_cached_tokens"]
            assert pool.block_table(st["req"]) == st["expect_table"]
        else:
            pool.free_request(st["req"])
        for bid, ref in st["expect_refs"].items():
            assert pool.blocks[int(bid)].ref_cnt == ref, (st["time"], bid)
        for bid in st.get("expect_hashed", []):
            assert pool.blocks[bid].block_hash is not None
        for bid in st.get("expect_unhashed", []):
            assert pool.blocks[bid].block_hash is None
        if "expect_map_size" in st:
            assert len(pool.cached) == st["expect_map_size"]
        if "expect_free" in st:
            assert pool.free_queue.ids() == st["expect_free"]
        if "expect_free_set" in st:
            assert sorted(pool.free_queue.ids()) == st["expect_free_set"]
        if "expect_evicted_prefix" in st:
            assert evicted_hash not in pool.cached  # evicted only when block 2 was handed out again
            for bid, prefix in st["expect_new_prefixes"].items():
                assert pool.blocks[int(bid)].block_hash == pool.block_hashes(letters(prefix))[-1]
    # the blocks handed out at time 4 are {2, 3} under any queue order
    assert set(pool.block_table(2)[2:]) == {2, 3}
    assert len(pool.cached) == 4 and B == 4


def test_plain_append_order_would_differ():
    """Appending every freed block at the tail (hashless ones included)
    would hand out block 2 before 3 at time 4; the pages' table [0,1,3,2]
    needs hashless blocks reclaimed first."""
    pool = BlockPool(4, block_size=4)
    pool.add_request(0, letters("ABCDEFGHIJKL"))
    pool.add_request(1, letters("ABCDEFGHXYZ"))
    pool.free_request(0)
    pool.free_request(1)
    assert pool.free_queue.ids()[0] == 3  # the hashless tail block leads


def test_prefix_granularity_25_tokens():
    """Every request starts with the same 25 tokens: 16 from the cache, 9 computed."""
    pool = BlockPool(16)
    common = list(range(100, 125))
    pool.add_request("a", common + [1, 2, 3])
    cached = pool.add_request("b", common + [7, 8])
    assert cached == 16
    assert len(common) - cached == 9


def test_partial_overlap_block_size_4():
    """Block size 4 and 10 shared tokens: two reusable blocks, 8 tokens."""
    pool = BlockPool(16, block_size=4)
    shared = list(range(10))
    pool.add_request(0, shared + [50, 51, 52])
    assert pool.add_request(1, shared + [60, 61, 62, 63]) == 8


def test_perfect_hit_recomputes_last_block():
    """A fully cached prompt still recomputes its last token: at most
    16 * floor((P-1)/16) tokens come from the cache."""
    for P in (16, 17, 32, 40, 48):
        pool = BlockPool(32)
        tokens = list(range(P))
        pool.add_request("first", tokens)
        assert pool.add_request("again", tokens) == 16 * ((P - 1) // 16)


def test_append_only_duplicate_hash():
    """Prompt ABCDEF, generated GHI at block size 4; a resubmission reuses
    block 0 only, and two physical blocks later carry hash(..EFGH)."""
    pool = BlockPool(8, block_size=4)
    pool.add_request(0, letters("ABCDEF"))
    for t in letters("GHI"):
        pool.append_token(0, t)
    h_efgh = pool.block_hashes(letters("ABCDEFGH"))[-1]
    assert list(pool.cached[h_efgh]) == [pool.block_table(0)[1]]
    assert pool.add_request(1, letters("ABCDEF")) == 4
    assert pool.block_table(1)[0] == pool.block_table(0)[0]
    assert pool.block_table(1)[1] != pool.block_table(0)[1]
    for t in letters("GH"):
        pool.append_token(1, t)
    owners = pool.cached[h_efgh]
    assert sorted(owners) == sorted([pool.block_table(0)[1], pool.block_table(1)[1]])


def test_cache_salt_isolates_tenants():
    pool = BlockPool(16)
    prompt = list(range(40))
    pool.add_request("t1", prompt, salt=b"tenant-1-secret")
    assert pool.add_request("t2", prompt, salt=b"tenant-2-secret") == 0
    assert not set(pool.block_table("t1")) & set(pool.block_table("t2"))
    assert pool.add_request("t1b", prompt, salt=b"tenant-1-secret") == 32


def test_extra_keys_change_identity():
    pool = BlockPool(16)
    prompt = list(range(32))
    pool.add_request("lora-a", prompt + [1], extra=b"adapter:a")
    assert pool.add_request("lora-b", prompt + [1], extra=b"adapter:b") == 0
    assert pool.add_request("lora-a2", prompt + [1], extra=b"adapter:a") == 32


def test_hash_chain_names_whole_prefix():
    a = hash_block(None, [1] * 16)
    b = hash_block(None, [2] * 16)
    assert hash_block(a, [5] * 16) != hash_block(b, [5] * 16)
    assert hash_block(a, [5] * 16) == hash_block(hash_block(None, [1] * 16), [5] * 16)
    assert len(a) == 32


def test_decode_boundary_allocates_at_16_to_17():
    pool = BlockPool(8)
    pool.add_request(0, list(range(15)))
    assert len(pool.block_table(0)) == 1
    pool.append_token(0, 99)              # 16th token: same block
    assert len(pool.block_table(0)) == 1
    slot = pool.append_token(0, 100)      # 17th token: new block
    assert len(pool.block_table(0)) == 2
    assert slot == pool.block_table(0)[1] * 16 + 0


def test_index_math():
    pool = BlockPool(8, initial_order=[5, 0, 1, 2, 3, 4, 6, 7], block_size=4)
    pool.add_request(0, letters("ABCDEFGH"))
    assert pool.block_table(0) == [5, 0]  # ABCD -> block 5, EFGH -> block 0 (paging figure)
    for i in range(8):
        assert pool.slot_of(0, i) == pool.block_table(0)[i // 4] * 4 + i % 4
    pool.add_request(1, letters("ABCDXYZW"))
    assert pool.block_table(1)[0] == 5  # both prompts share the ABCD block


def test_copy_on_write_simulation():
    g = load("bookkeeping_cow_sim.json")
    pool = BlockPool(g["num_blocks"], g["block_size"])
    pool.add_request(1, list(range(24)))
    assert pool.block_table(1) == g["after_register"]["table"]
    assert len(pool.free_queue) == g["after_register"]["free"]
    pool.fork(1, 2)
    for b, r in g["after_fork"]["refs"].items():
        assert pool.blocks[int(b)].ref_cnt == r
    assert len(pool.free_queue) == g["after_fork"]["free"]
    pool.append_token(1, 1000)
    s = g["after_decode_seq1"]
    assert pool.block_table(1) == s["seq1"] and pool.block_table(2) == s["seq2"]
    assert [list(c) for c in pool.pending_copies] == s["copies"]
    for b, r in s["refs"].items():
        assert pool.blocks[int(b)].ref_cnt == r
    pool.append_token(2, 2000)
    assert pool.block_table(2) == g["after_decode_seq2"]["seq2"]
    assert [list(c) for c in pool.pending_copies] == g["after_decode_seq2"]["copies"]
    while pool.num_tokens(1) < 31:
        pool.append_token(1, 3000)
    pool.append_token(1, 3001)  # position 31: still logical block 1
    e = g["end"]
    assert pool.block_table(1) == e["seq1"] and pool.block_table(2) == e["seq2"]
    for b, r in e["refs"].items():
        assert pool.blocks[int(b)].ref_cnt == r
    assert len(pool.free_queue) == e["free"]


def test_exhaustion_raises_and_preemption_frees():
    pool = BlockPool(4)
    pool.add_request("old", list(range(40)))   # 3 blocks
    pool.add_request("new", list(range(100, 110)))  # 1 block
    with pytest.raises(NoFreeBlocks):
        pool.add_request("third", list(range(200, 217)))
    with pytest.raises(NoFreeBlocks):
        for t in range(7):
            pool.append_token("new", t)
    pool.free_request("new", preempted=True)   # newest request loses all its blocks
    assert pool.stats()["preemptions"] == 1
    assert len(pool.free_queue) == 1


def test_referenced_block_never_handed_out():
    """Under eviction pressure only ref-0 blocks leave the free queue."""
    pool = BlockPool(6)
    pool.add_request("keep", list(range(32)))
    pool.add_request("tmp", list(range(50, 82)))
    pool.free_request("tmp")
    keep = set(pool.block_table("keep"))
    pool.add_request("x", list(range(900, 964)))  # takes all 4 free blocks, evicting tmp's
    assert not keep & set(pool.block_table("x"))
    assert all(pool.blocks[b].ref_cnt == 1 for b in keep)


def test_touch_removes_free_block_before_reuse():
    pool = BlockPool(3)
    pool.add_request("a", list(range(16)) + [7])
    pool.free_request("a")
    hit_block = pool.block_table  # noqa: F841
    pool.add_request("b", list(range(16)) + [8])  # hits the freed, still-hashed first block
    first = pool.requests["b"].blocks[0]
    assert first not in pool.free_queue and first.ref_cnt == 1
    pool.add_request("c", list(range(500, 516)))  # needs one block: must not take b's
    assert pool.requests["c"].blocks[0] is not first


def test_waste_figures():
    """1500 tokens in a reserved 8192-token slot leave about 82 % unused;
    paging leaves fewer than 16 slots per request."""
    assert abs(reservation_waste(1500, 8192) - 0.8169) < 1e-3
    for n in range(1, 200):
        assert 0 <= paging_waste_slots(n) <= 15


def test_sliding_window_release_and_rows():
    pool = BlockPool(64)
    pool.add_request(0, list(range(100)))
    W_ = 40
    released = pool.release_outside_window(0, W_)
    assert released == (100 - W_) // 16  # blocks 0..2 lie wholly before position 60
    row = pool.block_table(0, window=W_)
    assert len(row) == oracle.row_span(100, W_, 16)[2]
    for t in range(5):
        pool.append_token(0, t)
        pool.release_outside_window(0, W_)
        assert len(pool.block_table(0, window=W_)) == oracle.row_span(pool.num_tokens(0), W_, 16)[2]


def test_free_queue_operations():
    blocks = [KVCacheBlock(i) for i in range(5)]
    q = FreeBlockQueue(blocks)
    assert q.ids() == [0, 1, 2, 3, 4]
    q.remove(blocks[2])
    assert q.ids() == [0, 1, 3, 4] and len(q) == 4
    q.appendleft(blocks[2])
    assert q.popleft() is blocks[2]
    q.append(blocks[2])
    assert q.ids() == [0, 1, 3, 4, 2]
    with pytest.raises(ValueError):
        q.remove(KVCacheBlock(9))


def test_write_validator():
    pool = BlockPool(8)
    pool.add_request(0, list(range(20)))
    pool.fork(0, 1)
    s_private = pool.slot_of(0, 19)
    with pytest.raises(ValueError):
        pool.check_writes([s_private])           # block shared after the fork
    pool.append_token(0, 5)                      # copy-on-write gives request 0 its own block
    pool.check_writes([pool.slot_of(0, 20)])
    with pytest.raises(ValueError):
        pool.check_writes([3, 3])
    with pytest.raises(ValueError):
        pool.check_writes([8 * 16])


def test_generator_slots_match_bookkeeping():
    """The tiny fp32 workload's tables and next-token slots equal what the
    block pool produces when its free queue starts in the same order."""
    w = W.make(1)
    perm = np.random.default_rng(1).permutation(32)
    pool = BlockPool(32, initial_order=perm)
    for s, ctx in enumerate(w.seq_lens):
        pool.add_request(s, list(range(1000 * s, 1000 * s + int(ctx))))
    for s in range(w.num_seqs):
        assert pool.block_table(s) == list(w.block_tables[s, : w.row_blocks[s]])
    slots = [pool.append_token(s, 1) for s in range(w.num_seqs)]
    assert slots == list(w.slot_mapping)
    for s in range(w.num_seqs):
        assert pool.block_table(s) == list(w.block_tables_after[s, : w.row_blocks_after[s]])
    bt, lens = pool.tables(range(w.num_seqs))
    oracle.check_tables(bt, lens, 0, 16, 32)


def test_shared_prefix_blocks_of_a_batch():
    """Common leading blocks of a batch: equal ids in every row, full and
    attended in every sequence."""
    from paged_kv_cache_37_amd.blockpool import shared_prefix_blocks

    assert shared_prefix_blocks([], []) == 0
    rows = [[7, 3, 9, 1], [7, 3, 9, 4], [7, 3, 2]]
    assert shared_prefix_blocks(rows, [60, 64, 40]) == 2     # row 2 differs at entry 2
    assert shared_prefix_blocks(rows[:2], [60, 64]) == 3     # entry 3 differs
    assert shared_prefix_blocks(rows[:2], [47, 64]) == 2     # block 2 of sequence 0 is not full
    assert shared_prefix_blocks([[5, 6]], [32]) == 2         # one sequence: its full blocks
    # the bookkeeping's own prefix hits: two requests with a 40-token common
    # prompt share its two full blocks, not the partial third
    pool = BlockPool(16)
    prompt = list(range(40))
    pool.add_request("a", prompt)
    pool.add_request("b", prompt[:40] + [99, 98])
    rows = [pool.block_table("a"), pool.block_table("b")]
    assert shared_prefix_blocks(rows, [40, 42]) == 2


def test_rows_share_blocks_of_a_batch():
    """The shared_blocks hint: a block listed by two rows past the prefix,
    counting only the entries that hold attended positions."""
    from paged_kv_cache_37_amd.blockpool import rows_share_blocks

    assert not rows_share_blocks([], [])
    assert not rows_share_blocks([[1, 2], [3, 4]], [32, 20])
    assert rows_share_blocks([[1, 2], [3, 2]], [32, 20])           # block 2 in both rows
    assert not rows_share_blocks([[1, 2], [1, 4]], [32, 20], prefix_blocks=1)
    assert rows_share_blocks([[1, 2], [1, 4]], [32, 20])
    assert not rows_share_blocks([[1, 9], [3, 9]], [16, 10])       # entry 1 holds no attended position
    assert not rows_share_blocks([[1, 2], [1, 2]], [0, 0])         # empty sequences read nothing
    # a window of 16 at context 40 attends positions 24..39: blocks 1 and 2
    # of the row (the row lists them from entry 0)
    assert rows_share_blocks([[5, 6], [7, 6]], [40, 40], window=16)
    # at context 17 the same window attends positions 1..16: entries 0 and 1
    assert rows_share_blocks([[5, 6], [7, 6]], [40, 17], window=16)
    # at context 16 it attends 0..15: entry 0 only, so block 6 is not read
    assert not rows_share_blocks([[5, 6], [7, 6]], [40, 16], window=16)
    # parallel sampling: a forked request lists the parent's blocks until a
    # write into a shared block copies it
    pool = BlockPool(16)
    pool.add_request("p", list(range(40)))
    pool.fork("p", "c")
    rows = [pool.block_table("p"), pool.block_table("c")]
    assert rows_share_blocks(rows, [40, 40])
    assert not rows_share_blocks(rows, [40, 40], prefix_blocks=3)
    pool.append_token("p", 7)
    pool.append_token("c", 8)  # both wrote into the shared partial block: copied
    rows = [pool.block_table("p"), pool.block_table("c")]
    assert rows_share_blocks(rows, [41, 41])                       # the two full blocks still shared
    assert not rows_share_blocks(rows, [41, 41], prefix_blocks=2)  # the tails are private now
