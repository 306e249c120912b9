"""Pins for the allocator oracle.

* the pages' printed examples (tests/golden): the block table 0->5, 1->12, 2->3 and the three
  tables sharing blocks 1, 2 (all three) and 3 (A and B);
* invariants from [P1] §二/§三: a sequence of n tokens holds ceil(n/16) blocks (waste below one
  block), appending takes a block iff the length is a multiple of 16, freed blocks return to
  the pool, every block is either free or referenced, and after all sequences are freed the
  whole pool is free again;
* isolation under sharing: tracked token contents per sequence stay intact through forks,
  copy-on-write and frees (a token one sequence writes is never seen by another);
* all-or-nothing failure when the pool is exhausted, and the error codes.
"""

import json
import os

import numpy as np
import pytest

from oracle.allocator import AllocError, BlockAllocator

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BS = 16


def test_p1_block_table_example():
    g = json.load(open(os.path.join(GOLDEN, "p1_block_table.json")))
    rest = [b for b in range(16) if b not in g["free_order_head"]]
    a = BlockAllocator(16, g["block_size"], g["free_order_head"] + rest)
    a.add_seq("A")
    slots, cows = a.append(["A"], [g["context_len"]])
    rows, lens = a.tables(["A"], 4)
    assert rows[0][:3] == g["logical_to_physical"] and rows[0][3] == -1
    assert lens == [37] and cows == []
    # token t lives in physical block table[t // 16] at offset t % 16
    assert slots[0] == 5 * 16 and slots[16] == 12 * 16 and slots[36] == 3 * 16 + 4


def test_p1_shared_blocks_example():
    g = json.load(open(os.path.join(GOLDEN, "p1_shared_blocks.json")))
    r = g["replay"]
    a = BlockAllocator(r["num_blocks"], g["block_size"], r["free_order"])
    for op in r["ops"]:
        if op[0] == "add":
            a.add_seq(op[1])
        elif op[0] == "append":
            a.append([op[1]], [op[2]])
        elif op[0] == "fork":
            a.fork(op[1], op[2])
    rows, _ = a.tables(["A", "B", "C"], 4)
    assert rows == [g["tables"]["A"], g["tables"]["B"], g["tables"]["C"]]
    for b, c in g["refcounts"].items():
        assert a.refcount(int(b)) == c
    a.free_seq("A")
    after = r["after_free_A"]
    assert a.free_list()[-len(after["free_list_tail"]):] == after["free_list_tail"]
    for b, c in after["refcounts"].items():
        assert a.refcount(int(b)) == c


def _check_invariants(a):
    ref = [0] * a.num_blocks
    for s, blocks in a.blocks.items():
        n = a.length[s]
        assert len(blocks) == -(-n // BS)  # ceil(n/16) blocks: waste < one block
        assert len(blocks) * BS - n < BS
        for b in blocks:
            ref[b] += 1
    assert ref == a.ref
    free = a.free_list()
    assert len(set(free)) == len(free)
    assert all(a.ref[b] == 0 for b in free)
    assert len(free) + sum(1 for c in a.ref if c > 0) == a.num_blocks


def test_random_lifecycle_invariants_and_isolation():
    rng = np.random.default_rng(31)
    nb = 64
    a = BlockAllocator(nb, BS, rng.permutation(nb))
    content = {}  # slot -> token id currently stored there
    logical = {}  # seq -> list of token ids it wrote or inherited
    next_tok = [0]
    next_seq = [0]

    def new_id():
        next_tok[0] += 1
        return next_tok[0]

    for step in range(3000):
        op = rng.integers(0, 10)
        live = list(a.blocks)
        if op <= 1 or not live:
            s = next_seq[0]
            next_seq[0] += 1
            a.add_seq(s)
            logical[s] = []
        elif op <= 6:
            batch = list(rng.choice(live, size=min(len(live), rng.integers(1, 4)), replace=False))
            ntok = [int(rng.integers(0, 20)) for _ in batch]
            before = {s: a.seq_len(s) for s in batch}
            free_before = a.num_free()
            state = (list(a.free), list(a.ref), {s: list(b) for s, b in a.blocks.items()})
            try:
                slots, cows = a.append(batch, ntok)
            except AllocError as e:
                assert e.code == "OUT_OF_BLOCKS"
                assert (list(a.free), list(a.ref), {s: list(b) for s, b in a.blocks.items()}) \
                    == state
                continue
            for src, dst in cows:  # the caller copies the tile before writing
                for off in range(BS):
                    if src * BS + off in content:
                        content[dst * BS + off] = content[src * BS + off]
            k = 0
            for s, t in zip(batch, ntok):
                for j in range(t):
                    n = before[s] + j
                    if n % BS == 0:
                        pass  # a fresh block: checked by the invariants below
                    tid = new_id()
                    content[slots[k]] = tid
                    logical[s].append(tid)
                    k += 1
            assert a.num_free() <= free_before
        elif op <= 7:
            parent = live[rng.integers(len(live))]
            child = next_seq[0]
            next_seq[0] += 1
            a.fork(parent, child)
            logical[child] = list(logical[parent])
        else:
            s = live[rng.integers(len(live))]
            a.free_seq(s)
            del logical[s]
        _check_invariants(a)
        # every sequence still reads exactly its own tokens through its table
        for s, blocks in a.blocks.items():
            got = [content.get(blocks[t // BS] * BS + t % BS) for t in range(a.length[s])]
            assert got == logical[s]
    for s in list(a.blocks):
        a.free_seq(s)
    assert a.num_free() == nb and all(c == 0 for c in a.ref)


def test_append_takes_block_iff_length_multiple_of_block():
    a = BlockAllocator(8, BS)
    a.add_seq(0)
    for n in range(100):
        if n == 8 * BS:
            break
        free = a.num_free()
        a.append([0], [1])
        assert (free - a.num_free()) == (1 if n % BS == 0 else 0)


def test_copy_on_write_pair_reported():
    a = BlockAllocator(8, BS, [3, 1, 4, 0, 5, 2, 6, 7])
    a.add_seq("p")
    a.append(["p"], [20])  # blocks [3, 1], last block holds 4 tokens
    a.fork("p", "c")
    assert a.refcount(1) == 2
    slots, cows = a.append(["c"], [1])
    assert cows == [(1, 4)] and slots == [4 * BS + 4]
    assert a.tables(["p", "c"], 2)[0] == [[3, 1], [3, 4]]
    assert a.refcount(1) == 1 and a.refcount(4) == 1 and a.refcount(3) == 2
    # the parent now owns block 1 alone: no copy on its next append
    slots, cows = a.append(["p"], [1])
    assert cows == [] and slots == [1 * BS + 4]
    # a fork at a block boundary never copies
    a.add_seq("q")
    a.append(["q"], [16])
    a.fork("q", "r")
    _, cows = a.append(["r"], [3])
    assert cows == []


def test_out_of_blocks_is_atomic():
    a = BlockAllocator(4, BS)
    a.add_seq(0)
    a.add_seq(1)
    a.append([0], [40])  # 3 blocks
    state = (a.free_list(), list(a.ref), dict(a.length))
    with pytest.raises(AllocError) as e:
        a.append([1, 0], [1, 20])  # needs 1 + 1 > 1 free
    assert e.value.code == "OUT_OF_BLOCKS"
    assert (a.free_list(), list(a.ref), dict(a.length)) == state


def test_error_codes():
    a = BlockAllocator(4, BS)
    a.add_seq(1)
    with pytest.raises(AllocError) as e:
        a.add_seq(1)
    assert e.value.code == "SEQ_EXISTS"
    with pytest.raises(AllocError) as e:
        a.append([2], [1])
    assert e.value.code == "UNKNOWN_SEQ"
    with pytest.raises(AllocError) as e:
        a.free_seq(2)
    assert e.value.code == "UNKNOWN_SEQ"
    with pytest.raises(AllocError) as e:
        a.fork(1, 1)
    assert e.value.code == "SEQ_EXISTS"
    with pytest.raises(AllocError) as e:
        a.append([1, 1], [1, 1])
    assert e.value.code == "INVALID_ARG"
    with pytest.raises(AllocError) as e:
        BlockAllocator(4, BS, [0, 1, 1, 2])
    assert e.value.code == "INVALID_ARG"
    a.append([1], [33])
    with pytest.raises(AllocError) as e:
        a.tables([1], 2)
    assert e.value.code == "INVALID_ARG"


def _beams_on_a_partial_block(nb, free_after):
    """One sequence of 20 tokens (its second block holds 4) forked into 4 beams that share
    both blocks, in a pool with `free_after` blocks left free."""
    a = BlockAllocator(nb, BS)
    a.add_seq(0)
    a.append([0], [20])
    for c in (1, 2, 3):
        a.fork(0, c)
    filler = nb - 2 - free_after
    if filler:
        a.add_seq("fill")
        a.append(["fill"], [filler * BS])
    assert a.num_free() == free_after and a.refcount(a.blocks[0][1]) == 4
    return a


def test_sharers_of_a_partial_block_need_one_copy_fewer_than_they_are():
    # Copy-on-write moves an appender off a shared, partly filled block while others still
    # hold it; the last sharer to append finds it no longer shared and writes in place. Four
    # beams appending one token each therefore take exactly three blocks: a pool with three
    # free blocks holds the batch.
    a = _beams_on_a_partial_block(nb=8, free_after=3)
    shared = a.blocks[0][1]
    slots, cows = a.append([0, 1, 2, 3], [1, 1, 1, 1])
    assert [src for src, _ in cows] == [shared] * 3 and a.num_free() == 0
    assert a.blocks[3][1] == shared and a.refcount(shared) == 1
    assert slots[3] == shared * BS + 4  # the last sharer writes into the block itself
    assert len({s // BS for s in slots}) == 4


def test_sharers_of_a_partial_block_fail_atomically_one_block_short():
    a = _beams_on_a_partial_block(nb=7, free_after=2)
    state = (a.free_list(), list(a.ref), dict(a.length), {s: list(b) for s, b in a.blocks.items()})
    with pytest.raises(AllocError) as e:
        a.append([0, 1, 2, 3], [1, 1, 1, 1])
    assert e.value.code == "OUT_OF_BLOCKS"
    assert (a.free_list(), list(a.ref), dict(a.length),
            {s: list(b) for s, b in a.blocks.items()}) == state
