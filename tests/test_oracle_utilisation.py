"""Pins for the memory accounting oracle (contiguous preallocation versus paged blocks).

* the pages' worked examples (tests/golden/preallocation_waste.json): 100 of 2048 -> 1948
  wasted (95%); 200 of 2048 -> 90%; 200 / 500 / 1000 of 2048 each -> 1848 / 1548 / 1048;
* the paged bound: at most one partly empty block per sequence, so waste < 16 tokens per
  sequence, for every length (brute force over 0..4096);
* closed forms: a sequence of n tokens alone fills ceil(n/16) blocks with n slots; sharing
  (the pages' A/B/C example through the allocator) counts a shared block once while logical
  tokens count it per sequence;
* the allocator's live accounting after random operations equals the accounting of its
  exported tables.
"""

import json
import os

import numpy as np
import pytest

from oracle import allocator as AL
from oracle import utilisation as U

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "preallocation_waste.json")


def test_pages_worked_examples():
    g = json.load(open(GOLDEN))
    for ex in g["examples"]:
        reserved, used, util = U.contiguous_usage(ex["lengths"], g["max_len"])
        assert reserved == g["max_len"] * len(ex["lengths"])
        assert used == sum(ex["lengths"])
        assert [g["max_len"] - n for n in ex["lengths"]] == ex["wasted"]
        if "waste_fraction_rounded" in ex:
            assert round(1 - util, 2) == ex["waste_fraction_rounded"]
        # the same requests in 16-token blocks
        tables, pos = [], 0
        for n in ex["lengths"]:
            c = -(-n // g["block_size"])
            tables.append(list(range(pos, pos + c)))
            pos += c
        p = U.paged_usage(tables, ex["lengths"], g["block_size"])
        assert p["slots_filled"] == sum(ex["lengths"])
        waste = p["blocks_in_use"] * g["block_size"] - p["slots_filled"]
        assert waste < g["paged_bound"]["max_waste_per_sequence_tokens"] * len(ex["lengths"])
    # [P3] §3.1's three requests: contiguous 1700 / 6144 = 27.7%, paged 1700 / 1728 = 98.4%
    _, _, util_c = U.contiguous_usage([200, 500, 1000], 2048)
    p = U.paged_usage([list(range(13)), list(range(13, 45)), list(range(45, 108))],
                      [200, 500, 1000], 16)
    assert abs(util_c - 1700 / 6144) < 1e-15 and p["blocks_in_use"] == 108
    assert abs(p["utilisation"] - 1700 / 1728) < 1e-15


def test_paged_waste_below_one_block_for_every_length():
    for n in range(0, 4097):
        p = U.paged_usage([list(range(-(-n // 16)))], [n], 16)
        assert p["blocks_in_use"] == -(-n // 16) and p["slots_filled"] == n
        assert 0 <= p["blocks_in_use"] * 16 - n <= 15


def test_shared_blocks_counted_once():
    """[P1] §二's A/B/C tables: A [1,2,3,4], B [1,2,3,5], C [1,2,6,7], 64 tokens each."""
    tables = [[1, 2, 3, 4], [1, 2, 3, 5], [1, 2, 6, 7]]
    p = U.paged_usage(tables, [64, 64, 64], 16)
    assert p["logical_tokens"] == 192
    assert p["blocks_in_use"] == 7 and p["slots_filled"] == 7 * 16
    # a shared block partly filled by one owner and fuller for another: the fuller counts
    # (a second sequence holding 10 tokens of block 0 needs no entry past its first block)
    p = U.paged_usage([[0, 1], [0, 2]], [20, 10], 16)
    assert p["blocks_in_use"] == 2 and p["slots_filled"] == 16 + 4
    assert p["logical_tokens"] == 30


def test_contiguous_refuses_overlong_request():
    with pytest.raises(AssertionError):
        U.contiguous_usage([2049], 2048)


@pytest.mark.parametrize("seed", [0, 1])
def test_allocator_usage_equals_table_accounting(seed):
    rng = np.random.default_rng(300 + seed)
    nb = 64
    a = AL.BlockAllocator(nb, 16, rng.permutation(nb))
    next_id = 0
    for _ in range(400):
        live = list(a.blocks)
        op = rng.integers(0, 6)
        try:
            if op == 0 or not live:
                a.add_seq(next_id)
                next_id += 1
            elif op <= 2:
                s = live[int(rng.integers(len(live)))]
                a.append([s], [int(rng.integers(0, 30))])
            elif op == 3:
                a.fork(live[int(rng.integers(len(live)))], next_id)
                next_id += 1
            else:
                a.free_seq(live[int(rng.integers(len(live)))])
        except AL.AllocError:
            pass
        seqs = list(a.blocks)
        u = a.usage()
        assert u["blocks_in_use"] == nb - a.num_free()
        mb = max([1] + [len(a.blocks[s]) for s in seqs])
        tables, lens = a.tables(seqs, mb)
        assert u == U.paged_usage(tables, lens, 16)
        assert u["logical_tokens"] == sum(lens)
