"""Pins for the oracle allocator's automatic prefix caching.

* the pages' examples (tests/golden/prefix_cache_examples.json): [P3] §4.2's second request
  finds its first 2000+ tokens (every full block of the system prompt and the first
  exchange, decoded tokens included) in the cache; [P1] §五's three requests with one system
  prompt share its full blocks (refcount 3, written once);
* content: a synthetic model whose K/V at position p depend on all of tokens 0..p; requests
  drawn from a few shared prefixes write only the tokens after their cached ones, and every
  live sequence's K/V read through its table equal the model's values for its own tokens,
  bit for bit. A block whose ids match but whose earlier tokens differ must not be shared
  (constructed explicitly);
* lifecycle: a freed indexed block stays in the free list and is revived by a hit
  (refcount 1, out of the free list); fresh allocations evict indexed free blocks in FIFO
  order; an out-of-blocks add changes nothing; refcounts always equal table occurrences.
"""

import hashlib
import json
import os

import numpy as np
import pytest

import workloads as W
from oracle import allocator as AL
from oracle import cache_write as CW
from oracle import layout as L

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "prefix_cache_examples.json")))
BS = 16


def ids(rng, n):
    return [int(x) for x in rng.integers(0, 32000, size=n)]


def check_refcounts(a):
    count = {}
    for s, bl in a.blocks.items():
        for b in bl:
            count[b] = count.get(b, 0) + 1
    for b in range(a.num_blocks):
        assert a.ref[b] == count.get(b, 0)
    assert sorted(list(a.free) + list(count)) == list(range(a.num_blocks))
    for b in a.free:
        assert a.ref[b] == 0


def test_p3_system_prompt_reuse():
    g = GOLDEN["system_prompt_reuse"]
    rng = np.random.default_rng(600)
    a = AL.BlockAllocator(400, BS, rng.permutation(400))
    system = ids(rng, g["system_prompt_tokens"])
    q1 = ids(rng, g["question_tokens"])
    _, cached = a.add_seq_tokens(1, system + q1)
    assert cached == 0
    answer = ids(rng, g["answer_tokens"])
    for t in answer:  # decoded one token per step, with its id
        a.append_tokens([1], [1], [t])
    a.free_seq(1)  # the first request finishes; its blocks stay indexed
    q2 = ids(rng, g["second_question_tokens"])
    slots, cached = a.add_seq_tokens(2, system + q1 + answer + q2)
    assert cached == g["second_request_cached_tokens"]
    assert cached >= g["system_prompt_tokens"]
    assert len(slots) == len(system + q1 + answer + q2)
    check_refcounts(a)


def test_p1_three_requests_share_the_system_prompt():
    g = GOLDEN["shared_system_prompt"]
    rng = np.random.default_rng(601)
    a = AL.BlockAllocator(64, BS, rng.permutation(64))
    system = ids(rng, 40)
    cached = []
    for r in range(g["requests"]):
        _, c = a.add_seq_tokens(r, system + ids(rng, 9 + r))
        cached.append(c)
    assert cached == [0, 32, 32]
    shared = a.blocks[0][:2]
    for r in range(g["requests"]):
        assert a.blocks[r][:2] == shared
    assert [a.refcount(b) for b in shared] == [3, 3]
    assert a.blocks[0][2] != a.blocks[1][2] != a.blocks[2][2]
    check_refcounts(a)


def model_kv(tokens, p, hkv, hd, dtype):
    """The synthetic model: K/V of position p, a function of tokens 0..p."""
    h = hashlib.sha256(np.asarray(tokens[:p + 1], np.int64).tobytes()).digest()
    rng = np.random.default_rng(int.from_bytes(h[:8], "little"))
    return (W.normal_values(rng, (hkv, hd), dtype), W.normal_values(rng, (hkv, hd), dtype))


def test_shared_blocks_hold_each_sequences_own_kv():
    dtype, hkv, hd, nb = "bf16", 2, 64, 96
    rng = np.random.default_rng(602)
    a = AL.BlockAllocator(nb, BS, rng.permutation(nb))
    kc = np.zeros(nb * hkv * hd * BS, np.uint16)
    vc = np.zeros(nb * hkv * hd * BS, np.uint16)
    prefixes = [ids(rng, 37), ids(rng, 50), ids(rng, 16)]
    # two prefixes whose second blocks hold the same ids but whose first blocks differ
    twin = ids(rng, 16)
    prefixes.append(ids(rng, 16) + twin)
    prefixes.append(ids(rng, 16) + twin)
    toks = {}
    next_id = 0
    hits = 0
    for step in range(60):
        live = list(a.blocks)
        if live and (rng.random() < 0.35 or len(live) > 6):
            s = live[int(rng.integers(len(live)))]
            a.free_seq(s)
            del toks[s]
        else:
            t = prefixes[int(rng.integers(len(prefixes)))] + ids(rng, int(rng.integers(0, 20)))
            try:
                slots, cached = a.add_seq_tokens(next_id, t)
            except AL.AllocError:
                continue
            hits += cached
            # write only what the cache does not hold
            new = range(cached, len(t))
            kv = [model_kv(t, p, hkv, hd, dtype) for p in new]
            if kv:
                kc, vc = CW.write_kv(np.stack([x[0] for x in kv]), np.stack([x[1] for x in kv]),
                                     kc, vc, np.int32(slots[cached:]), hkv=hkv, hd=hd, bs=BS,
                                     dtype=dtype)
            toks[next_id] = t
            next_id += 1
        # decode a token for one live sequence now and then, with its id
        live = list(a.blocks)
        if live and rng.random() < 0.5:
            s = live[int(rng.integers(len(live)))]
            tok = ids(rng, 1)
            try:
                slots, cows = a.append_tokens([s], [1], tok)
            except AL.AllocError:
                continue
            assert not cows
            toks[s] = toks[s] + tok
            k, v = model_kv(toks[s], len(toks[s]) - 1, hkv, hd, dtype)
            kc, vc = CW.write_kv(k[None], v[None], kc, vc, np.int32(slots), hkv=hkv, hd=hd,
                                 bs=BS, dtype=dtype)
        check_refcounts(a)
        kv_view, vv_view = L.token_slot_views(kc, vc, hkv, hd, BS, dtype)
        for s, t in toks.items():
            for p in range(len(t)):
                b = a.blocks[s][p // BS]
                k, v = model_kv(t, p, hkv, hd, dtype)
                assert np.array_equal(kv_view[b, p % BS].reshape(hkv, hd), k), (s, p)
                assert np.array_equal(vv_view[b, p % BS], v), (s, p)
    assert hits > 0


def test_revival_eviction_and_atomicity():
    rng = np.random.default_rng(603)
    nb = 8
    a = AL.BlockAllocator(nb, BS, list(range(nb)))
    p = ids(rng, 48)  # 3 full blocks
    _, c = a.add_seq_tokens(0, p)
    assert c == 0 and a.blocks[0] == [0, 1, 2] and a.cached_blocks() == 3
    a.free_seq(0)
    assert list(a.free) == [3, 4, 5, 6, 7, 0, 1, 2] and a.cached_blocks() == 3
    # a hit revives the free blocks: out of the free list, refcount 1
    _, c = a.add_seq_tokens(1, p[:32] + ids(rng, 5))
    assert c == 32 and a.blocks[1][:2] == [0, 1]
    assert list(a.free) == [4, 5, 6, 7, 2] and a.refcount(0) == 1 and a.blocks[1][2] == 3
    # fresh allocations pop the front; popping block 2 evicts its entry
    a.add_seq(2)
    a.append([2], [16 * 4])
    assert a.blocks[2] == [4, 5, 6, 7] and list(a.free) == [2]
    a.append([2], [1])
    assert a.blocks[2][-1] == 2 and a.cached_blocks() == 2 and a.num_free() == 0
    # p's first two blocks still hit (held by sequence 1), its third was evicted, and no block
    # is free for the rest: all-or-nothing
    before = (list(a.free), list(a.ref), dict(a.blocks))
    with pytest.raises(AL.AllocError):
        a.add_seq_tokens(4, p + ids(rng, 40))
    assert (list(a.free), list(a.ref), dict(a.blocks)) == before
    check_refcounts(a)
