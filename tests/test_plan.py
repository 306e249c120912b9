"""The shared-prefix planner (pkv_decode_plan, host code) against brute-force definitions.

For tables shaped like the pages' sharing cases (a common prefix, beam groups sharing tails,
partly filled shared blocks, unrelated sequences, padding rows):
* skip_s is the longest prefix of s's table that some other sequence's table repeats block
  for block (brute force over all pairs);
* the units that name s cover exactly its blocks [0, skip_s), each once, and every unit's
  members all hold the unit's blocks at the unit's indices;
* each sequence's piece list is exactly the cells of its units, in unit order;
* units hold at most 16 / G members; float32 and G > 16 give plans without runs;
* a corrupted plan is refused by pkv_decode_planned before any device work.
"""

import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_459_amd as m
from paged_kv_cache_459_amd import lib

HDR = 16


def parse(p, B):
    U, M, L, cells = int(p[4]), int(p[5]), int(p[6]), int(p[7])
    o = HDR
    skip = p[o:o + B]; o += B
    blocks = p[o:o + B]; o += B
    ptr = p[o:o + B + 1]; o += B + 1
    units = p[o:o + 6 * U].reshape(U, 6); o += 6 * U
    members = p[o:o + M]; o += M
    lst = p[o:o + L]; o += L
    assert o == len(p)
    return dict(H=int(p[2]), GS=int(p[3]), U=U, cells=cells, skip=skip, blocks=blocks, ptr=ptr,
                units=units, members=members, list=lst, chunk=int(p[8]))


def brute_skip(tables, lens, nb):
    B = len(lens)
    c = [-(-int(n) // 16) for n in lens]

    def ok(s, j):
        e = int(tables[s, j])
        return e >= 0 and (e & ~0x40000000) < nb

    out = []
    for s in range(B):
        best = 0
        for t in range(B):
            if t == s:
                continue
            j = 0
            while (j < c[s] and j < c[t] and ok(s, j) and ok(t, j) and
                   (tables[s, j] & ~0x40000000) == (tables[t, j] & ~0x40000000)):
                j += 1
            best = max(best, j)
        out.append(best)
    return np.array(out)


def case(rng, kind):
    nb = 400
    if kind == "prefix":  # a common prefix, private tails
        B, pre = 12, 7
        lens = 16 * pre + rng.integers(1, 60, size=B)
        tables = np.full((B, 16), -1, np.int32)
        free = iter(rng.permutation(np.arange(pre, nb)))
        for s in range(B):
            tables[s, :pre] = np.arange(pre)
            for j in range(pre, -(-int(lens[s]) // 16)):
                tables[s, j] = next(free)
    elif kind == "beam":  # prefix, group tails, own last blocks; some groups end mid-block
        groups, beams, pre = 4, 4, 5
        B = groups * beams
        tables = np.full((B, 16), -1, np.int32)
        lens = np.zeros(B, np.int64)
        free = iter(rng.permutation(np.arange(pre, nb)))
        for g in range(groups):
            tail = int(rng.integers(1, 5))
            tb = [next(free) for _ in range(tail)]
            n = 16 * (pre + tail) + int(rng.integers(1, 16))
            for b in range(beams):
                s = g * beams + b
                tables[s, :pre] = np.arange(pre)
                tables[s, pre:pre + tail] = tb
                tables[s, pre + tail] = next(free)
                lens[s] = n
    elif kind == "wide":  # many sharers: more than 8 member tiles per chunk (several groups)
        B, pre = 40, 11
        lens = 16 * pre + rng.integers(1, 40, size=B)
        tables = np.full((B, 16), -1, np.int32)
        free = iter(rng.permutation(np.arange(pre, nb)))
        for s in range(B):
            tables[s, :pre] = np.arange(pre)
            for j in range(pre, -(-int(lens[s]) // 16)):
                tables[s, j] = next(free)
    else:  # mixed: shared partial last blocks, unrelated rows, empty rows, bad entries
        B = 10
        tables = np.full((B, 8), -1, np.int32)
        lens = np.array([40, 35, 40, 0, 60, 60, 17, 17, 33, 50])
        tables[0, :3] = [1, 2, 3]
        tables[1, :3] = [1, 2, 3]          # ends inside block 3 (shared, partly filled)
        tables[2, :3] = [1, 2, 9]          # parts at index 2
        tables[4, :4] = [5, 6, 7, 8]
        tables[5, :4] = [5, 6, 7, 8]       # the whole sequence shared
        tables[6, :2] = [11, 12]
        tables[7, :2] = [11, 12 | 0x40000000]  # a marked entry: the same block
        tables[8, :3] = [13, nb + 5, 14]   # an entry outside the pool: never shared
        tables[9, :4] = [13, nb + 5, 14, 15]
    return tables, np.asarray(lens, np.int32), nb


@pytest.mark.parametrize("kind", ["prefix", "beam", "mixed", "wide"])
@pytest.mark.parametrize("hq,hkv,dt", [(8, 8, torch.float16), (28, 4, torch.bfloat16),
                                       (16, 8, torch.bfloat16), (32, 2, torch.bfloat16)])
def test_plan_matches_brute_force(kind, hq, hkv, dt):
    rng = np.random.default_rng(800 + hq)
    tables, lens, nb = case(rng, kind)
    B = len(lens)
    G = hq // hkv
    p = m.pkv_decode_plan(tables, lens, num_q_heads=hq, num_kv_heads=hkv, num_blocks=nb,
                          max_context_len=16 * tables.shape[1], dtype=dt,
                          max_group=16)
    P = parse(p, B)
    kernel = m.pkv_decode_kernel(hq, hkv, dt)
    assert (P["H"], P["GS"]) == ((hkv, G) if kernel == 2 else (hq, 1))
    if G > 16:
        assert P["U"] == 0 and not P["skip"].any()
        return
    np.testing.assert_array_equal(P["skip"], brute_skip(tables, lens, nb))
    np.testing.assert_array_equal(P["blocks"], [-(-int(n) // 16) for n in lens])
    cover = [[] for _ in range(B)]
    lists = [[] for _ in range(B)]
    cell = 0
    for u in P["units"]:
        ref, b0, b1, off, cnt, cbase = (int(x) for x in u)
        assert cbase == cell and 1 <= cnt <= max(1, 16 // G) and b0 < b1 <= b0 + P["chunk"]
        mem = P["members"][off:off + cnt]
        assert len(set(mem.tolist())) == cnt
        for k, s in enumerate(mem):
            np.testing.assert_array_equal(tables[s, b0:b1] & ~0x40000000,
                                          tables[ref, b0:b1] & ~0x40000000)
            cover[s].extend(range(b0, b1))
            lists[s].append(cbase + k * P["H"])
        cell += cnt * P["H"]
    assert cell == P["cells"]
    for s in range(B):
        assert sorted(cover[s]) == list(range(P["skip"][s])), s
        assert P["list"][P["ptr"][s]:P["ptr"][s + 1]].tolist() == lists[s]


def test_float32_plans_have_no_runs():
    rng = np.random.default_rng(3)
    tables, lens, nb = case(rng, "prefix")
    p = m.pkv_decode_plan(tables, lens, num_q_heads=4, num_kv_heads=4, num_blocks=nb,
                          max_context_len=256, dtype=torch.float32)
    P = parse(p, len(lens))
    assert P["U"] == 0 and not P["skip"].any() and P["cells"] == 0


def test_corrupted_plans_are_refused_on_the_host():
    rng = np.random.default_rng(4)
    tables, lens, nb = case(rng, "beam")
    B = len(lens)
    p = m.pkv_decode_plan(tables, lens, num_q_heads=8, num_kv_heads=8, num_blocks=nb,
                          max_context_len=256, dtype=torch.float16)
    buf = (ctypes.c_uint8 * (1 << 16))()
    fake = ctypes.c_void_p((ctypes.addressof(buf) + 255) & ~255)
    W = 64

    def call(plan, append=False):
        # workspace_bytes = 0: a plan that passes the checks stops at the workspace check
        # (PKV_ERR_WORKSPACE = 6), so nothing here ever reaches a launch
        q = np.ascontiguousarray(plan, np.int32)
        return lib.pkv_decode_planned(0, fake, fake, fake if append else None,
                                      fake if append else None, fake, fake, fake, fake, B, 8, 8,
                                      64, 16, nb, 16, 256, 0.1, 1, q.ctypes.data, fake, q.size,
                                      W, fake, 0, None)
    assert call(p) == 6 and call(p, append=True) == 6
    P = parse(p, B)
    o_units = HDR + 3 * B + 1
    bad = []
    for idx, val in [(0, 0), (1, B + 1), (2, 3), (4, P["U"] + 1), (7, -1),
                     (o_units, B), (o_units + 1, -1), (o_units + 2, 17), (o_units + 4, 0),
                     (o_units + 5, P["cells"]), (HDR, 99), (HDR + 2 * B + B, 0)]:
        c = p.copy()
        c[idx] = val
        bad.append(c)
    c = p.copy()
    c[-1] = P["cells"]  # a piece cell past the shared cells
    bad.append(c)
    bad.append(p[:-1])  # truncated
    for c in bad:
        assert call(c) == 1
    # append mode: a plan that shares a sequence's last block is refused
    c = p.copy()
    c[HDR] = c[HDR + B]  # skip_0 = blocks_0
    assert call(c, append=True) == 1


def test_planned_grid_limit():
    """A plan whose shared pass (one wave per unit and kv head) plus the stream workers would
    pass 2^31 - 1 work-items is refused (PKV_ERR_UNSUPPORTED) before any device work; one unit
    fewer passes every check and stops at the workspace (PKV_ERR_WORKSPACE)."""
    B, H, W = 2, 16384, 64  # G = 1: the vector kernel, head slots = q heads
    buf = (ctypes.c_uint8 * (1 << 16))()
    fake = ctypes.c_void_p((ctypes.addressof(buf) + 255) & ~255)

    def plan(U):
        hdr = [0x504C4E31, B, H, 1, U, 1, 0, H, 16] + [0] * (HDR - 9)
        skip, blocks, ptr = [1, 1], [1, 1], [0, 0, 0]
        units = [0, 0, 1, 0, 1, 0] * U  # every unit: sequence 0's block 0, cells 0..H-1
        return np.asarray(hdr + skip + blocks + ptr + units + [0], np.int32)

    def call(q):
        return lib.pkv_decode_planned(0, fake, fake, None, None, fake, fake, fake, fake, B, H,
                                      H, 64, 16, 4, 1, 16, 0.1, 1, q.ctypes.data, fake, q.size,
                                      W, fake, 0, None)
    limit = (2**31 - 1) // 64 - W - 32  # largest units * Hkv allowed
    ok = limit // H
    assert call(plan(ok)) == 6
    assert call(plan(ok + 1)) == 2


@pytest.mark.parametrize("hq,hkv,runs", [(8, 8, True), (16, 4, True), (28, 4, False),
                                         (32, 2, False)])
def test_default_group_threshold(hq, hkv, runs):
    """By default only G <= 4 gets runs (at least four sequences per 16-row tile)."""
    rng = np.random.default_rng(5)
    tables, lens, nb = case(rng, "prefix")
    p = m.pkv_decode_plan(tables, lens, num_q_heads=hq, num_kv_heads=hkv, num_blocks=nb,
                          max_context_len=256, dtype=torch.bfloat16)
    assert (parse(p, len(lens))["U"] > 0) == runs
    with pytest.raises(m.PkvError):
        m.pkv_decode_plan(tables, lens, num_q_heads=hq, num_kv_heads=hkv, num_blocks=nb,
                          max_context_len=256, dtype=torch.bfloat16, max_group=17)


def _shared_then_private(B, shared, private, nb=200):
    """B sequences holding the same `shared` blocks, then `private` blocks each (the last one
    partly filled)."""
    tables = np.full((B, shared + private), -1, np.int32)
    nxt = shared
    for s in range(B):
        tables[s, :shared] = np.arange(shared)
        tables[s, shared:] = np.arange(nxt, nxt + private)
        nxt += private
    lens = np.full(B, 16 * (shared + private) - 5, np.int64)
    assert nxt <= nb
    return tables, lens, nb


@pytest.mark.parametrize("B,shared,private,hq,hkv,kernel,W,want", [
    (4, 10, 1, 8, 8, 0, 1024, 1),   # the shared pass reads 10 tiles per head, the stream 4
    (4, 2, 5, 8, 8, 0, 1024, 2),    # 2 against 20: the stream pass dominates
    (4, 5, 5, 8, 8, 0, 1024, 2),    # 5 against 20
    (2, 10, 5, 8, 8, 0, 1024, 1),   # 10 against 10: ties take one launch
    (4, 0, 6, 8, 8, 0, 1024, 1),    # no runs: no shared pass, the stream pass alone
    (4, 10, 1, 8, 8, 0, 1028, 2),   # workers not a multiple of 8 work-groups: no one launch
    (4, 10, 1, 8, 4, 0, 1024, 2),   # G = 2: the matrix-core stream kernel has none
    (4, 10, 1, 8, 4, 1, 1024, 1),   # G = 2 on the vector kernel: 10 x 4 against 4 x 8
])
def test_planned_launches_rule(B, shared, private, hq, hkv, kernel, W, want):
    """The automatic choice of one or two launches for the shared and stream passes: one where
    the one-launch kernel exists and the shared pass reads at least as many (block, head)
    tiles as the stream pass (host only)."""
    tables, lens, nb = _shared_then_private(B, shared, private)
    prev = m.pkv_set_attn_kernel(kernel)
    try:
        p = m.pkv_decode_plan(tables, lens, num_q_heads=hq, num_kv_heads=hkv, num_blocks=nb,
                              max_context_len=16 * tables.shape[1], dtype=torch.bfloat16)
        assert (parse(p, B)["U"] > 0) == (shared > 0)
        got = m.pkv_decode_planned_launches(p, batch=B, num_q_heads=hq, num_kv_heads=hkv,
                                            max_blocks=tables.shape[1], dtype=torch.bfloat16,
                                            num_workers=W)
    finally:
        m.pkv_set_attn_kernel(prev)
    assert got == want


def test_planned_launches_refuses_bad_plans():
    tables, lens, nb = _shared_then_private(4, 10, 1)
    p = m.pkv_decode_plan(tables, lens, num_q_heads=8, num_kv_heads=8, num_blocks=nb,
                          max_context_len=16 * 11, dtype=torch.bfloat16)
    args = dict(batch=4, num_q_heads=8, num_kv_heads=8, max_blocks=11, dtype=torch.bfloat16,
                num_workers=1024)
    assert m.pkv_decode_planned_launches(p, **args) == 1
    assert m.pkv_decode_planned_launches(p, **dict(args, batch=5)) == 0  # plan for another B
    assert m.pkv_decode_planned_launches(p, **dict(args, num_workers=1022)) == 0
    assert m.pkv_decode_planned_launches(p, **dict(args, num_kv_heads=3)) == 0
    bad = p.copy()
    bad[0] ^= 1  # magic
    assert m.pkv_decode_planned_launches(bad, **args) == 0
    assert m.pkv_decode_planned_launches(p[:20], **args) == 0  # truncated
