"""Pins for the oracle's copy-on-write block copy, and for a beam-search loop driven through
the oracle's allocator, block copy and cache write.

* the copy, read back through the header's scalar index formulas (not the oracle's reshapes):
  every element of every kv head's tile of block dst equals block src's, in both caches, and
  no other element changes; pairs outside the pool are skipped; overlapping pairs refused;
* beam search ([P2] vLLM overview, "共享和复用" and the Beam Search item of "PagedAttention 的
  优势": candidates share the blocks of their common history): beams are forked at arbitrary
  (mostly not block-aligned) lengths, re-selected every step, and append one token each.
  Beside the paged cache the test keeps every beam's history as a dense array (a child's
  history is its parent's plus its own new token). After every step, every live beam's
  tokens read through its table equal its dense history bit for bit (so no write became
  visible to another beam and every copied block arrived whole), and at the end the
  attention oracle over the paged cache equals dense attention over the histories.
"""

import numpy as np
import pytest

import workloads as W
from oracle import allocator as AL
from oracle import attention as A
from oracle import cache_write as CW
from tests import helpers as H


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("hd", [64, 128])
def test_copy_blocks_scalar_formula(dtype, hd):
    rng = np.random.default_rng(41)
    nb, hkv, bs = 9, 3, 16
    size = nb * hkv * hd * bs
    kc = W.normal_values(rng, (size,), dtype)
    vc = W.normal_values(rng, (size,), dtype)
    pairs = [(2, 5), (2, 7), (0, 1), (3, nb), (-1, 4), (6, 8)]  # src 2 twice; two skipped
    kc2, vc2 = CW.copy_blocks(kc, vc, pairs, hkv=hkv, hd=hd, bs=bs, dtype=dtype)
    h = np.arange(hkv)[:, None, None]
    t = np.arange(bs)[None, :, None]
    d = np.arange(hd)[None, None, :]
    changed_k = np.zeros(size, bool)
    changed_v = np.zeros(size, bool)
    for s, dst in [(2, 5), (2, 7), (0, 1), (6, 8)]:
        kd = H.k_offsets(dst, h, t, d, hkv, hd, bs, dtype)
        vd = H.v_offsets(dst, h, t, d, hkv, hd, bs)
        np.testing.assert_array_equal(kc2[kd].view(np.uint8),
                                      kc[H.k_offsets(s, h, t, d, hkv, hd, bs, dtype)].view(np.uint8))
        np.testing.assert_array_equal(vc2[vd].view(np.uint8),
                                      vc[H.v_offsets(s, h, t, d, hkv, hd, bs)].view(np.uint8))
        changed_k[kd] = True
        changed_v[vd] = True
    assert changed_k.sum() == 4 * hkv * hd * bs
    np.testing.assert_array_equal(kc2[~changed_k].view(np.uint8), kc[~changed_k].view(np.uint8))
    np.testing.assert_array_equal(vc2[~changed_v].view(np.uint8), vc[~changed_v].view(np.uint8))
    # the inputs are not modified
    kc3, _ = CW.copy_blocks(kc, vc, [], hkv=hkv, hd=hd, bs=bs, dtype=dtype)
    np.testing.assert_array_equal(kc3.view(np.uint8), kc.view(np.uint8))


def test_copy_blocks_refuses_overlapping_pairs():
    kc = np.zeros(4 * 64 * 16, np.float32)
    with pytest.raises(AssertionError):
        CW.copy_blocks(kc, kc, [(0, 2), (1, 2)], hkv=1, hd=64, bs=16, dtype="f32")
    with pytest.raises(AssertionError):
        CW.copy_blocks(kc, kc, [(0, 1), (1, 2)], hkv=1, hd=64, bs=16, dtype="f32")


def read_history(kc, vc, row, n, hkv, hd, bs, dtype):
    """Tokens 0..n-1 of a sequence read through its table with the scalar formulas:
    storage arrays [n, Hkv, hd]."""
    K = np.empty((n, hkv, hd), kc.dtype)
    V = np.empty((n, hkv, hd), vc.dtype)
    h = np.arange(hkv)[:, None]
    d = np.arange(hd)[None, :]
    for tok in range(n):
        b = int(row[tok // bs])
        K[tok] = kc[H.k_offsets(b, h, tok % bs, d, hkv, hd, bs, dtype)]
        V[tok] = vc[H.v_offsets(b, h, tok % bs, d, hkv, hd, bs)]
    return K, V


def run_oracle_beam_loop(seed, dtype, *, groups=3, beams=3, hq=4, hkv=2, hd=64, steps=40,
                         prompt_lens=(21, 16, 7), nb=96, check_every_step=True):
    """Beam search through the oracle. Returns (final caches, tables, lengths, histories)."""
    bs = 16
    rng = np.random.default_rng(seed)
    alloc = AL.BlockAllocator(nb, bs, rng.permutation(nb))
    size = nb * hkv * hd * bs
    kc = np.full(size, H.NAN_BITS[dtype], H.STORAGE[dtype])
    vc = np.full(size, H.NAN_BITS[dtype], H.STORAGE[dtype])
    hist = {}
    next_id = 0
    live = []  # [groups][beams] sequence ids
    for g in range(groups):  # the prompt: one sequence per group, then its beams are forked
        root = next_id
        next_id += 1
        alloc.add_seq(root)
        n = prompt_lens[g]
        slots, cows = alloc.append([root], [n])
        assert not cows
        k = W.normal_values(rng, (n, hkv, hd), dtype)
        v = W.normal_values(rng, (n, hkv, hd), dtype)
        kc, vc = CW.write_kv(k, v, kc, vc, np.int32(slots), hkv=hkv, hd=hd, bs=bs, dtype=dtype)
        hist[root] = (k, v)
        row = []
        for _ in range(beams):
            alloc.fork(root, next_id)
            hist[next_id] = hist[root]
            row.append(next_id)
            next_id += 1
        alloc.free_seq(root)
        del hist[root]
        live.append(row)
    total_cows = 0
    for step in range(steps):
        if step > 0:  # re-select: each new beam forks from a parent of its group
            parents = W.beam_parents(rng, groups, beams)
            new_live = []
            for g in range(groups):
                row = []
                for p in parents[g]:
                    alloc.fork(live[g][p], next_id)
                    hist[next_id] = hist[live[g][p]]
                    row.append(next_id)
                    next_id += 1
                for s in live[g]:
                    alloc.free_seq(s)
                    del hist[s]
                new_live.append(row)
            live = new_live
        seqs = [s for row in live for s in row]
        slots, cows = alloc.append(seqs, [1] * len(seqs))
        total_cows += len(cows)
        kc, vc = CW.copy_blocks(kc, vc, cows, hkv=hkv, hd=hd, bs=bs, dtype=dtype)
        k_new = W.normal_values(rng, (len(seqs), hkv, hd), dtype)
        v_new = W.normal_values(rng, (len(seqs), hkv, hd), dtype)
        kc, vc = CW.write_kv(k_new, v_new, kc, vc, np.int32(slots), hkv=hkv, hd=hd, bs=bs,
                             dtype=dtype)
        for i, s in enumerate(seqs):
            k0, v0 = hist[s]
            hist[s] = (np.concatenate([k0, k_new[i:i + 1]]), np.concatenate([v0, v_new[i:i + 1]]))
        if check_every_step or step == steps - 1:
            tables, lens = alloc.tables(seqs, max(len(alloc.blocks[s]) for s in seqs))
            for s, row, n in zip(seqs, tables, lens):
                K, V = read_history(kc, vc, row, n, hkv, hd, bs, dtype)
                np.testing.assert_array_equal(K.view(np.uint8), hist[s][0].view(np.uint8))
                np.testing.assert_array_equal(V.view(np.uint8), hist[s][1].view(np.uint8))
    assert total_cows > 0  # the loop did exercise copy-on-write
    return kc, vc, np.int32(tables), np.int32(lens), [hist[s] for s in seqs], alloc


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_beam_loop_keeps_every_beams_history(dtype):
    hq, hkv, hd = 4, 2, 64
    kc, vc, tables, lens, hist, alloc = run_oracle_beam_loop(51, dtype, hq=hq, hkv=hkv, hd=hd)
    rng = np.random.default_rng(52)
    q = W.normal_values(rng, (len(lens), hq, hd), dtype)
    out = A.decode_attention(q, kc, vc, tables, lens, scale=0.125, hkv=hkv, hd=hd, bs=16,
                             dtype=dtype)
    for i, (K, V) in enumerate(hist):
        Kf, Vf = H.f64(K, dtype), H.f64(V, dtype)
        for h in range(hq):
            s = 0.125 * Kf[:, h // 2] @ H.f64(q[i, h], dtype)
            w = np.exp(s - s.max())
            np.testing.assert_allclose(out[i, h], w @ Vf[:, h // 2] / w.sum(), atol=1e-12)
    # every block in use is held by exactly the beams whose tables name it
    held = {}
    for row, n in zip(tables, lens):
        for b in row[:-(-int(n) // 16)]:
            held[int(b)] = held.get(int(b), 0) + 1
    for b, c in held.items():
        assert alloc.refcount(b) == c
    assert alloc.num_free() == alloc.num_blocks - len(held)
