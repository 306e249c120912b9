"""Cache write (scatter of new tokens' K/V into their slots) and the copy-on-write block
copy, both bitwise.

Test infrastructure only (see the package docstring).

[P1] §三 步驟二 and 步驟三: the K/V of each new token are written into the current block of
its sequence (a fresh block having been taken when the current one was full). The slot that
says where, ``slot = physical_block * bs + offset``, comes from the allocator; this function
only performs the write, for the T tokens of one call:

    for every i with 0 <= slot[i] < NB * bs:
        K cache (block slot[i] // bs, head h, token slot[i] % bs, :) = k[i, h, :]   (all h)
        V cache (same)                                                  = v[i, h, :]

Negative slots are padding and are skipped. Two tokens with one slot in one call have no
defined result, so the oracle refuses them. ``copy_blocks`` is documented where it is defined.
"""

import numpy as np

from .layout import token_slot_views


def write_kv(k, v, k_cache, v_cache, slot_mapping, *, hkv, hd, bs, dtype):
    """Return copies of (k_cache, v_cache) with the T tokens scattered into their slots.

    k, v: storage arrays [T, Hkv, hd]; caches: storage arrays in the documented layout.
    Copies bits: values (NaN payloads included) are moved, never converted.
    """
    k = np.asarray(k)
    v = np.asarray(v)
    slots = np.asarray(slot_mapping).astype(np.int64)
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    nb = kc.size // (hkv * hd * bs)
    live = slots[(slots >= 0) & (slots < nb * bs)]
    assert len(np.unique(live)) == len(live), "duplicate slots in one write"
    kv, vv = token_slot_views(kc, vc, hkv, hd, bs, dtype)
    x = kv.shape[-1]
    for i, s in enumerate(slots):
        if s < 0 or s >= nb * bs:
            continue
        b, off = int(s // bs), int(s % bs)
        kv[b, off] = k[i].reshape(hkv, hd // x, x)
        vv[b, off] = v[i]
    return kc, vc


def copy_blocks(k_cache, v_cache, pairs, *, hkv, hd, bs, dtype):
    """Return copies of (k_cache, v_cache) where block dst holds block src's bits, per pair.

    [P2] vLLM overview, "共享和复用" and the Beam Search item of "PagedAttention 的优势": beam
    candidates share the physical blocks of their common history. The pages do not say what
    happens when one of them appends into a shared, partly filled block; our reading is that
    the appender first gets a private copy (copy-on-write): the allocator gives it a fresh
    block dst in place of src and reports (src, dst), and this is the copy. A block is every
    kv head's tile of it, in both caches; the copy is bitwise and whole (slots past the
    filled ones included).

    pairs: sequence of (src, dst). Pairs naming a block outside [0, NB) are skipped. Every dst
    must be distinct and no dst may be a src of the same call (the allocator's pairs never
    are: a dst comes from the free list, a src still has owners), so the order of the copies
    does not matter; the oracle refuses anything else.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    per_block = hkv * hd * bs
    nb = kc.size // per_block
    live = [(int(s), int(d)) for s, d in pairs if 0 <= s < nb and 0 <= d < nb]
    dsts = [d for _, d in live]
    assert len(set(dsts)) == len(dsts), "one block is the target of two copies"
    assert not set(dsts) & {s for s, _ in live}, "a copy target is also a copy source"
    k2 = kc.reshape(nb, per_block)
    v2 = vc.reshape(nb, per_block)
    for s, d in live:
        k2[d] = k2[s]
        v2[d] = v2[s]
    return kc, vc
