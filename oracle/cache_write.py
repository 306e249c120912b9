"""Cache write (scatter of new tokens' K/V into their slots), bitwise.

Test infrastructure only (see the package docstring).

[P1] §三 步驟二 and 步驟三: the K/V of each new token are written into the current block of
its sequence (a fresh block having been taken when the current one was full). The slot that
says where, ``slot = physical_block * bs + offset``, comes from the allocator; this function
only performs the write, for the T tokens of one call:

    for every i with 0 <= slot[i] < NB * bs:
        K cache (block slot[i] // bs, head h, token slot[i] % bs, :) = k[i, h, :]   (all h)
        V cache (same)                                                  = v[i, h, :]

Negative slots are padding and are skipped. Two tokens with one slot in one call have no
defined result, so the oracle refuses them.
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
