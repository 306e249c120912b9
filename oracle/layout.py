"""Paged KV-cache layout and dtype handling for the oracle (float64, NumPy).

Test infrastructure only (see the package docstring).

Storage arrays are NumPy arrays holding the exact bits of the device buffers:
``f32`` -> float32, ``f16`` -> float16, ``bf16`` -> uint16 (the raw bfloat16 bits; NumPy has
no bfloat16). ``to_f64`` widens them exactly.

Cache layout (the library's documented contract; the pages fix only the 16-token block,
[P1] §二 "具體運作方式" and [P3] §3.2). With E element bytes and X = 16 // E:

* K cache: shape [NB, Hkv, hd // X, bs, X]; token t, dim d of the tile (b, h) is
  ``k[b, h, d // X, t, d % X]``.
* V cache: shape [NB, Hkv, hd, bs]; token t, dim d of the tile (b, h) is ``v[b, h, d, t]``.
"""

import numpy as np

DTYPES = ("f32", "f16", "bf16")
_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
_ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def storage_dtype(dtype):
    return _STORAGE[dtype]


def elem_bytes(dtype):
    return _ELEM_BYTES[dtype]


def chunk_elems(dtype):
    """X: elements in one 16-byte chunk of the K layout."""
    return 16 // _ELEM_BYTES[dtype]


def to_f64(a, dtype):
    """Exact widening of a storage array to float64."""
    a = np.asarray(a)
    if dtype == "bf16":
        bits = a.astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def k_cache_shape(nb, hkv, hd, bs, dtype):
    x = chunk_elems(dtype)
    assert hd % x == 0
    return (nb, hkv, hd // x, bs, x)


def v_cache_shape(nb, hkv, hd, bs, dtype):
    return (nb, hkv, hd, bs)


def k_tile_tokens(k_cache, block, hkv, hd, bs, dtype):
    """Tile (block, all kv heads) of the K cache as [bs, Hkv, hd] storage values."""
    x = chunk_elems(dtype)
    tile = np.asarray(k_cache).reshape(-1, hkv, hd // x, bs, x)[block]  # [Hkv, hd/X, bs, X]
    return tile.transpose(2, 0, 1, 3).reshape(bs, hkv, hd)


def v_tile_tokens(v_cache, block, hkv, hd, bs, dtype):
    """Tile (block, all kv heads) of the V cache as [bs, Hkv, hd] storage values."""
    tile = np.asarray(v_cache).reshape(-1, hkv, hd, bs)[block]  # [Hkv, hd, bs]
    return tile.transpose(2, 0, 1)


def token_slot_views(k_cache, v_cache, hkv, hd, bs, dtype):
    """Views of both caches indexed as [NB, bs, Hkv, hd] (writable views, same memory)."""
    x = chunk_elems(dtype)
    k5 = np.asarray(k_cache).reshape(-1, hkv, hd // x, bs, x)
    v4 = np.asarray(v_cache).reshape(-1, hkv, hd, bs)
    kv = k5.transpose(0, 3, 1, 2, 4)  # [NB, bs, Hkv, hd/X, X]
    vv = v4.transpose(0, 3, 1, 2)  # [NB, bs, Hkv, hd]
    return kv, vv


def poison_unused(k_cache, v_cache, block_tables, context_lens, hkv, hd, bs, dtype):
    """Fill every cache slot that holds no valid token of any sequence with NaN (in place).

    A slot is valid when some sequence i has it at logical position t < n_i (reading the
    table entry t // bs). Free blocks and the unfilled tail of a last block become NaN, so a
    kernel that reads past a sequence's length, or picks the wrong block, cannot go unseen.
    """
    nb = np.asarray(k_cache).size // (hkv * hd * bs)
    used = np.zeros((nb, bs), dtype=bool)
    for row, n in zip(np.asarray(block_tables), np.asarray(context_lens)):
        for t in range(int(n)):
            used[int(row[t // bs]), t % bs] = True
    kv, vv = token_slot_views(k_cache, v_cache, hkv, hd, bs, dtype)
    nan = _nan_value(dtype)
    kv[~used] = nan
    vv[~used] = nan


def _nan_value(dtype):
    if dtype == "bf16":
        return np.uint16(0x7FC0)
    return _STORAGE[dtype](np.nan)
