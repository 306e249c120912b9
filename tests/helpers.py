"""Test-side construction of paged caches, independent of both the oracle and the library.

The caches are built element by element from the documented layout formulas (the library
header states them):

    K element (block b, kv head h, token t, dim d) at ((b*Hkv + h)*(hd/X) + d/X)*bs*X + t*X + d%X
    V element (block b, kv head h, token t, dim d) at ((b*Hkv + h)*hd + d)*bs + t

with X = 16 / element bytes. The oracle reads caches through reshapes/transposes of its own
and the GPU kernels through their own address arithmetic; a test that feeds all of them the
same buffers therefore checks three separate readings of one contract.
"""

import numpy as np

import workloads as W

STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
NAN_BITS = {"f32": np.float32(np.nan), "f16": np.float16(np.nan), "bf16": np.uint16(0x7FC0)}


def k_offsets(b, h, t, d, hkv, hd, bs, dtype):
    x = 16 // ELEM_BYTES[dtype]
    return ((b * hkv + h) * (hd // x) + d // x) * bs * x + t * x + d % x


def v_offsets(b, h, t, d, hkv, hd, bs):
    return ((b * hkv + h) * hd + d) * bs + t


def place_tokens(k_flat, v_flat, block, offset, k_row, v_row, hkv, hd, bs, dtype):
    """Store one token's K/V ([Hkv, hd] storage arrays) at (block, offset), in place."""
    h = np.arange(hkv)[:, None]
    d = np.arange(hd)[None, :]
    k_flat[k_offsets(block, h, offset, d, hkv, hd, bs, dtype)] = k_row
    v_flat[v_offsets(block, h, offset, d, hkv, hd, bs)] = v_row


def build_caches(seq_k, seq_v, tables, lengths, nb, hkv, hd, bs, dtype, fill="nan"):
    """Flat K and V caches holding sequence i's token t at (tables[i][t//bs], t%bs).

    seq_k / seq_v: lists of storage arrays [n_i, Hkv, hd]. A block shared by several
    sequences must receive identical tokens from each of them (checked). Slots that no
    sequence fills hold NaN (fill="nan") or zero (fill="zero").
    """
    size = nb * hkv * hd * bs
    if fill == "nan":
        k_flat = np.full(size, NAN_BITS[dtype], dtype=STORAGE[dtype])
    else:
        k_flat = np.zeros(size, dtype=STORAGE[dtype])
    v_flat = k_flat.copy()
    written = {}
    for i, n in enumerate(lengths):
        for t in range(int(n)):
            blk, off = int(tables[i][t // bs]), t % bs
            key = (blk, off)
            if key in written:
                j, u = written[key]
                assert np.array_equal(seq_k[j][u].view(np.uint8), seq_k[i][t].view(np.uint8)), \
                    "shared slot with different contents"
                continue
            written[key] = (i, t)
            place_tokens(k_flat, v_flat, blk, off, seq_k[i][t], seq_v[i][t], hkv, hd, bs, dtype)
    return k_flat, v_flat


def random_problem(rng, lengths, hq, hkv, hd, dtype, nb=None, bs=16, fill="nan", slack=1.25):
    """Seeded paged-attention input: q, per-sequence logical K/V, random placement, caches.

    Draw order: placement, q, then K and V per sequence.
    """
    lengths = np.asarray(lengths, dtype=np.int32)
    if nb is None:
        nb = W.pool_blocks(lengths, slack=slack, bs=bs)
    order = rng.permutation(nb).astype(np.int32)
    tables = W.place_sequences(lengths, order, bs=bs)
    q = W.normal_values(rng, (len(lengths), hq, hd), dtype)
    seq_k = [W.normal_values(rng, (int(n), hkv, hd), dtype) for n in lengths]
    seq_v = [W.normal_values(rng, (int(n), hkv, hd), dtype) for n in lengths]
    k_flat, v_flat = build_caches(seq_k, seq_v, tables, lengths, nb, hkv, hd, bs, dtype, fill)
    return dict(q=q, seq_k=seq_k, seq_v=seq_v, tables=tables, lengths=lengths, nb=nb,
                k_cache=k_flat, v_cache=v_flat, hq=hq, hkv=hkv, hd=hd, bs=bs, dtype=dtype,
                order=order)


def f64(a, dtype):
    a = np.asarray(a)
    if dtype == "bf16":
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)
