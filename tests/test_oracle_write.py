"""Pins for the cache-write oracle.

* round trip: every written token reads back bit-exactly through the header's scalar index
  formula (independent of the oracle's reshape-based views);
* slots nobody wrote keep their old bits; negative and out-of-pool slots are skipped;
* duplicates in one call are refused;
* write-then-attend ([P1] §三 步驟三: the new token's K/V are written, then attention runs
  over all of the sequence's tokens) equals dense attention over the old tokens plus the new.
"""

import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from oracle import cache_write as CW
from tests import helpers as H


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("hd", [64, 128])
def test_round_trip_and_untouched(dtype, hd):
    rng = np.random.default_rng(21)
    nb, hkv, bs, T = 6, 3, 16, 20
    size = nb * hkv * hd * bs
    kc = W.normal_values(rng, (size,), dtype)
    vc = W.normal_values(rng, (size,), dtype)
    k = W.normal_values(rng, (T, hkv, hd), dtype)
    v = W.normal_values(rng, (T, hkv, hd), dtype)
    slots = rng.choice(nb * bs, size=T, replace=False).astype(np.int32)
    slots[3] = -1
    slots[7] = nb * bs + 5  # outside the pool: skipped
    kc2, vc2 = CW.write_kv(k, v, kc, vc, slots, hkv=hkv, hd=hd, bs=bs, dtype=dtype)
    touched_k = np.zeros(size, bool)
    touched_v = np.zeros(size, bool)
    d = np.arange(hd)[None, :]
    h = np.arange(hkv)[:, None]
    for i, s in enumerate(slots):
        if s < 0 or s >= nb * bs:
            continue
        ko = H.k_offsets(s // bs, h, s % bs, d, hkv, hd, bs, dtype)
        vo = H.v_offsets(s // bs, h, s % bs, d, hkv, hd, bs)
        np.testing.assert_array_equal(kc2[ko].view(np.uint8), k[i].view(np.uint8))
        np.testing.assert_array_equal(vc2[vo].view(np.uint8), v[i].view(np.uint8))
        touched_k[ko] = True
        touched_v[vo] = True
    np.testing.assert_array_equal(kc2[~touched_k].view(np.uint8), kc[~touched_k].view(np.uint8))
    np.testing.assert_array_equal(vc2[~touched_v].view(np.uint8), vc[~touched_v].view(np.uint8))


def test_nan_payload_is_copied_bitwise():
    k = np.full((1, 1, 64), 0x7E01, np.uint16)  # a bf16 NaN with a payload
    v = np.full((1, 1, 64), 0xFFFF, np.uint16)
    kc = np.zeros(2 * 64 * 16, np.uint16)
    vc = np.zeros(2 * 64 * 16, np.uint16)
    kc2, vc2 = CW.write_kv(k, v, kc, vc, np.int32([17]), hkv=1, hd=64, bs=16, dtype="bf16")
    assert (kc2 == 0x7E01).sum() == 64 and (vc2 == 0xFFFF).sum() == 64


def test_duplicate_slots_refused():
    k = np.zeros((2, 1, 64), np.float32)
    with pytest.raises(AssertionError):
        CW.write_kv(k, k, np.zeros(1024, np.float32), np.zeros(1024, np.float32),
                    np.int32([3, 3]), hkv=1, hd=64, bs=16, dtype="f32")


def test_write_then_attend_includes_new_token():
    rng = np.random.default_rng(22)
    hkv, hd, bs, dtype = 2, 64, 16, "f16"
    lens_before = [15, 16, 31]
    p = H.random_problem(rng, lens_before, 4, hkv, hd, dtype, nb=12)
    # slot of each sequence's next token: the next offset in its last block, or a fresh block
    used = sum(-(-n // bs) for n in lens_before)
    fresh = iter(int(b) for b in p["order"][used:])
    tables = p["tables"].copy()
    tables = np.concatenate([tables, np.full((3, 1), -1, np.int32)], axis=1)
    slots = []
    for i, n in enumerate(lens_before):
        if n % bs == 0:
            tables[i, n // bs] = next(fresh)
        slots.append(tables[i, n // bs] * bs + n % bs)
    k_new = W.normal_values(rng, (3, hkv, hd), dtype)
    v_new = W.normal_values(rng, (3, hkv, hd), dtype)
    kc, vc = CW.write_kv(k_new, v_new, p["k_cache"], p["v_cache"], np.int32(slots), hkv=hkv,
                         hd=hd, bs=bs, dtype=dtype)
    lens_after = np.int32(lens_before) + 1
    out = A.decode_attention(p["q"], kc, vc, tables, lens_after, scale=0.125, hkv=hkv, hd=hd,
                             bs=bs, dtype=dtype)
    # dense reference on the concatenated logical K/V
    for i in range(3):
        K = np.concatenate([p["seq_k"][i], k_new[i:i + 1]]).astype(np.float64)
        V = np.concatenate([p["seq_v"][i], v_new[i:i + 1]]).astype(np.float64)
        for h in range(4):
            s = 0.125 * K[:, h // 2] @ p["q"][i, h].astype(np.float64)
            w = np.exp(s - s.max())
            np.testing.assert_allclose(out[i, h], w @ V[:, h // 2] / w.sum(), atol=1e-12)
