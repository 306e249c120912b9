"""Pins for the prefill oracle (causal attention of new prompt tokens over the paged cache).

* the first prompt token (position 0) returns its own V exactly (softmax of one score);
* the last new token of a sequence sees every token: it equals decode attention of that
  sequence (the decode oracle is pinned separately);
* a pure-Python brute force (scalar loops, math.exp) on tiny inputs, to 1e-12;
* chunked prefill: the same prompt attended in two chunks (the first chunk's K/V in the cache
  when the second runs) gives the same outputs as one prefill, since a query only ever sees
  tokens at or before its own position;
* a prompt whose first tokens were cached (a shared prefix) needs queries only for the rest;
* invariance under block placement and sharing of the prefix blocks.
"""

import math

import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from tests import helpers as H


def prompt_problem(rng, lens, hq, hkv, hd, dtype, nb=None):
    p = H.random_problem(rng, lens, hq, hkv, hd, dtype, nb=nb)
    return p


@pytest.mark.parametrize("dtype,hq,hkv", [("f32", 2, 2), ("bf16", 4, 2), ("f16", 8, 2)])
def test_first_token_returns_its_value_and_last_equals_decode(dtype, hq, hkv):
    rng = np.random.default_rng(1100)
    lens = [1, 17, 40, 5]
    p = prompt_problem(rng, lens, hq, hkv, 64, dtype)
    qs = np.cumsum([0] + lens)  # whole prompts
    T = int(qs[-1])
    q = W.normal_values(rng, (T, hq, 64), dtype)
    out = A.prefill_attention(q, p["k_cache"], p["v_cache"], p["tables"], p["lengths"], qs,
                              scale=0.125, hkv=hkv, hd=64, bs=16, dtype=dtype)
    G = hq // hkv
    for i in range(len(lens)):
        first = int(qs[i])
        for h in range(hq):
            np.testing.assert_array_equal(out[first, h], H.f64(p["seq_v"][i][0, h // G], dtype))
        last = int(qs[i + 1]) - 1
        dec = A.decode_attention(q[last:last + 1], p["k_cache"], p["v_cache"],
                                 p["tables"][i:i + 1], p["lengths"][i:i + 1], scale=0.125,
                                 hkv=hkv, hd=64, bs=16, dtype=dtype)
        np.testing.assert_allclose(out[last], dec[0], atol=1e-12)


def test_brute_force_tiny():
    rng = np.random.default_rng(1101)
    lens, hq, hkv, hd = [3, 18], 2, 1, 64
    p = prompt_problem(rng, lens, hq, hkv, hd, "f32")
    qs = [0, 2, 7]  # 2 new tokens of sequence 0, 5 of sequence 1
    q = W.normal_values(rng, (7, hq, hd), "f32")
    out = A.prefill_attention(q, p["k_cache"], p["v_cache"], p["tables"], p["lengths"], qs,
                              scale=0.3, hkv=hkv, hd=hd, bs=16, dtype="f32")
    for i, (a, b) in enumerate(zip(qs, qs[1:])):
        n = lens[i]
        K, V = p["seq_k"][i], p["seq_v"][i]
        for k in range(b - a):
            pos = n - (b - a) + k
            for h in range(hq):
                sc = [0.3 * sum(float(q[a + k, h, d]) * float(K[t, 0, d]) for d in range(hd))
                      for t in range(pos + 1)]
                mx = max(sc)
                w = [math.exp(x - mx) for x in sc]
                want = [sum(w[t] * float(V[t, 0, d]) for t in range(pos + 1)) / sum(w)
                        for d in range(hd)]
                np.testing.assert_allclose(out[a + k, h], want, atol=1e-12)


def test_chunked_prefill_equals_one_prefill():
    rng = np.random.default_rng(1102)
    lens, hq, hkv, hd, dtype = [50, 33], 4, 2, 64, "bf16"
    p = prompt_problem(rng, lens, hq, hkv, hd, dtype)
    T = sum(lens)
    q = W.normal_values(rng, (T, hq, hd), dtype)
    whole = A.prefill_attention(q, p["k_cache"], p["v_cache"], p["tables"], p["lengths"],
                                [0, 50, 83], scale=0.1, hkv=hkv, hd=hd, bs=16, dtype=dtype)
    # chunk 1: the first 20 / 9 tokens (the cache holds them; later slots are not read)
    c1 = A.prefill_attention(np.concatenate([q[:20], q[50:59]]), p["k_cache"], p["v_cache"],
                             p["tables"], np.int32([20, 9]), [0, 20, 29], scale=0.1, hkv=hkv,
                             hd=hd, bs=16, dtype=dtype)
    # chunk 2: the rest, over the whole cached prompt
    c2 = A.prefill_attention(np.concatenate([q[20:50], q[59:83]]), p["k_cache"], p["v_cache"],
                             p["tables"], np.int32(lens), [0, 30, 54], scale=0.1, hkv=hkv,
                             hd=hd, bs=16, dtype=dtype)
    np.testing.assert_allclose(np.concatenate([c1[:20], c2[:30], c1[20:], c2[30:]]), whole,
                               atol=1e-12)


def test_placement_and_shared_prefix_invariance():
    rng = np.random.default_rng(1103)
    hq, hkv, hd, dtype = 4, 4, 64, "f16"
    lens = [37, 37]
    p = prompt_problem(rng, lens, hq, hkv, hd, dtype)
    # sequence 1 holds the same tokens as sequence 0: point its first two blocks at sequence 0's
    seq_k = [p["seq_k"][0], p["seq_k"][0].copy()]
    seq_v = [p["seq_v"][0], p["seq_v"][0].copy()]
    nb = p["nb"]
    kc, vc = H.build_caches(seq_k, seq_v, p["tables"], lens, nb, hkv, hd, 16, dtype)
    shared = p["tables"].copy()
    shared[1, :2] = shared[0, :2]
    q = W.normal_values(rng, (10, hq, hd), dtype)
    qs = [0, 5, 10]  # the last 5 tokens of each
    a = A.prefill_attention(q, kc, vc, p["tables"], np.int32(lens), qs, scale=0.1, hkv=hkv,
                            hd=hd, bs=16, dtype=dtype)
    b = A.prefill_attention(q, kc, vc, shared, np.int32(lens), qs, scale=0.1, hkv=hkv, hd=hd,
                            bs=16, dtype=dtype)
    np.testing.assert_array_equal(a, b)
    # the same queries on sequence 1 (same tokens) give the same outputs
    c = A.prefill_attention(q[:5], kc, vc, p["tables"][1:], np.int32([37]), [0, 5], scale=0.1,
                            hkv=hkv, hd=hd, bs=16, dtype=dtype)
    np.testing.assert_array_equal(c, a[:5])
