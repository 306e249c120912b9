"""Pins for the attention oracle, each against something other than the oracle itself.

* a library routine: torch's scaled_dot_product_attention (float64, CPU) on the dense K/V;
* a hand-worked example (tests/golden/attention_hand_example.json);
* closed forms: one token -> its V row exactly; equal V rows -> that row; equal K rows ->
  the mean of V; one dominant score -> that V row;
* invariants the pages imply: any physical placement gives the same result (all 4! placements
  of a 4-block pool); a shared block == private duplicated copies; grouped-query attention ==
  multi-head attention with each kv head repeated; n = 0 -> zeros;
* the layout: the oracle's reshape-based reading == the header's scalar index formula;
* split context: merging partition pieces == the unsplit result, for several partition sizes.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from oracle import layout as L
from tests import helpers as H

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def run_oracle(p, scale=None, **kw):
    scale = 1.0 / math.sqrt(p["hd"]) if scale is None else scale
    return A.decode_attention(p["q"], p["k_cache"], p["v_cache"], p["tables"], p["lengths"],
                              scale=scale, hkv=p["hkv"], hd=p["hd"], bs=p["bs"],
                              dtype=p["dtype"], **kw)


def sdpa_reference(p, scale):
    """torch.nn.functional.scaled_dot_product_attention per sequence on the dense K/V."""
    G = p["hq"] // p["hkv"]
    outs = []
    for i, n in enumerate(p["lengths"]):
        q = torch.from_numpy(H.f64(p["q"][i], p["dtype"]))[None, :, None, :]  # [1,Hq,1,hd]
        if n == 0:
            outs.append(np.zeros((p["hq"], p["hd"])))
            continue
        K = torch.from_numpy(H.f64(p["seq_k"][i], p["dtype"])).permute(1, 0, 2)  # [Hkv,n,hd]
        V = torch.from_numpy(H.f64(p["seq_v"][i], p["dtype"])).permute(1, 0, 2)
        K = K.repeat_interleave(G, dim=0)[None].contiguous()
        V = V.repeat_interleave(G, dim=0)[None].contiguous()
        o = torch.nn.functional.scaled_dot_product_attention(q, K, V, scale=scale)
        outs.append(o[0, :, 0, :].numpy())
    return np.stack(outs)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("hq,hkv", [(2, 2), (8, 2), (7, 1)])
def test_matches_torch_sdpa(dtype, hq, hkv):
    rng = np.random.default_rng(11)
    p = H.random_problem(rng, [1, 5, 16, 17, 40, 100], hq, hkv, 64, dtype)
    scale = 0.37
    np.testing.assert_allclose(run_oracle(p, scale), sdpa_reference(p, scale), rtol=0,
                               atol=1e-12)


def test_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "attention_hand_example.json")))
    hd, bs, nb = g["head_dim"], g["block_size"], g["num_blocks"]
    k = np.zeros(nb * hd * bs, np.float32)
    v = np.zeros(nb * hd * bs, np.float32)
    # sequence 0
    s0 = g["sequences"][0]
    for t, tok in enumerate(s0["tokens"]):
        H.place_tokens(k, v, s0["table"][t // bs], t % bs, np.float32([tok["k"]]),
                       np.float32([tok["v"]]), 1, hd, bs, "f32")
    out0 = A.decode_attention(np.float32([[s0["q"]]]), k, v, np.int32([s0["table"]]),
                              np.int32([3]), scale=g["scale"], hkv=1, hd=hd, bs=bs, dtype="f32")
    np.testing.assert_allclose(out0[0, 0], s0["expected"], rtol=0, atol=1e-12)
    # sequence 1: 18 tokens over blocks [3, 1]
    s1 = g["sequences"][1]
    k[:] = 0
    v[:] = 0
    for t in range(18):
        kk = [1, 0, 0, 0] if t == 17 else [0, 0, 0, 0]
        vv = [0, 1, 0, 0] if t == 17 else [1, 0, 0, 0]
        H.place_tokens(k, v, s1["table"][t // bs], t % bs, np.float32([kk]), np.float32([vv]),
                       1, hd, bs, "f32")
    out1 = A.decode_attention(np.float32([[s1["q"]]]), k, v, np.int32([s1["table"]]),
                              np.int32([18]), scale=g["scale"], hkv=1, hd=hd, bs=bs, dtype="f32")
    np.testing.assert_allclose(out1[0, 0], s1["expected"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_single_token_returns_v_exactly(dtype):
    rng = np.random.default_rng(5)
    p = H.random_problem(rng, [1, 1, 1], 4, 2, 64, dtype)
    out = run_oracle(p)
    for i in range(3):
        want = H.f64(p["seq_v"][i][0], dtype)  # [Hkv, hd]
        np.testing.assert_array_equal(out[i], np.repeat(want, 2, axis=0))


def test_zero_length_gives_zeros():
    rng = np.random.default_rng(6)
    p = H.random_problem(rng, [0, 3, 0], 2, 2, 64, "f32")
    out = run_oracle(p)
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.all(np.isfinite(out[1]))


def test_closed_forms():
    rng = np.random.default_rng(7)
    n, hd = 29, 64
    p = H.random_problem(rng, [n, n, n], 2, 2, hd, "f32", fill="zero")
    c = rng.standard_normal(hd).astype(np.float32)
    # seq 0: all V rows equal c -> out = c
    p["seq_v"][0][:] = c
    # seq 1: all K rows equal -> uniform weights -> mean of V
    p["seq_k"][1][:] = p["seq_k"][1][0]
    # seq 2: token 7 dominates by a score gap of ~1000 -> out = its V row (to 1e-12)
    p["seq_k"][2][:] = 0
    p["seq_k"][2][7] = p["q"][2] * np.float32(1000.0 / np.dot(p["q"][2][0], p["q"][2][0]))
    k, v = H.build_caches(p["seq_k"], p["seq_v"], p["tables"], p["lengths"], p["nb"], 2, hd,
                          16, "f32", fill="zero")
    p["k_cache"], p["v_cache"] = k, v
    out = run_oracle(p, scale=1.0)
    np.testing.assert_allclose(out[0], np.tile(c.astype(np.float64), (2, 1)), atol=1e-12)
    np.testing.assert_allclose(out[1], p["seq_v"][1].astype(np.float64).mean(axis=0),
                               atol=1e-12)
    for h in range(2):
        np.testing.assert_allclose(out[2][h], p["seq_v"][2][7][h].astype(np.float64),
                                   atol=1e-12)


def test_all_placements_give_identical_results():
    """Two sequences of two blocks each on a 4-block pool: all 24 placements."""
    rng = np.random.default_rng(8)
    lens = [20, 32]
    hq = hkv = 2
    hd = 64
    base = H.random_problem(rng, lens, hq, hkv, hd, "f16", nb=4)
    ref = None
    for perm in itertools.permutations(range(4)):
        tables = np.array([[perm[0], perm[1]], [perm[2], perm[3]]], dtype=np.int32)
        k, v = H.build_caches(base["seq_k"], base["seq_v"], tables, lens, 4, hkv, hd, 16, "f16")
        out = A.decode_attention(base["q"], k, v, tables, lens, scale=0.125, hkv=hkv, hd=hd,
                                 bs=16, dtype="f16")
        if ref is None:
            ref = out
        np.testing.assert_array_equal(out, ref)


def test_shared_blocks_equal_duplicated_blocks():
    rng = np.random.default_rng(9)
    hkv, hd, bs = 2, 64, 16
    prefix_k = W.normal_values(rng, (48, hkv, hd), "bf16")
    prefix_v = W.normal_values(rng, (48, hkv, hd), "bf16")
    tails = [5, 16, 23]
    seq_k = [np.concatenate([prefix_k, W.normal_values(rng, (t, hkv, hd), "bf16")]) for t in tails]
    seq_v = [np.concatenate([prefix_v, W.normal_values(rng, (t, hkv, hd), "bf16")]) for t in tails]
    lens = [48 + t for t in tails]
    q = W.normal_values(rng, (3, 4, hd), "bf16")
    # shared: blocks 0,1,2 hold the prefix for everyone
    shared = np.array([[0, 1, 2, 3, -1], [0, 1, 2, 4, -1], [0, 1, 2, 5, 6]], dtype=np.int32)
    # duplicated: private copies of the prefix
    dup = np.array([[0, 1, 2, 3, -1], [7, 8, 9, 4, -1], [10, 11, 12, 5, 6]], dtype=np.int32)
    out = []
    for tables in (shared, dup):
        k, v = H.build_caches(seq_k, seq_v, tables, lens, 13, hkv, hd, bs, "bf16")
        out.append(A.decode_attention(q, k, v, tables, lens, scale=0.125, hkv=hkv, hd=hd, bs=bs,
                                      dtype="bf16"))
    np.testing.assert_array_equal(out[0], out[1])


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(10)
    hq, hkv, hd = 8, 2, 64
    G = hq // hkv
    p = H.random_problem(rng, [3, 17, 33], hq, hkv, hd, "f32")
    gqa = run_oracle(p)
    rep_k = [np.repeat(k, G, axis=1) for k in p["seq_k"]]
    rep_v = [np.repeat(v, G, axis=1) for v in p["seq_v"]]
    k, v = H.build_caches(rep_k, rep_v, p["tables"], p["lengths"], p["nb"], hq, hd, 16, "f32")
    mha = A.decode_attention(p["q"], k, v, p["tables"], p["lengths"], scale=1 / 8, hkv=hq,
                             hd=hd, bs=16, dtype="f32")
    np.testing.assert_array_equal(gqa, mha)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_layout_reading_matches_header_formula(dtype):
    rng = np.random.default_rng(12)
    nb, hkv, hd, bs = 3, 2, 64, 16
    size = nb * hkv * hd * bs
    k = W.normal_values(rng, (size,), dtype)
    v = W.normal_values(rng, (size,), dtype)
    for b in range(nb):
        kt = L.k_tile_tokens(k, b, hkv, hd, bs, dtype)
        vt = L.v_tile_tokens(v, b, hkv, hd, bs, dtype)
        for t in (0, 5, 15):
            for h in range(hkv):
                d = np.arange(hd)
                np.testing.assert_array_equal(kt[t, h], k[H.k_offsets(b, h, t, d, hkv, hd, bs,
                                                                       dtype)])
                np.testing.assert_array_equal(vt[t, h], v[H.v_offsets(b, h, t, d, hkv, hd, bs)])


def test_poisoned_unused_slots_do_not_change_result():
    rng = np.random.default_rng(13)
    p = H.random_problem(rng, [3, 16, 21], 2, 2, 64, "f16", fill="zero")
    ref = run_oracle(p)
    k, v = p["k_cache"].copy(), p["v_cache"].copy()
    L.poison_unused(k, v, p["tables"], p["lengths"], 2, 64, 16, "f16")
    assert np.isnan(k.astype(np.float32)).sum() > 0
    p["k_cache"], p["v_cache"] = k, v
    np.testing.assert_array_equal(run_oracle(p), ref)


@pytest.mark.parametrize("part", [16, 32, 48, 64, 512])
def test_partition_merge_equals_unsplit(part):
    rng = np.random.default_rng(14)
    p = H.random_problem(rng, [1, 16, 40, 100, 129], 4, 2, 64, "bf16")
    ref = run_oracle(p, scale=0.2)
    pieces = A.partition_partials(p["q"], p["k_cache"], p["v_cache"], p["tables"], p["lengths"],
                                  scale=0.2, hkv=2, hd=64, bs=16, dtype="bf16", part_tokens=part)
    for i, (m, l, o) in enumerate(pieces):
        assert m.shape[0] == -(-int(p["lengths"][i]) // part)
        for h in range(4):
            np.testing.assert_allclose(A.merge_partials(m[:, h], l[:, h], o[:, h]), ref[i, h],
                                       rtol=0, atol=1e-12)


def test_arbitrary_cuts_merge_to_unsplit():
    """Any cut of [0, n) into consecutive token ranges (including empty and past-the-end
    ones) recombines to the unsplit result."""
    rng = np.random.default_rng(16)
    p = H.random_problem(rng, [1, 37, 300], 6, 2, 64, "f16")
    ref = run_oracle(p, scale=0.15)
    for i, n in enumerate(p["lengths"]):
        for trial in range(4):
            cuts = sorted(set([0, int(n) + 5] + rng.integers(0, int(n) + 6, size=trial * 3).tolist()))
            pieces = [A.range_partials(p["q"], p["k_cache"], p["v_cache"], p["tables"],
                                       p["lengths"], seq=i, lo=a, hi=b, scale=0.15, hkv=2, hd=64,
                                       bs=16, dtype="f16") for a, b in zip(cuts, cuts[1:])]
            m, l, o = (np.stack(x) for x in zip(*pieces))
            for h in range(6):
                np.testing.assert_allclose(A.merge_partials(m[:, h], l[:, h], o[:, h]), ref[i, h],
                                           rtol=0, atol=1e-12)


def test_single_token_partition_closed_form():
    """Partitions of one token each: m = that token's score, l = 1, o = its V row."""
    rng = np.random.default_rng(15)
    p = H.random_problem(rng, [3], 2, 2, 64, "f32")
    pieces = A.partition_partials(p["q"], p["k_cache"], p["v_cache"], p["tables"], p["lengths"],
                                  scale=0.5, hkv=2, hd=64, bs=16, dtype="f32", part_tokens=1)
    m, l, o = pieces[0]
    assert m.shape == (3, 2)
    for t in range(3):
        for h in range(2):
            s = 0.5 * float(np.dot(p["q"][0][h].astype(np.float64),
                                   p["seq_k"][0][t, h].astype(np.float64)))
            assert m[t, h] == pytest.approx(s, abs=1e-12)
            assert l[t, h] == 1.0
            np.testing.assert_array_equal(o[t, h], p["seq_v"][0][t, h].astype(np.float64))


def test_merge_skips_empty_pieces():
    o = np.arange(8, dtype=np.float64).reshape(2, 4)
    out = A.merge_partials([-np.inf, 0.0], [0.0, 2.0], o)
    np.testing.assert_array_equal(out, o[1] / 2.0)
    assert np.all(A.merge_partials([-np.inf], [0.0], o[:1]) == 0)
