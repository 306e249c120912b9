"""Pins for the oracle's continuous-batching loop ([P1] §四: requests leave when done and join
at any step; blocks are taken on demand and released per request).

Driven by a seeded request stream, the loop must:
* admit requests first-come first-served, never before their arrival, never more than
  max_batch at once, and never so many that a running request could later run out of blocks
  (free blocks >= what the running requests may still take, after every admission);
* decode every request exactly max_new times, each output equal to dense attention over that
  request's own history (its prompt K/V, then its generated K/V, tracked beside the cache);
* keep the paged waste below one block per running request at every step;
* end with every block back in the pool.
"""

import numpy as np
import pytest

import workloads as W
from oracle import batching as OB
from oracle import utilisation as U
from tests import helpers as H


def dense(q, K, V, scale, G):
    out = np.zeros((q.shape[0], K.shape[-1]))
    for h in range(q.shape[0]):
        s = scale * K[:, h // G] @ q[h]
        w = np.exp(s - s.max())
        out[h] = w @ V[:, h // G] / w.sum()
    return out


@pytest.mark.parametrize("nb,max_batch", [(40, 8), (12, 4), (200, 16)])
def test_loop_follows_its_rules(nb, max_batch):
    dtype, hq, hkv, hd, bs, scale = "f32", 4, 2, 64, 16, 0.125
    rng = np.random.default_rng(400 + nb)
    reqs = W.request_stream(rng, 30, prompt=(1, 60), new=(1, 30), rate=0.7)
    assert all(-(-(p + m) // bs) <= nb for _, p, m, _ in reqs)  # each fits an empty pool
    loop = OB.BatchingLoop(nb, bs, hkv, hd, dtype, max_batch=max_batch,
                           free_order=rng.permutation(nb), storage_dtype=np.float32,
                           nan_fill=np.float32(np.nan))
    for r in reqs:
        loop.submit(*r)
    hist, done, order, max_new = {}, {}, [], {r[0]: r[2] for r in reqs}
    arrival = {r[0]: r[3] for r in reqs}
    steps = 0
    while not loop.idle():
        retired, admitted, slots = loop.schedule()
        for rid in retired:
            assert done.get(rid, 0) == max_new[rid]
        for r in admitted:
            assert arrival[r.rid] <= loop.step_no
            order.append(r.rid)
        assert len(loop.running) <= max_batch
        assert loop.alloc.num_free() >= loop._future_blocks()
        if len(slots):
            k = W.normal_values(rng, (len(slots), hkv, hd), dtype)
            v = W.normal_values(rng, (len(slots), hkv, hd), dtype)
            loop.write_prompts(k, v, slots)
            pos = 0
            for r in admitted:
                hist[r.rid] = (k[pos:pos + r.prompt_len], v[pos:pos + r.prompt_len])
                pos += r.prompt_len
        B = len(loop.running)
        q = W.normal_values(rng, (B, hq, hd), dtype)
        kn = W.normal_values(rng, (B, hkv, hd), dtype)
        vn = W.normal_values(rng, (B, hkv, hd), dtype)
        out, _, tables, lens = loop.decode(q, kn, vn, scale)
        if B:
            for i, r in enumerate(loop.running):
                K0, V0 = hist[r.rid]
                hist[r.rid] = (np.concatenate([K0, kn[i:i + 1]]), np.concatenate([V0, vn[i:i + 1]]))
                done[r.rid] = done.get(r.rid, 0) + 1
                K, V = hist[r.rid]
                assert lens[i] == len(K)
                np.testing.assert_allclose(out[i], dense(H.f64(q[i], dtype), H.f64(K, dtype),
                                                         H.f64(V, dtype), scale, hq // hkv),
                                           atol=1e-12)
            u = U.paged_usage(tables, lens, bs)
            assert u["blocks_in_use"] * bs - u["slots_filled"] <= (bs - 1) * B
        steps += 1
        assert steps < 2000
    assert order == sorted(order)  # ids are in arrival order
    assert all(done[r[0]] == r[2] for r in reqs)
    assert loop.alloc.num_free() == nb


def test_loop_with_prefix_cache():
    """Requests share system prompts ([P3] §4.2); admission writes only the tokens after the
    cached ones. With K/V from a model where position p depends on tokens 0..p, every decode
    output equals dense attention over the model's K/V of that request's own tokens, and the
    cache serves a large share of the prompt tokens."""
    import hashlib
    dtype, hq, hkv, hd, bs, scale = "f32", 4, 2, 64, 16, 0.125

    def model_kv(tokens, p):
        h = hashlib.sha256(np.asarray(tokens[:p + 1], np.int64).tobytes()).digest()
        r = np.random.default_rng(int.from_bytes(h[:8], "little"))
        return W.normal_values(r, (hkv, hd), dtype), W.normal_values(r, (hkv, hd), dtype)

    rng = np.random.default_rng(450)
    systems = [list(rng.integers(0, 1000, size=n)) for n in (70, 33)]
    reqs = W.request_stream(rng, 24, prompt=(1, 30), new=(1, 20), rate=0.6)
    nb = 60
    loop = OB.BatchingLoop(nb, bs, hkv, hd, dtype, max_batch=6, free_order=rng.permutation(nb),
                           storage_dtype=np.float32, nan_fill=np.float32(np.nan),
                           prefix_cache=True)
    toks = {}
    for rid, p, m, a in reqs:
        t = [int(x) for x in systems[rid % 2]] + [int(x) for x in rng.integers(0, 1000, size=p)]
        toks[rid] = t
        loop.submit(rid, len(t), m, a, token_ids=t)
    prompt_total, cached_total = 0, 0
    while not loop.idle():
        _, admitted, slots = loop.schedule()
        rows = []
        for r in admitted:
            prompt_total += r.prompt_len
            cached_total += r.cached
            rows += [model_kv(toks[r.rid], p) for p in range(r.cached, r.prompt_len)]
        assert len(rows) == len(slots)
        if rows:
            loop.write_prompts(np.stack([x[0] for x in rows]), np.stack([x[1] for x in rows]),
                               slots)
        B = len(loop.running)
        new_ids = [int(x) for x in rng.integers(0, 1000, size=B)]
        kv = []
        for r, i in zip(loop.running, new_ids):
            toks[r.rid] = toks[r.rid] + [i]
            kv.append(model_kv(toks[r.rid], len(toks[r.rid]) - 1))
        q = W.normal_values(rng, (B, hq, hd), dtype)
        kn = np.stack([x[0] for x in kv]) if kv else np.zeros((0, hkv, hd), np.float32)
        vn = np.stack([x[1] for x in kv]) if kv else np.zeros((0, hkv, hd), np.float32)
        out, _, _, lens = loop.decode(q, kn, vn, scale, new_ids=new_ids)
        for i, r in enumerate(loop.running):
            t = toks[r.rid]
            assert lens[i] == len(t)
            K = np.stack([model_kv(t, p)[0] for p in range(len(t))]).astype(np.float64)
            V = np.stack([model_kv(t, p)[1] for p in range(len(t))]).astype(np.float64)
            np.testing.assert_allclose(out[i], dense(q[i].astype(np.float64), K, V, scale,
                                                     hq // hkv), atol=1e-12)
    assert cached_total > 0.4 * prompt_total
    loop.schedule()
    assert loop.alloc.num_free() == nb
